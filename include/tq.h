/*
 * tq.h -- TurboQuant-style KV-cache compression and compressed-cache decode
 * attention for AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes.
 *
 * The method (sources are the pages this library is built from):
 *   - Each per-head key or value vector x (fp16, head dim d) is split into its
 *     norm, stored in FP16, and the unit vector x / ||x||
 *     ("We Built a Python Library That Cuts LLM Memory Usage by 80%", section
 *     "The Paper").
 *   - The unit vector is rotated by the randomized Hadamard transform
 *     y = (1/sqrt d) H D x (AdapTQ page, "How it works (HAR + VQ)", step 1),
 *     computed as a fast Walsh-Hadamard transform.  D is a per-layer diagonal
 *     of signs, shared by keys, values and queries of that layer.
 *   - Each rotated coordinate, distributed about N(0, 1/d), is quantized
 *     independently with the Lloyd-Max codebook for that Gaussian at 2, 3 or 4
 *     bits ("We Built ...", "The Paper"; AdapTQ page, step 2), and the codes
 *     are bit-packed ("We Built ...", "What's Next": bit-packing).
 *   - Decode attention rotates the query once and scores it against the codes
 *     through codebook lookups without dequantizing back to the original
 *     domain (AdapTQ page, step 3); values are accumulated in the rotated
 *     domain and rotated back once, the transform being reversible
 *     ("TurboQuant: 4-bit KV Cache Quantization ... FWHT Preprocessing",
 *     section "FWHT Preprocessing Layer").
 *
 * Conventions for every call:
 *   - Device pointers are allocated and owned by the caller; the library never
 *     allocates or frees them.  Host pointers are marked "host".
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls that launch kernels are asynchronous on that stream.
 *   - Every argument the host can check is checked before any launch; on an
 *     error nothing is written and nothing is launched.  Launch failures
 *     return TQ_ERR_DEVICE.
 *   - Supported: head_dim in {64, 128, 256}; bits in {2, 3, 4}.
 *   - fp16 values travel as their 16-bit patterns (uint16_t).
 *
 * Packed formats:
 *   Row layout (tq_encode output, the key cache):
 *     one vector = d*bits/8 bytes, a little-endian bit string; coordinate i's
 *     code occupies bits [bits*i, bits*i + bits); bit j is bit (j % 8) of byte
 *     j / 8.  Code k means the k-th smallest codebook level.
 *   Value-tile layout (the value cache):
 *     the codes of 32 consecutive tokens form a tile of 32*d*bits/8 bytes, cut
 *     into 64 segments of d*bits/16 bytes.  Segment l = 16*q + r (q in 0..3,
 *     r in 0..15) is a little-endian bit string holding, for m in 0..d/16-1 and
 *     u in 0..7, at bit offset (8*m + u)*bits, the code of coordinate
 *     r*(d/16) + m of tile token tok(q,u) = 8q + u.  The order matches the
 *     matrix-core operand layout of the decode kernel, so one load per lane
 *     feeds its value products, and each half tile (16 tokens) is a
 *     contiguous half of the bytes.
 *   Norms: fp16 (RNE of the exact Euclidean norm), one per vector.
 *   Sign bits: d bits per layer, LSB-first in d/8 bytes; bit i set means
 *     D_ii = -1.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_ARG = 1,         /* null pointer, bad size, misaligned buffer */
  TQ_ERR_UNSUPPORTED = 2, /* head_dim / bits / group size outside the supported set */
  TQ_ERR_CAPACITY = 3,    /* an append would write past the cache capacity */
  TQ_ERR_WORKSPACE = 4,   /* decode workspace smaller than required */
  TQ_ERR_DEVICE = 5       /* a HIP call or kernel launch failed */
} tq_status;

/* Human-readable name of a status code (static string). */
const char* tq_status_str(tq_status s);

/* ------------------------------------------------------------- codebooks -- */

/* Lloyd-Max codebook for N(0, 1/d) ("We Built ...", "The Paper"; AdapTQ page,
 * step 2: Max-Lloyd codebooks).  Host only, no device work.
 * centroids (host, 2^bits floats): the levels in increasing order;
 * bounds (host, 2^bits - 1 floats): the decision thresholds (midpoints).
 * Returns TQ_ERR_UNSUPPORTED for d or bits outside the supported set. */
tq_status tq_codebook_compute(int head_dim, int bits, float* centroids, float* bounds);

typedef struct tq_codebook_s* tq_codebook;

/* Build the codebook for (head_dim, bits) and upload its device tables (the
 * encoder's bucket table and the decoder's lookup table) to the current HIP
 * device.  Synchronous.  *out receives an immutable handle, usable from any
 * thread and stream on that device; release it with tq_codebook_free. */
tq_status tq_codebook_init(int head_dim, int bits, tq_codebook* out);

/* Host copy of the levels / thresholds the device tables were built from
 * (same as tq_codebook_compute), and the handle's parameters. */
tq_status tq_codebook_read(tq_codebook cb, float* centroids, float* bounds);
int tq_codebook_head_dim(tq_codebook cb);
int tq_codebook_bits(tq_codebook cb);

/* Frees the handle and its device tables (synchronises the device). */
void tq_codebook_free(tq_codebook cb);

/* ---------------------------------------------------------------- encode -- */

/* Encode n vectors ("We Built ...", "The Paper": norm split, rotation,
 * per-coordinate codebook quantization; AdapTQ page, steps 1-2).
 * x:         device, fp16 [n][x_stride] (the first d values of each row are
 *            the vector), 16-byte aligned, x_stride % 8 == 0, x_stride >= d.
 * sign_bits: device, d/8 bytes (this layer's D), 4-byte aligned.
 * codes:     device, [n][d*bits/8] row layout, 8-byte aligned.
 * norms:     device, fp16 [n], 2-byte aligned.
 * The codebook fixes d and bits.  n == 0 is a no-op. */
tq_status tq_encode(tq_codebook cb, const uint16_t* x, int64_t n, int64_t x_stride,
                    const uint8_t* sign_bits, uint8_t* codes, uint16_t* norms,
                    void* stream);

/* ------------------------------------------------------------- the cache -- */

/* One compressed KV cache layer; layer i of a multi-layer call lives at the
 * base pointers plus i * layer_stride (bytes) of each array.
 *
 * Contiguous storage (block_table == NULL):
 *   k_codes: [batch][kv_heads][capacity][d*bits_k/8]     row layout
 *   v_codes: [batch][kv_heads][capacity/32][32*d*bits_v/8] value-tile layout
 *   k_norms, v_norms: fp16 [batch][kv_heads][capacity]
 * capacity % 32 == 0, and capacity * d * max(bits_k, bits_v) / 8 < 2^31 (one
 * (sequence, head) stream of codes is addressed with 32-bit offsets; larger
 * caches return TQ_ERR_UNSUPPORTED).
 *
 * Paged storage (block_table != NULL): each layer's arrays are a pool of
 * num_pages pages of page_tokens tokens, shared by all sequences:
 *   k_codes: [num_pages][kv_heads][page_tokens][d*bits_k/8]
 *   v_codes: [num_pages][kv_heads][page_tokens/32][32*d*bits_v/8]
 *   k_norms, v_norms: fp16 [num_pages][kv_heads][page_tokens]
 * block_table (device int32 [batch][max_pages], 4-byte aligned, the same for
 * every layer) maps page p of sequence b (its tokens p*page_tokens ..
 * (p+1)*page_tokens - 1) to a pool page.  page_tokens is a power of two
 * >= 32, capacity == max_pages * page_tokens (tokens per sequence), and each
 * pool array of a layer is < 2^31 bytes (else TQ_ERR_UNSUPPORTED).  Entries
 * outside [0, num_pages) make appends skip those rows and decode read page 0
 * or num_pages - 1 instead (no access outside the pool).
 *
 * Both: code arrays 16-byte aligned, norm arrays 8-byte aligned, layer
 * strides multiples of 16.  Rows at or past a sequence's length are never
 * read by decode.  Paging fields are ignored (and may be zero) when
 * block_table is NULL. */
typedef struct {
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint16_t* k_norms;
  uint16_t* v_norms;
  int batch, kv_heads, head_dim, bits_k, bits_v, capacity;
  int64_t layer_stride_k_codes, layer_stride_v_codes;
  int64_t layer_stride_k_norms, layer_stride_v_norms;
  const int32_t* block_table; /* NULL: contiguous storage */
  int page_tokens, max_pages, num_pages;
} tq_kv_cache;

/* Bytes of each array for one layer (host helper, no device work): the
 * contiguous arrays, or the page pools. */
tq_status tq_cache_layer_bytes(const tq_kv_cache* c, int64_t* k_codes, int64_t* v_codes,
                               int64_t* k_norms, int64_t* v_norms);

/* Append t_new tokens per sequence to n_layers layers ("We Built ...",
 * "Under the Hood": the cache compresses on each update).
 * k_new, v_new: device fp16 [n_layers][batch][kv_heads][t_new][d], 16-byte
 *               aligned, contiguous.
 * sign_bits:    device [n_layers][d/8], 4-byte aligned.
 * pos:          device int32 [batch]: the first row written for sequence b;
 *               rows pos[b] .. pos[b] + t_new - 1 of every layer and head are
 *               written, nothing else changes (partially covered value tiles
 *               keep their other tokens' bits).
 * host_max_pos: max_b pos[b] if the caller knows it (then host_max_pos + t_new
 *               <= capacity is checked, else TQ_ERR_CAPACITY), or -1 (then rows
 *               at or past capacity are skipped on the device).
 * cbk, cbv:     codebooks with (head_dim, bits_k) and (head_dim, bits_v).
 * Writing a token with tq_append equals encoding it alone with tq_encode, bit
 * for bit (value codes rearranged into the tile layout). */
tq_status tq_append(const tq_kv_cache* c, tq_codebook cbk, tq_codebook cbv,
                    const uint8_t* sign_bits, const uint16_t* k_new, const uint16_t* v_new,
                    int t_new, const int32_t* pos, int32_t host_max_pos, int n_layers,
                    void* stream);

/* ---------------------------------------------------------------- decode -- */

/* Workspace (device bytes, 256-byte aligned) tq_decode_attn needs for these
 * shapes; 0 means none.  Host helper.  The workspace must be zero-filled
 * before its first use; every call leaves it ready for the next (its arrival
 * counters return to zero).  Calls that share a workspace must not overlap. */
size_t tq_decode_workspace_bytes(const tq_kv_cache* c, int q_heads, int max_len,
                                 int n_layers);

/* One decode step of attention over the compressed cache for n_layers layers
 * ("We Built ...", "Test Suite": softmax(Q K^T / sqrt d) V; AdapTQ page,
 * step 3: rotated query scored against the packed codes through lookup
 * tables).  Query head h reads KV head h / (q_heads / kv_heads).
 * q:        device fp16 [n_layers][batch][q_heads][d], 16-byte aligned.
 * seq_lens: device int32 [batch]: tokens 0 .. len-1 are attended; values are
 *           clamped to [0, max_len]; len 0 gives a zero output.
 * max_len:  host upper bound on seq_lens, <= capacity (sizes the grid).
 * out:      device fp32 [n_layers][batch][q_heads][d], in the original domain.
 * ws:       device workspace of at least tq_decode_workspace_bytes(...) bytes.
 * Supported group sizes q_heads / kv_heads: 1 .. 8. */
tq_status tq_decode_attn(const tq_kv_cache* c, tq_codebook cbk, tq_codebook cbv,
                         const uint8_t* sign_bits, const uint16_t* q, int q_heads,
                         const int32_t* seq_lens, int max_len, int n_layers, float* out,
                         void* ws, size_t ws_bytes, void* stream);

/* tq_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation and kernels, with the split workspace held by the
 * library, one array of 16 MiB per GPU that stays until the process ends (its
 * address is looked up, and the array cleared, on the first call on a
 * device).  Allocates nothing.  Calls whose workspace
 * (tq_decode_workspace_bytes) exceeds 16 MiB return TQ_ERR_WORKSPACE before
 * anything is launched.  Every call on a GPU shares that GPU's array; calls
 * that overlap on one GPU (other streams, other threads) race and must not
 * be issued.  Arguments as tq_decode_attn, without ws and ws_bytes. */
tq_status tq_decode_attn_noalloc(const tq_kv_cache* c, tq_codebook cbk, tq_codebook cbv,
                                 const uint8_t* sign_bits, const uint16_t* q, int q_heads,
                                 const int32_t* seq_lens, int max_len, int n_layers, float* out,
                                 void* stream);

/* Prefill (extend) attention over the compressed cache: t_new query tokens
 * per sequence, already written to the cache (e.g. by tq_append), each
 * attending causally to its sequence's cached tokens ("We Built ...", "Test
 * Suite": softmax(Q K^T / sqrt d) V; AdapTQ page, step 3, with many queries;
 * the prefill the TurboQuant+ page times).  Query i of sequence b sits at
 * position pos[b] + i and attends to cache rows 0 .. pos[b] + i, the result
 * equalling tq_decode_attn with that query and length pos[b] + i + 1.
 * q:    device fp16 [n_layers][batch][q_heads][t_new][d], 16-byte aligned.
 * pos:  device int32 [batch], 4-byte aligned; negative values count as 0,
 *       rows at or past capacity are never read.
 * out:  device fp32 [n_layers][batch][q_heads][t_new][d], 16-byte aligned,
 *       in the original domain.
 * Query head h reads KV head h / (q_heads / kv_heads); group sizes 1 .. 8.
 * Contiguous or paged cache.  t_new == 0 is a no-op.  No workspace. */
tq_status tq_prefill_attn(const tq_kv_cache* c, tq_codebook cbk, tq_codebook cbv,
                          const uint8_t* sign_bits, const uint16_t* q, int q_heads, int t_new,
                          const int32_t* pos, int n_layers, float* out, void* stream);

/* ------------------------------------------------------------------ QJL -- */

/* The method's second stage, the 1-bit residual sketch of keys ("We Built
 * ...", "Why not both stages?": a one-bit-per-coordinate correction of the
 * residual that makes inner-product estimates unbiased; that page skips it in
 * attention).  For each key x with
 * stage-1 codes (from tq_encode, row layout) the residual in the rotated unit
 * domain is r = R x / ||x|| - c[codes]; the sketch is gamma = fp16(||r||)
 * and d sign bits of S r, bit i set iff (S r)_i >= 0 (LSB first, d/8 bytes).
 * x, x_stride, sign_bits: as tq_encode (x 16-byte aligned, stride % 8 == 0).
 * S:     device fp16 [d][d] row-major, 16-byte aligned: the caller's draw of
 *        i.i.d. N(0,1) entries (fixed per layer, like the sign bits).
 * codes: device, the keys' tq_encode rows [n][d*bits/8], 8-byte aligned
 *        (as tq_encode requires).
 * signs: device [n][d/8], 4-byte aligned (16-byte alignment lets a key's
 *        sign row go out in vector stores).  gamma: device fp16 [n].
 * Misaligned pointers or a bad stride: TQ_ERR_ARG before any device work.
 * The codebook gives d and bits.  n == 0 is a no-op. */
tq_status tq_qjl_encode(tq_codebook cb, const uint16_t* x, int64_t n, int64_t x_stride,
                        const uint8_t* sign_bits, const uint16_t* S, const uint8_t* codes,
                        uint8_t* signs, uint16_t* gamma, void* stream);

/* Estimates of <q_g, x_t> for n_q (1..8) queries q (device fp16 [n_q][d],
 * original domain) over n_keys sketched keys:
 *   n16_t * ( <R q, c[codes_t]> + sqrt(pi/2) / d * gamma_t * <S R q, z_t> ),
 * z_t = +-1 from the sign bits; unbiased for <q, x_t> n16_t / ||x_t|| over
 * the draw of S.  codes [n_keys][d*bits/8] (8-byte aligned), norms fp16
 * [n_keys] (tq_encode), signs (4-byte aligned), gamma as tq_qjl_encode; out:
 * device fp32 [n_q][n_keys]. */
tq_status tq_qjl_scores(tq_codebook cb, const uint16_t* q, int n_q, const uint8_t* sign_bits,
                        const uint16_t* S, const uint8_t* codes, const uint16_t* norms,
                        const uint8_t* signs, const uint16_t* gamma, int64_t n_keys, float* out,
                        void* stream);

/* tq_decode_attn with the Sparse V gate ("TurboQuant+: Compresion de Cache KV
 * 6.4x para LLMs", section "Sparse V": the value work of positions with
 * negligible attention weight is skipped; the page gives no threshold).
 * Per 32-token tile of a (layer, sequence, KV head): the tile's value codes
 * are neither read nor accumulated when, for every query head of the group
 * and every token of the tile, the weight exp(s - m) is below eps, where m
 * is a running maximum of that head's scores (never above the final one).
 * So every skipped token has final weight exp(s - max s) < eps, and every
 * token at or above eps is accumulated; which tokens below eps are skipped
 * depends on the order tiles are visited in.  The softmax denominator keeps
 * every token.  The output therefore differs from tq_decode_attn's by at most
 * sum over tokens with weight < eps of p |v| / l per coordinate.  A
 * sequence's ragged last tile is never skipped.
 * eps:         0 gives tq_decode_attn exactly; > 0 and finite (above 1 every
 *              full tile is skipped); NaN, negative or infinite: TQ_ERR_ARG.
 * skip_counts: device uint32 [n_layers][batch][kv_heads], 4-byte aligned, or
 *              NULL; the number of tiles skipped for each (layer, sequence,
 *              KV head) is ADDED to it (the caller zeroes it).
 * skip_tiles:  device uint32 [n_layers][batch][kv_heads][(max_len + 1023) /
 *              1024], 4-byte aligned, or NULL; when tile t (tokens 32 t ..
 *              32 t + 31) of a unit is skipped, bit t % 32 of that unit's word
 *              t / 32 is OR-ed in (the caller zeroes it), so the exact set of
 *              left-out positions is known.
 * Other arguments as tq_decode_attn (same workspace). */
tq_status tq_decode_attn_sparse(const tq_kv_cache* c, tq_codebook cbk, tq_codebook cbv,
                                const uint8_t* sign_bits, const uint16_t* q, int q_heads,
                                const int32_t* seq_lens, int max_len, int n_layers, float eps,
                                uint32_t* skip_counts, uint32_t* skip_tiles, float* out, void* ws,
                                size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
