/*
 * Internal declarations shared by the host entry points (tq_host.cpp) and the
 * gfx950 kernels (tq_encode.hip, tq_decode.hip).
 */
#ifndef TQ_INTERNAL_H
#define TQ_INTERNAL_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"

/* Encoder bucket table.  The rotated, normalised coordinate y in [-1, 1]
 * maps to u = (y + 1) * nb_half + 1/2 + enc_shift and bucket r = u rounded to
 * an integer, r in 0 .. 2*nb_half + 1 (enc_shift < 0.45, so a few ulps beyond
 * |y| = 1 still round into that range).  Bucket r holds the thresholds whose
 * u lies in [r - 1/2, r + 1/2), at most one, and base = the number of
 * thresholds below r - 1/2.  The code is base + (y nb_half > t nb_half), the
 * comparison decided exactly as the sign of one fused multiply-add
 * h * scale - t nb_half (h * scale = y nb_half), with neg_t = fp32(-t nb_half)
 * (-inf for buckets without a threshold).  enc_shift keeps every threshold's
 * u at least 1/64 of a bucket away from the bucket edges, so that the fp32
 * rounding of u never puts a coordinate in a bucket on the far side of a
 * threshold it lies close to. */
struct alignas(8) tq_enc_entry {
  float neg_t;
  uint32_t base;
};

/* Rows of the encoder table a kernel keeps for (d, bits): 2 * nb_half + 2 for
 * the nb_half the codebook build picks (the smallest power of two whose
 * buckets are narrower than the closest pair of thresholds with a 2% margin:
 * 16 / 32 / 32 buckets per unit of y for 2 / 3 / 4 bits at d = 64,
 * 16 / 32 / 64 at d = 128, 32 / 64 / 64 at d = 256).  The codebook build
 * checks its table against this bound. */
__host__ __device__ constexpr int tq_enc_rows_max(int d, int bits) {
  return 2 * (bits == 2 ? (d == 256 ? 32 : 16)
                        : bits == 3 ? (d == 256 ? 64 : 32) : (d == 64 ? 32 : 64)) +
         2;
}

struct tq_codebook_s {
  int d, bits;
  int nb_half;           /* buckets per unit of y */
  int enc_entries;       /* 2 * nb_half + 2 */
  float enc_shift;       /* bucket grid offset in [0, 0.45) */
  float sigma;           /* decoder lookup-table scale (levels stored as fp16(c * sigma)) */
  double centroids64[16];
  double bounds64[15];
  float centroids[16];
  float bounds[15];
  int device;
  void* dev_mem;         /* one device allocation: encoder table, then decoder table */
  const tq_enc_entry* enc_table;
  const uint32_t* dec_lut; /* one word (two fp16 levels) per pair of codes: 2^(2*bits) words */
  const uint32_t* dec_lut_lo; /* same shape: two fp16 remainders (level - fp16 level) * 2^11 */
  const uint32_t* dec_quad;   /* bits 2: four fp16 levels (two words) per byte of codes */
  /* one word per code: fp16(level * sigma * 2^pre_exp) in the low half, the
   * fp16 of its remainder (unscaled) in the high half; pre_exp puts the
   * largest level in [16, 32), so every remainder is far above fp16's
   * absolute rounding step */
  const uint32_t* pre_klut;
  int pre_exp;
};

/* Host-side Lloyd-Max (levels / thresholds in fp64, N(0, 1/d)). */
int tq_lloyd_max_host(int d, int bits, double* c, double* t);

/* Launchers (argument checks are done by the callers). */
tq_status tq_launch_encode_rows(const tq_codebook_s* cb, const uint16_t* x, int64_t n,
                                int64_t x_stride, const uint8_t* sign_bits, uint8_t* codes,
                                uint16_t* norms, hipStream_t stream);

tq_status tq_launch_append(const tq_kv_cache* c, const tq_codebook_s* cbk,
                           const tq_codebook_s* cbv, const uint8_t* sign_bits,
                           const uint16_t* k_new, const uint16_t* v_new, int t_new,
                           const int32_t* pos, int n_layers, hipStream_t stream);

tq_status tq_launch_prefill(const tq_kv_cache* c, const tq_codebook_s* cbk,
                            const tq_codebook_s* cbv, const uint8_t* sign_bits,
                            const uint16_t* q, int q_heads, int t_new, const int32_t* pos,
                            int n_layers, float* out, hipStream_t stream);

tq_status tq_launch_qjl_encode(const tq_codebook_s* cb, const uint16_t* x, int64_t n,
                               int64_t stride, const uint8_t* sign_bits, const uint16_t* S,
                               const uint8_t* codes, uint8_t* signs, uint16_t* gamma,
                               hipStream_t stream);
tq_status tq_launch_qjl_scores(const tq_codebook_s* cb, const uint16_t* q, int G,
                               const uint8_t* sign_bits, const uint16_t* S, const uint8_t* codes,
                               const uint16_t* norms, const uint8_t* signs,
                               const uint16_t* gamma, int64_t T, float* out, hipStream_t stream);

/* Split count and workspace layout of one decode call. */
struct tq_decode_plan {
  int splits;          /* token splits per (layer, seq, kv head) */
  int tiles_per_split; /* 32-token tiles per split */
  int upb;             /* (layer, seq, kv head) units per block; > 1 only with one split */
  size_t ctr_bytes;    /* per-unit arrival counters, 256-byte padded */
  size_t ws_bytes;     /* counters + (m, l, acc[d]) records; 0 when splits == 1 */
};
tq_decode_plan tq_plan_decode(const tq_kv_cache* c, int q_heads, int max_len, int n_layers);

tq_status tq_launch_decode(const tq_kv_cache* c, const tq_codebook_s* cbk,
                           const tq_codebook_s* cbv, const uint8_t* sign_bits,
                           const uint16_t* q, int q_heads, const int32_t* seq_lens,
                           int max_len, int n_layers, float* out, void* ws,
                           const tq_decode_plan& plan, float sparse_eps, uint32_t* skip_counts,
                           uint32_t* skip_tiles, hipStream_t stream);

/* Bytes of the library-held decode workspace of tq_decode_attn_noalloc (one
 * array per GPU, held until the process ends). */
#define TQ_NOALLOC_SCRATCH_BYTES (16u << 20)

/* This device's library-held workspace (tq_noalloc.hip): its address, looked
 * up (and the array cleared on `stream`) on the first call on a device. */
tq_status tq_noalloc_scratch(void** out, hipStream_t stream);

/* Words per (layer, sequence, KV head) of a Sparse V skip bitmap: one bit per
 * 32-token tile of a context of up to max_len tokens. */
inline int tq_skip_words(int max_len) { return (max_len + 1023) / 1024; }

#endif
