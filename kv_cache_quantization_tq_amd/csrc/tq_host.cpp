/*
 * Host side of the C ABI: status strings, codebook construction and upload,
 * argument validation, dispatch to the gfx950 launchers.
 */
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "tq.h"
#include "tq_internal.h"

extern "C" const char* tq_status_str(tq_status s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_ARG: return "TQ_ERR_ARG";
    case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
    case TQ_ERR_CAPACITY: return "TQ_ERR_CAPACITY";
    case TQ_ERR_WORKSPACE: return "TQ_ERR_WORKSPACE";
    case TQ_ERR_DEVICE: return "TQ_ERR_DEVICE";
  }
  return "TQ_ERR_UNKNOWN";
}

static bool supported_dim(int d) { return d == 64 || d == 128 || d == 256; }
static bool supported_bits(int b) { return b >= 2 && b <= 4; }

/* ------------------------------------------------------------ Lloyd-Max -- */

/* P(Z > x) for Z ~ N(0,1), accurate in the tails. */
static double upper_tail(double x) { return 0.5 * erfc(x * 0.70710678118654752440); }
static double gauss_pdf(double x) { return 0.39894228040143267794 * exp(-0.5 * x * x); }

/* Probability of the cell (a, b), written so that no tail is computed as a
 * difference of numbers near 1. */
static double cell_mass(double a, double b) {
  if (a >= 0.0) return upper_tail(a) - upper_tail(b);
  if (b <= 0.0) return upper_tail(-b) - upper_tail(-a);
  return 1.0 - upper_tail(-a) - upper_tail(b);
}

/* Lloyd-Max quantizer of N(0,1) by the fixed-point iteration of the two
 * optimality conditions, with the conditional means in closed form:
 * E[Z | a < Z < b] = (pdf(a) - pdf(b)) / P(a < Z < b).  Levels start uniform
 * on [-3, 3]; the set is made exactly antisymmetric at the end; levels and
 * thresholds are then scaled by 1/sqrt(d) for the N(0, 1/d) coordinates. */
int tq_lloyd_max_host(int d, int bits, double* c, double* t) {
  const int L = 1 << bits;
  for (int k = 0; k < L; ++k) c[k] = -3.0 + 6.0 * (k + 0.5) / L;
  int it = 0;
  for (; it < 1000000; ++it) {
    for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
    double move = 0.0;
    for (int k = 0; k < L; ++k) {
      double a = k == 0 ? -INFINITY : t[k - 1];
      double b = k == L - 1 ? INFINITY : t[k];
      double pa = k == 0 ? 0.0 : gauss_pdf(a), pb = k == L - 1 ? 0.0 : gauss_pdf(b);
      double nc = (pa - pb) / cell_mass(a, b);
      move = fmax(move, fabs(nc - c[k]));
      c[k] = nc;
    }
    if (move < 1e-15) break;
  }
  for (int k = 0; k < L / 2; ++k) {
    double m = 0.5 * (c[L - 1 - k] - c[k]);
    c[k] = -m;
    c[L - 1 - k] = m;
  }
  double s = 1.0 / sqrt((double)d);
  for (int k = 0; k < L; ++k) c[k] *= s;
  for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
  return it;
}

extern "C" tq_status tq_codebook_compute(int head_dim, int bits, float* centroids,
                                         float* bounds) {
  if (!supported_dim(head_dim) || !supported_bits(bits)) return TQ_ERR_UNSUPPORTED;
  if (!centroids || !bounds) return TQ_ERR_ARG;
  double c[16], t[15];
  tq_lloyd_max_host(head_dim, bits, c, t);
  for (int k = 0; k < (1 << bits); ++k) centroids[k] = (float)c[k];
  for (int k = 0; k + 1 < (1 << bits); ++k) bounds[k] = (float)t[k];
  return TQ_OK;
}

/* ------------------------------------------------------ decoder LUT scale -- */

/* fp16 bits nearest (ties to even) to a positive double in fp16's normal range. */
static uint16_t half_rne_normal(double v) {
  uint64_t u;
  memcpy(&u, &v, 8);
  int e = (int)((u >> 52) & 0x7FF) - 1023;
  uint64_t sig = (u & 0x000FFFFFFFFFFFFFull) | (1ull << 52);
  uint64_t q = sig >> 42, rem = sig & ((1ull << 42) - 1), half = 1ull << 41;
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (q == 2048) { q = 1024; ++e; }
  return (uint16_t)(((e + 15) << 10) | (uint16_t)(q - 1024));
}

/* fp16 bits of v, round to nearest even, subnormals included (|v| < 65504). */
static uint16_t half_rne(double v) {
  const double a = fabs(v);
  uint16_t m;
  if (a < ldexp(1.0, -14)) {
    m = (uint16_t)nearbyint(ldexp(a, 24)); /* 1024 lands on the smallest normal */
  } else {
    m = half_rne_normal(a);
  }
  return (uint16_t)(v < 0 ? (m | 0x8000) : m);
}

static double half_value(uint16_t h) {
  int e = (h >> 10) & 31, f = h & 1023;
  double v = e ? ldexp(1024.0 + f, e - 25) : ldexp((double)f, -24);
  return (h & 0x8000) ? -v : v;
}

/* The decoder stores levels as fp16(c_k * sigma); queries are scaled by
 * 1/sigma and outputs by 1/sigma, so sigma cancels.  Pick sigma in [1, 2) that
 * minimises the worst relative fp16 rounding error over the levels. */
static float lut_scale(const double* c, int L) {
  double best = 1e300, best_s = 1.0;
  const int steps = 1 << 20;
  for (int i = 0; i < steps; ++i) {
    double s = 1.0 + (double)i / steps, worst = 0.0;
    for (int k = L / 2; k < L; ++k) {
      double v = c[k] * s;
      double r = fabs(half_value(half_rne_normal(v)) / v - 1.0);
      if (r > worst) worst = r;
      if (worst >= best) break;
    }
    if (worst < best) { best = worst; best_s = s; }
  }
  return (float)best_s;
}

/* --------------------------------------------------------------- handles -- */

static tq_status build_codebook(int d, int bits, tq_codebook_s* cb) {
  const int L = 1 << bits;
  cb->d = d;
  cb->bits = bits;
  tq_lloyd_max_host(d, bits, cb->centroids64, cb->bounds64);
  for (int k = 0; k < L; ++k) cb->centroids[k] = (float)cb->centroids64[k];
  for (int k = 0; k + 1 < L; ++k) cb->bounds[k] = (float)cb->bounds64[k];
  /* bucket width below 1/1.02 of the closest threshold gap, so that no
   * bucket holds two thresholds */
  double gap = 1e300;
  for (int k = 0; k + 2 < L; ++k) gap = fmin(gap, cb->bounds64[k + 1] - cb->bounds64[k]);
  int nbh = 1;
  while (nbh * gap <= 1.02) nbh *= 2;
  cb->nb_half = nbh;
  cb->enc_entries = 2 * nbh + 2;
  cb->sigma = lut_scale(cb->centroids64, L);
  return TQ_OK;
}

extern "C" tq_status tq_codebook_init(int head_dim, int bits, tq_codebook* out) {
  if (!out) return TQ_ERR_ARG;
  *out = nullptr;
  if (!supported_dim(head_dim) || !supported_bits(bits)) return TQ_ERR_UNSUPPORTED;
  tq_codebook_s* cb = (tq_codebook_s*)calloc(1, sizeof(tq_codebook_s));
  if (!cb) return TQ_ERR_ARG;
  build_codebook(head_dim, bits, cb);
  const int L = 1 << bits;

  /* encoder bucket table: the grid offset that keeps the thresholds
   * farthest from bucket edges (edges at half-integers of u) */
  const int ne = cb->enc_entries;
  const double nbh = cb->nb_half;
  double best_gap = -1.0;
  for (int i = 0; i < 90; ++i) {
    const double shift = 0.005 * i;
    double gap = 0.5;
    for (int k = 0; k + 1 < L; ++k) {
      const double g = (cb->bounds64[k] + 1.0) * nbh + shift; /* u - 1/2 */
      gap = fmin(gap, fabs(g - nearbyint(g)));
    }
    if (gap > best_gap) { best_gap = gap; cb->enc_shift = (float)shift; }
  }
  tq_enc_entry* et = (tq_enc_entry*)calloc((size_t)ne, sizeof(tq_enc_entry));
  double thr_u[15];
  for (int k = 0; k + 1 < L; ++k)
    thr_u[k] = (cb->bounds64[k] + 1.0) * nbh + 0.5 + (double)cb->enc_shift;
  for (int j = 0; j < ne; ++j) {
    uint32_t base = 0;
    float neg_t = -INFINITY;
    int inside = 0;
    for (int k = 0; k + 1 < L; ++k) {
      if (thr_u[k] < j - 0.5) ++base;
      else if (thr_u[k] < j + 0.5) { neg_t = (float)(-cb->bounds64[k] * nbh); ++inside; }
    }
    /* one threshold per bucket, thresholds clear of the bucket edges, and no
     * more rows than the kernels keep */
    if (inside > 1 || best_gap < 1.0 / 64 || ne > tq_enc_rows_max(head_dim, bits)) {
      free(et);
      free(cb);
      return TQ_ERR_UNSUPPORTED;
    }
    et[j].neg_t = neg_t;
    et[j].base = base;
  }
  /* decoder lookup table: fp16(level * sigma) */
  uint16_t h[16];
  for (int k = 0; k < L; ++k) {
    double v = cb->centroids64[k] * cb->sigma;
    uint16_t m = half_rne_normal(fabs(v));
    h[k] = (uint16_t)(v < 0 ? (m | 0x8000) : m);
  }
  /* Decoder tables (device copies are spread over LDS rows by the kernel):
   *  pair[e]:    the fp16 levels of the two codes held by index e (first
   *              code in the low half); e is a byte (bits 4), 6 bits (bits 3)
   *              or a nibble (bits 2).
   *  pair_lo[e]: the same codes' remainders fp16((level - fp16 level) * 2^11),
   *              so that hi + lo * 2^-11 carries a level to ~2^-22 relative
   *              (key scores at long context need more than fp16).
   *  quad[e]:    bits 2 only, e a byte of four codes: their four fp16 levels
   *              (two words, first code lowest). */
  uint16_t r16[16];
  for (int k = 0; k < L; ++k) {
    double v = cb->centroids64[k] * cb->sigma;
    r16[k] = half_rne((v - half_value(h[k])) * 2048.0);
  }
  const size_t pw = bits == 2 ? 16 : (bits == 3 ? 64 : 256);
  const size_t qw = bits == 2 ? 512 : 0;
  uint32_t* lut = (uint32_t*)calloc(2 * pw + qw + 16, 4);
  for (size_t e = 0; e < pw; ++e) {
    lut[e] = h[e & (L - 1)] | ((uint32_t)h[e >> bits] << 16);
    lut[pw + e] = r16[e & (L - 1)] | ((uint32_t)r16[e >> bits] << 16);
  }
  for (size_t e = 0; e < qw / 2; ++e) {
    lut[2 * pw + 2 * e] = h[e & 3] | ((uint32_t)h[(e >> 2) & 3] << 16);
    lut[2 * pw + 2 * e + 1] = h[(e >> 4) & 3] | ((uint32_t)h[(e >> 6) & 3] << 16);
  }
  /*  pre[k]:     per code, fp16(level * sigma * 2^e) and the fp16 of the
   *              exact remainder, e putting the largest level in [16, 32)
   *              (the many-query products add the remainder term in full
   *              precision instead of scaling it) */
  int pe = 0;
  {
    const double top = fabs(cb->centroids64[L - 1] * cb->sigma);
    while (top * ldexp(1.0, pe) < 16.0) ++pe;
    while (top * ldexp(1.0, pe) >= 32.0) --pe;
  }
  cb->pre_exp = pe;
  for (int k = 0; k < L; ++k) {
    const double v = ldexp(cb->centroids64[k] * cb->sigma, pe);
    const uint16_t hi = half_rne(v);
    lut[2 * pw + qw + k] = hi | ((uint32_t)half_rne(v - half_value(hi)) << 16);
  }
  const size_t lut_words = 2 * pw + qw + 16;
  size_t enc_bytes = ((size_t)ne * sizeof(tq_enc_entry) + 255) & ~(size_t)255;
  size_t total = enc_bytes + lut_words * 4;
  tq_status st = TQ_OK;
  if (hipGetDevice(&cb->device) != hipSuccess || hipMalloc(&cb->dev_mem, total) != hipSuccess) {
    st = TQ_ERR_DEVICE;
  } else if (hipMemcpy(cb->dev_mem, et, (size_t)ne * sizeof(tq_enc_entry),
                       hipMemcpyHostToDevice) != hipSuccess ||
             hipMemcpy((char*)cb->dev_mem + enc_bytes, lut, lut_words * 4,
                       hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(cb->dev_mem);
    st = TQ_ERR_DEVICE;
  }
  free(et);
  free(lut);
  if (st != TQ_OK) { free(cb); return st; }
  cb->enc_table = (const tq_enc_entry*)cb->dev_mem;
  cb->dec_lut = (const uint32_t*)((char*)cb->dev_mem + enc_bytes);
  cb->dec_lut_lo = cb->dec_lut + (bits == 2 ? 16 : (bits == 3 ? 64 : 256));
  cb->dec_quad = bits == 2 ? cb->dec_lut + 32 : nullptr;
  cb->pre_klut = cb->dec_lut + 2 * pw + qw;
  *out = cb;
  return TQ_OK;
}

extern "C" tq_status tq_codebook_read(tq_codebook cb, float* centroids, float* bounds) {
  if (!cb || !centroids || !bounds) return TQ_ERR_ARG;
  for (int k = 0; k < (1 << cb->bits); ++k) centroids[k] = cb->centroids[k];
  for (int k = 0; k + 1 < (1 << cb->bits); ++k) bounds[k] = cb->bounds[k];
  return TQ_OK;
}

extern "C" int tq_codebook_head_dim(tq_codebook cb) { return cb ? cb->d : 0; }
extern "C" int tq_codebook_bits(tq_codebook cb) { return cb ? cb->bits : 0; }

extern "C" void tq_codebook_free(tq_codebook cb) {
  if (!cb) return;
  if (cb->dev_mem) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != cb->device) (void)hipSetDevice(cb->device);
    (void)hipDeviceSynchronize();
    (void)hipFree(cb->dev_mem);
    if (cur >= 0 && cur != cb->device) (void)hipSetDevice(cur);
  }
  free(cb);
}

/* ------------------------------------------------------------ validation -- */

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

extern "C" tq_status tq_encode(tq_codebook cb, const uint16_t* x, int64_t n, int64_t x_stride,
                               const uint8_t* sign_bits, uint8_t* codes, uint16_t* norms,
                               void* stream) {
  if (!cb || n < 0) return TQ_ERR_ARG;
  if (n == 0) return TQ_OK;
  if (!x || !sign_bits || !codes || !norms) return TQ_ERR_ARG;
  if (x_stride < cb->d || x_stride % 8 != 0) return TQ_ERR_ARG;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(norms, 2) || !aligned(sign_bits, 4))
    return TQ_ERR_ARG;
  return tq_launch_encode_rows(cb, x, n, x_stride, sign_bits, codes, norms,
                               (hipStream_t)stream);
}

/* Rows of one layer's storage: batch * heads * capacity (contiguous), or the
 * pool's num_pages * heads * page_tokens (paged). */
static int64_t storage_rows(const tq_kv_cache* c) {
  return c->block_table ? (int64_t)c->num_pages * c->kv_heads * c->page_tokens
                        : (int64_t)c->batch * c->kv_heads * c->capacity;
}

/* Shape checks shared by the entry points and tq_cache_layer_bytes. */
static tq_status check_shape(const tq_kv_cache* c) {
  if (!c) return TQ_ERR_ARG;
  if (!supported_dim(c->head_dim) || !supported_bits(c->bits_k) || !supported_bits(c->bits_v))
    return TQ_ERR_UNSUPPORTED;
  if (c->batch <= 0 || c->kv_heads <= 0 || c->capacity <= 0 || c->capacity % 32 != 0)
    return TQ_ERR_ARG;
  const int maxbits = c->bits_k > c->bits_v ? c->bits_k : c->bits_v;
  if (c->block_table) {
    const int p = c->page_tokens;
    if (p < 32 || (p & (p - 1)) != 0 || c->max_pages <= 0 || c->num_pages <= 0 ||
        (int64_t)c->max_pages * p != c->capacity || !aligned(c->block_table, 4))
      return TQ_ERR_ARG;
    /* a layer's pool is addressed with 32-bit offsets */
    if (storage_rows(c) * c->head_dim * maxbits / 8 >= ((int64_t)1 << 31)) return TQ_ERR_UNSUPPORTED;
  } else {
    /* one (sequence, head) stream of codes is addressed with 32-bit offsets */
    if ((int64_t)c->capacity * c->head_dim * maxbits / 8 >= ((int64_t)1 << 31))
      return TQ_ERR_UNSUPPORTED;
  }
  return TQ_OK;
}

static tq_status check_cache(const tq_kv_cache* c) {
  const tq_status st = check_shape(c);
  if (st != TQ_OK) return st;
  if (!c->k_codes || !c->v_codes || !c->k_norms || !c->v_norms) return TQ_ERR_ARG;
  if (!aligned(c->k_codes, 16) || !aligned(c->v_codes, 16) || !aligned(c->k_norms, 8) ||
      !aligned(c->v_norms, 8))
    return TQ_ERR_ARG;
  if (c->layer_stride_k_codes % 16 || c->layer_stride_v_codes % 16 ||
      c->layer_stride_k_norms % 16 || c->layer_stride_v_norms % 16)
    return TQ_ERR_ARG;
  return TQ_OK;
}

extern "C" tq_status tq_cache_layer_bytes(const tq_kv_cache* c, int64_t* k_codes,
                                          int64_t* v_codes, int64_t* k_norms,
                                          int64_t* v_norms) {
  const tq_status st = check_shape(c);
  if (st != TQ_OK) return st;
  const int64_t rows = storage_rows(c);
  if (k_codes) *k_codes = rows * c->head_dim * c->bits_k / 8;
  if (v_codes) *v_codes = rows * c->head_dim * c->bits_v / 8;
  if (k_norms) *k_norms = rows * 2;
  if (v_norms) *v_norms = rows * 2;
  return TQ_OK;
}

static bool codebook_matches(const tq_codebook_s* cb, int d, int bits) {
  return cb && cb->d == d && cb->bits == bits;
}

extern "C" tq_status tq_append(const tq_kv_cache* c, tq_codebook cbk, tq_codebook cbv,
                               const uint8_t* sign_bits, const uint16_t* k_new,
                               const uint16_t* v_new, int t_new, const int32_t* pos,
                               int32_t host_max_pos, int n_layers, void* stream) {
  tq_status st = check_cache(c);
  if (st != TQ_OK) return st;
  if (!codebook_matches(cbk, c->head_dim, c->bits_k) ||
      !codebook_matches(cbv, c->head_dim, c->bits_v))
    return TQ_ERR_ARG;
  if (t_new < 0 || n_layers < 1) return TQ_ERR_ARG;
  if (t_new == 0) return TQ_OK;
  if (!sign_bits || !k_new || !v_new || !pos) return TQ_ERR_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(pos, 4) || !aligned(sign_bits, 4))
    return TQ_ERR_ARG;
  if (host_max_pos < -1) return TQ_ERR_ARG;
  if (host_max_pos >= 0 && (int64_t)host_max_pos + t_new > c->capacity) return TQ_ERR_CAPACITY;
  return tq_launch_append(c, cbk, cbv, sign_bits, k_new, v_new, t_new, pos, n_layers,
                          (hipStream_t)stream);
}

static tq_status check_decode(const tq_kv_cache* c, int q_heads, int max_len, int n_layers) {
  tq_status st = check_cache(c);
  if (st != TQ_OK) return st;
  if (q_heads <= 0 || n_layers < 1 || max_len < 0 || max_len > c->capacity) return TQ_ERR_ARG;
  if (q_heads % c->kv_heads != 0) return TQ_ERR_ARG;
  if (q_heads / c->kv_heads > 8) return TQ_ERR_UNSUPPORTED;
  return TQ_OK;
}

extern "C" size_t tq_decode_workspace_bytes(const tq_kv_cache* c, int q_heads, int max_len,
                                            int n_layers) {
  if (check_decode(c, q_heads, max_len, n_layers) != TQ_OK) return 0;
  return tq_plan_decode(c, q_heads, max_len, n_layers).ws_bytes;
}

static tq_status decode_common(const tq_kv_cache* c, tq_codebook cbk, tq_codebook cbv,
                               const uint8_t* sign_bits, const uint16_t* q, int q_heads,
                               const int32_t* seq_lens, int max_len, int n_layers, float* out,
                               void* ws, size_t ws_bytes, float sparse_eps,
                               uint32_t* skip_counts, uint32_t* skip_tiles, void* stream) {
  tq_status st = check_decode(c, q_heads, max_len, n_layers);
  if (st != TQ_OK) return st;
  if (!codebook_matches(cbk, c->head_dim, c->bits_k) ||
      !codebook_matches(cbv, c->head_dim, c->bits_v))
    return TQ_ERR_ARG;
  if (!sign_bits || !q || !seq_lens || !out) return TQ_ERR_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(seq_lens, 4)) return TQ_ERR_ARG;
  tq_decode_plan plan = tq_plan_decode(c, q_heads, max_len, n_layers);
  if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes || !aligned(ws, 256)))
    return TQ_ERR_WORKSPACE;
  return tq_launch_decode(c, cbk, cbv, sign_bits, q, q_heads, seq_lens, max_len, n_layers, out,
                          ws, plan, sparse_eps, skip_counts, skip_tiles, (hipStream_t)stream);
}

extern "C" tq_status tq_decode_attn(const tq_kv_cache* c, tq_codebook cbk, tq_codebook cbv,
                                    const uint8_t* sign_bits, const uint16_t* q, int q_heads,
                                    const int32_t* seq_lens, int max_len, int n_layers,
                                    float* out, void* ws, size_t ws_bytes, void* stream) {
  return decode_common(c, cbk, cbv, sign_bits, q, q_heads, seq_lens, max_len, n_layers, out, ws,
                       ws_bytes, 0.0f, nullptr, nullptr, stream);
}

extern "C" tq_status tq_decode_attn_noalloc(const tq_kv_cache* c, tq_codebook cbk,
                                            tq_codebook cbv, const uint8_t* sign_bits,
                                            const uint16_t* q, int q_heads,
                                            const int32_t* seq_lens, int max_len, int n_layers,
                                            float* out, void* stream) {
  tq_status st = check_decode(c, q_heads, max_len, n_layers);
  if (st != TQ_OK) return st;
  if (!codebook_matches(cbk, c->head_dim, c->bits_k) ||
      !codebook_matches(cbv, c->head_dim, c->bits_v))
    return TQ_ERR_ARG;
  if (!sign_bits || !q || !seq_lens || !out) return TQ_ERR_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(seq_lens, 4)) return TQ_ERR_ARG;
  const tq_decode_plan plan = tq_plan_decode(c, q_heads, max_len, n_layers);
  if (plan.ws_bytes > TQ_NOALLOC_SCRATCH_BYTES) return TQ_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan.ws_bytes > 0) {
    st = tq_noalloc_scratch(&ws, (hipStream_t)stream);
    if (st != TQ_OK) return st;
  }
  return tq_launch_decode(c, cbk, cbv, sign_bits, q, q_heads, seq_lens, max_len, n_layers, out,
                          ws, plan, 0.0f, nullptr, nullptr, (hipStream_t)stream);
}

extern "C" tq_status tq_prefill_attn(const tq_kv_cache* c, tq_codebook cbk, tq_codebook cbv,
                                     const uint8_t* sign_bits, const uint16_t* q, int q_heads,
                                     int t_new, const int32_t* pos, int n_layers, float* out,
                                     void* stream) {
  tq_status st = check_decode(c, q_heads, 0, n_layers);
  if (st != TQ_OK) return st;
  if (t_new < 0) return TQ_ERR_ARG;
  if (!codebook_matches(cbk, c->head_dim, c->bits_k) ||
      !codebook_matches(cbv, c->head_dim, c->bits_v))
    return TQ_ERR_ARG;
  if (!sign_bits || !q || !pos || !out) return TQ_ERR_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(pos, 4)) return TQ_ERR_ARG;
  if (t_new == 0) return TQ_OK;
  return tq_launch_prefill(c, cbk, cbv, sign_bits, q, q_heads, t_new, pos, n_layers, out,
                           (hipStream_t)stream);
}

extern "C" tq_status tq_qjl_encode(tq_codebook cb, const uint16_t* x, int64_t n,
                                   int64_t x_stride, const uint8_t* sign_bits, const uint16_t* S,
                                   const uint8_t* codes, uint8_t* signs, uint16_t* gamma,
                                   void* stream) {
  if (!cb || n < 0) return TQ_ERR_ARG;
  if (n == 0) return TQ_OK;
  const int d = cb->d;
  if (!x || !sign_bits || !S || !codes || !signs || !gamma) return TQ_ERR_ARG;
  if (x_stride < d || x_stride % 8 != 0 || !aligned(x, 16) || !aligned(S, 16) ||
      !aligned(codes, 8) || !aligned(signs, 4) || !aligned(gamma, 2))
    return TQ_ERR_ARG;
  return tq_launch_qjl_encode(cb, x, n, x_stride, sign_bits, S, codes, signs, gamma,
                              (hipStream_t)stream);
}

extern "C" tq_status tq_qjl_scores(tq_codebook cb, const uint16_t* q, int n_q,
                                   const uint8_t* sign_bits, const uint16_t* S,
                                   const uint8_t* codes, const uint16_t* norms,
                                   const uint8_t* signs, const uint16_t* gamma, int64_t n_keys,
                                   float* out, void* stream) {
  if (!cb || n_keys < 0) return TQ_ERR_ARG;
  if (n_q < 1 || n_q > 8) return TQ_ERR_UNSUPPORTED;
  if (n_keys == 0) return TQ_OK;
  if (!q || !sign_bits || !S || !codes || !norms || !signs || !gamma || !out) return TQ_ERR_ARG;
  if (!aligned(q, 2) || !aligned(norms, 2) || !aligned(gamma, 2) || !aligned(out, 4) ||
      !aligned(S, 2) || !aligned(codes, 8) || !aligned(signs, 4))
    return TQ_ERR_ARG;
  return tq_launch_qjl_scores(cb, q, n_q, sign_bits, S, codes, norms, signs, gamma, n_keys, out,
                              (hipStream_t)stream);
}

extern "C" tq_status tq_decode_attn_sparse(const tq_kv_cache* c, tq_codebook cbk,
                                           tq_codebook cbv, const uint8_t* sign_bits,
                                           const uint16_t* q, int q_heads,
                                           const int32_t* seq_lens, int max_len, int n_layers,
                                           float eps, uint32_t* skip_counts,
                                           uint32_t* skip_tiles, float* out, void* ws,
                                           size_t ws_bytes, void* stream) {
  if (!(eps >= 0.0f) || eps == INFINITY) return TQ_ERR_ARG; /* NaN, negative or infinite */
  if (skip_counts && !aligned(skip_counts, 4)) return TQ_ERR_ARG;
  if (skip_tiles && !aligned(skip_tiles, 4)) return TQ_ERR_ARG;
  return decode_common(c, cbk, cbv, sign_bits, q, q_heads, seq_lens, max_len, n_layers, out, ws,
                       ws_bytes, eps, skip_counts, skip_tiles, stream);
}
