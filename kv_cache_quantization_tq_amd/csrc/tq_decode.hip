/*
 * gfx950 decode attention over the compressed cache.
 *
 * Math (per layer, sequence, KV head; G query heads share the pass):
 *   q'' = H D q * log2(e) / (d * sigma_K)          rotated query, softmax scale
 *                                                 and log2 folded in
 *   s_gj = n_j * sum_i q''_gi * (sigma_K c_K[code_ji])   = log2(e) q_g.k_j / sqrt d
 *   online softmax in base 2 over j;  acc_g = sum_j p_gj m_j (sigma_V c_V[code_j])
 *   o_g = D H acc_g / (sqrt(d) sigma_V l_g)        one inverse FWHT at the end
 * ("We Built a Python Library That Cuts LLM Memory Usage by 80%", "Test Suite":
 * softmax(Q K^T / sqrt d) V; AdapTQ page, "How it works (HAR + VQ)", step 3:
 * the query is rotated once and scored against the packed codes through
 * lookup tables; the inverse rotation exists because the FWHT is reversible,
 * "TurboQuant ... FWHT Preprocessing", "FWHT Preprocessing Layer".)
 *
 * Both products run on the matrix cores (v_mfma_f32_16x16x32_f16) with fp16
 * operands dequantized through byte-indexed lookup tables in LDS:
 *   scores: S^T[16 tokens x 16 cols] = Kdeq[16 x 32 coords] * Q[32 x 16 cols],
 *           columns 0..7 carry fp16(q'') of the G heads and columns 8..15 the
 *           fp16 remainder q'' - fp16(q''); a row_ror:8 DPP add joins them.
 *   values: Acc^T[16 coords x 16 cols] += Vdeq[16 x 32 tokens] * P'[32 x 16],
 *           P' = fp16(p * m_j), one MFMA per 16 coordinates.
 * The levels are stored as fp16(c * sigma) with sigma chosen per codebook to
 * minimise their fp16 rounding; sigma is divided out of the query and output.
 *
 * Lane roles in a wave (lane = 16 q4 + n):
 *   K operand: token n of a 16-token block, coordinates [q4 d/4, (q4+1) d/4)
 *              of its row, which is one contiguous d*bits/32-byte load;
 *   score out: tokens 4 q4 .. 4 q4 + 3 of the block, column n;
 *   V operand: segment lane of the 32-token value tile (see tq.h);
 *   value out: coordinates [q4 d/4, (q4+1) d/4) of head n.
 */
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;        /* waves per workgroup */
constexpr int kRep = 8;          /* lookup-table copies in LDS (lane % kRep) */
constexpr float kLog2e = 1.4426950408889634f;

template <int B>
struct Lut {
  /* bits 2: byte -> 4 halves (2 words); 3: 6 bits -> 2 halves; 4: byte -> 2 halves */
  static constexpr int ENTRIES = B == 3 ? 64 : 256;
  static constexpr int WORDS = B == 2 ? 2 : 1;
  static constexpr int BYTES = ENTRIES * WORDS * 4 * kRep;
};

/* Copy a lookup table into LDS with kRep interleaved copies:
 * entry e copy r at word (e * kRep + r) * WORDS. */
template <int B>
__device__ inline void load_lut(uint32_t* dst, const uint32_t* src) {
  constexpr int W = Lut<B>::WORDS;
  for (int i = threadIdx.x; i < Lut<B>::ENTRIES * kRep; i += blockDim.x) {
    const int e = i / kRep;
#pragma unroll
    for (int w = 0; w < W; ++w) dst[i * W + w] = src[e * W + w];
  }
}

/* Dequantize an 8*B-bit field (8 codes) into 8 fp16 (4 words). */
template <int B>
__device__ inline u32x4 deq8(const uint32_t* lut, uint32_t f) {
  u32x4 o;
  if constexpr (B == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = lut[((f >> (8 * k)) & 0xFFu) * kRep];
  } else if constexpr (B == 3) {
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = lut[((f >> (6 * k)) & 0x3Fu) * kRep];
  } else {
    const uint2 a = *(const uint2*)(lut + ((f & 0xFFu) * kRep) * 2);
    const uint2 b = *(const uint2*)(lut + (((f >> 8) & 0xFFu) * kRep) * 2);
    o[0] = a.x;
    o[1] = a.y;
    o[2] = b.x;
    o[3] = b.y;
  }
  return o;
}

/* Bits [8*B*s, 8*B*(s+1)) of a little-endian bit string held in words. */
template <int B, int NW>
__device__ inline uint32_t field(const uint32_t (&w)[NW], int s) {
  const int off = 8 * B * s;
  const int i = off / 32, sh = off % 32;
  if constexpr (B == 4) return w[i];
  uint64_t v = w[i];
  if (i + 1 < NW) v |= (uint64_t)w[i + 1] << 32;
  return (uint32_t)(v >> sh) & ((1u << (8 * B)) - 1u);
}

/* Load N bytes (N % 4 == 0 or N == 6) from p, aligned to A bytes. */
template <int N, int A>
__device__ inline void load_words(const uint8_t* p, uint32_t (&w)[(N + 3) / 4]) {
  if constexpr (A >= 16 && N % 16 == 0) {
#pragma unroll
    for (int k = 0; k < N / 16; ++k) {
      uint4 t = *(const uint4*)(p + 16 * k);
      w[4 * k] = t.x; w[4 * k + 1] = t.y; w[4 * k + 2] = t.z; w[4 * k + 3] = t.w;
    }
  } else if constexpr (A >= 8 && N % 8 == 0) {
#pragma unroll
    for (int k = 0; k < N / 8; ++k) {
      uint2 t = *(const uint2*)(p + 8 * k);
      w[2 * k] = t.x; w[2 * k + 1] = t.y;
    }
  } else if constexpr (A >= 4 && N % 4 == 0) {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) w[k] = *(const uint32_t*)(p + 4 * k);
  } else {
    static_assert(N == 6, "unsupported load");
    const uint16_t* h = (const uint16_t*)p;
    w[0] = h[0] | ((uint32_t)h[1] << 16);
    w[1] = h[2];
  }
}

__device__ inline float ror8_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
}

__device__ inline float h2f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
__device__ inline uint32_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

template <int D, int BK, int BV>
struct DecGeo {
  static constexpr int KQ = D / 4;              /* coordinates per lane quarter */
  static constexpr int KS = D / 32;             /* score MFMAs per block */
  static constexpr int VM = D / 16;             /* value MFMAs per tile */
  static constexpr int RB = D * BK / 8;         /* key row bytes */
  static constexpr int KB = KQ * BK / 8;        /* key bytes per lane per token */
  static constexpr int KW = (KB + 3) / 4;
  static constexpr int KA = (KB % 16 == 0) ? 16 : (KB % 8 == 0 ? 8 : (KB % 4 == 0 ? 4 : 2));
  static constexpr int SEG = D * BV / 16;       /* value segment bytes */
  static constexpr int VW = SEG / 4;
  static constexpr int VA = (SEG % 16 == 0) ? 16 : (SEG % 8 == 0 ? 8 : 4);
  static constexpr int TILE = 32 * D * BV / 8;  /* value tile bytes */
};

struct DecArgs {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint8_t* k_norms;
  const uint8_t* v_norms;
  int64_t ls_kc, ls_vc, ls_kn, ls_vn;
  int batch, kv_heads, capacity, q_heads, group, n_layers;
  int max_len, splits, tiles_per_split;
  const uint8_t* sign_bits;
  const uint16_t* q;
  const int32_t* seq_lens;
  const uint32_t* lut_k;
  const uint32_t* lut_v;
  float qscale;    /* log2(e) / (d * sigma_K) */
  float oscale;    /* 1 / (sqrt(d) * sigma_V) */
  float* out;
  float* ws;
};

/* In-LDS Walsh-Hadamard transform of G rows of D floats (block-wide). */
template <int D>
__device__ inline void lds_fwht(float* buf, int G) {
  for (int h = 1; h < D; h <<= 1) {
    for (int t = threadIdx.x; t < G * D / 2; t += blockDim.x) {
      const int g = t / (D / 2), k = t % (D / 2);
      const int i = (k / h) * 2 * h + (k % h);
      float* r = buf + g * D;
      const float a = r[i], b = r[i + h];
      r[i] = a + b;
      r[i + h] = a - b;
    }
    __syncthreads();
  }
}

template <int D, int BK, int BV>
__global__ void __launch_bounds__(64 * kWaves)
decode_kernel(DecArgs a) {
  using DG = DecGeo<D, BK, BV>;
  extern __shared__ __align__(16) char smem[];
  uint32_t* lut_k = (uint32_t*)smem;
  uint32_t* lut_v = (uint32_t*)(smem + Lut<BK>::BYTES);
  const int lut_bytes = Lut<BK>::BYTES + Lut<BV>::BYTES;
  const int merge_bytes = kWaves * (8 * D + 16) * 4;
  float* qbuf = (float*)(smem + (lut_bytes > merge_bytes ? lut_bytes : merge_bytes));
  float* mbuf = (float*)smem; /* aliases the tables after the token loop */

  const int G = a.group;
  const int split = blockIdx.x % a.splits;
  int64_t unit = blockIdx.x / a.splits;
  const int kv = (int)(unit % a.kv_heads);
  unit /= a.kv_heads;
  const int b = (int)(unit % a.batch);
  const int layer = (int)(unit / a.batch);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int q4 = lane / 16, n = lane % 16;

  load_lut<BK>(lut_k, a.lut_k);
  load_lut<BV>(lut_v, a.lut_v);
  /* rotated queries: qbuf[g][i] = (D q_g)_i, then FWHT, then scale */
  const uint8_t* sb = a.sign_bits + (int64_t)layer * (D / 8);
  const uint16_t* qg = a.q + (((int64_t)layer * a.batch + b) * a.q_heads + (int64_t)kv * G) * D;
  for (int t = threadIdx.x; t < G * D; t += blockDim.x) {
    const int i = t % D;
    const float v = h2f(qg[t]);
    qbuf[t] = ((sb[i >> 3] >> (i & 7)) & 1) ? -v : v;
  }
  __syncthreads();
  lds_fwht<D>(qbuf, G);

  /* B operands of the score products (hi part in columns 0..7, lo in 8..15) */
  half8 bq[DG::KS];
  {
    const int g = n & 7;
#pragma unroll
    for (int s = 0; s < DG::KS; ++s) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float v = g < G ? qbuf[g * D + q4 * DG::KQ + 8 * s + r] * a.qscale : 0.0f;
        _Float16 hi = (_Float16)v;
        bq[s][r] = n < 8 ? hi : (_Float16)(v - (float)hi);
      }
    }
  }

  int len = a.seq_lens[b];
  len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
  const int ntiles = (len + 31) / 32;
  const int t_begin = split * a.tiles_per_split;
  int t_end = t_begin + a.tiles_per_split;
  if (t_end > ntiles) t_end = ntiles;

  const int64_t sh = (int64_t)b * a.kv_heads + kv;
  const uint8_t* kbase = a.k_codes + layer * a.ls_kc + sh * a.capacity * DG::RB + q4 * DG::KB;
  const uint8_t* vbase = a.v_codes + layer * a.ls_vc + sh * (a.capacity / 32) * DG::TILE +
                         lane * DG::SEG;
  const uint16_t* knb = (const uint16_t*)(a.k_norms + layer * a.ls_kn) + sh * a.capacity + 4 * q4;
  const uint16_t* vnb = (const uint16_t*)(a.v_norms + layer * a.ls_vn) + sh * a.capacity + 4 * q4;
  const uint32_t* lk = lut_k + (lane % kRep) * Lut<BK>::WORDS;
  const uint32_t* lv = lut_v + (lane % kRep) * Lut<BV>::WORDS;

  floatx4 acc[DG::VM];
#pragma unroll
  for (int m = 0; m < DG::VM; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.0f;

  for (int tile = t_begin + wave; tile < t_end; tile += kWaves) {
    const int tok0 = tile * 32;
    uint32_t kw0[DG::KW], kw1[DG::KW], vw[DG::VW];
    load_words<DG::KB, DG::KA>(kbase + (int64_t)(tok0 + n) * DG::RB, kw0);
    load_words<DG::KB, DG::KA>(kbase + (int64_t)(tok0 + 16 + n) * DG::RB, kw1);
    load_words<DG::SEG, DG::VA>(vbase + (int64_t)tile * DG::TILE, vw);
    const uint2 kn0 = *(const uint2*)(knb + tok0);
    const uint2 kn1 = *(const uint2*)(knb + tok0 + 16);
    const uint2 vn0 = *(const uint2*)(vnb + tok0);
    const uint2 vn1 = *(const uint2*)(vnb + tok0 + 16);

    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DG::KS; ++s) {
      const u32x4 a0 = deq8<BK>(lk, field<BK>(kw0, s));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a0), bq[s], s0, 0, 0, 0);
      const u32x4 a1 = deq8<BK>(lk, field<BK>(kw1, s));
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a1), bq[s], s1, 0, 0, 0);
    }
    /* scores of tokens tok0 + 4 q4 + i (block 0) and tok0 + 16 + 4 q4 + i */
    float sc[8];
    const uint32_t knw[4] = {kn0.x, kn0.y, kn1.x, kn1.y};
    const uint32_t vnw[4] = {vn0.x, vn0.y, vn1.x, vn1.y};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = ror8_add(s0[i]);
      sc[4 + i] = ror8_add(s1[i]);
    }
    float mt = -1e30f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int tok = tok0 + (u < 4 ? 4 * q4 + u : 16 + 4 * q4 + (u - 4));
      const uint32_t kh = (knw[u / 2] >> (16 * (u & 1))) & 0xFFFFu;
      const float v = sc[u] * h2f(kh);
      sc[u] = tok < len ? v : -INFINITY;
      mt = fmaxf(mt, sc[u]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    if (__any(m_new > m_run)) { /* rescale the running sums, lazily */
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int m = 0; m < DG::VM; ++m) acc[m] *= alpha;
      m_run = m_new;
    }
    half8 pb;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float p = __builtin_amdgcn_exp2f(sc[u] - m_run);
      l_run += p;
      const uint32_t vh = (vnw[u / 2] >> (16 * (u & 1))) & 0xFFFFu;
      const int tok = tok0 + (u < 4 ? 4 * q4 + u : 16 + 4 * q4 + (u - 4));
      pb[u] = tok < len ? (_Float16)(p * h2f(vh)) : (_Float16)0.0f;
    }
#pragma unroll
    for (int m = 0; m < DG::VM; ++m) {
      const u32x4 av = deq8<BV>(lv, field<BV>(vw, m));
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av), pb, acc[m], 0, 0, 0);
    }
  }
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  /* merge the waves: mbuf[w] = {m[8], l[8], acc[8][D]} */
  __syncthreads(); /* tables are dead from here on */
  float* mw = mbuf + wave * (8 * D + 16);
  if (n < 8) {
    if (q4 == 0) {
      mw[n] = m_run;
      mw[8 + n] = l_run;
    }
#pragma unroll
    for (int m = 0; m < DG::VM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) mw[16 + n * D + (4 * q4 + i) * DG::VM + m] = acc[m][i];
  }
  __syncthreads();
  /* merged record per head in qbuf (reused): qbuf[g][i] */
  float* res = qbuf;
  __shared__ float mg[8], lg[8];
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = -1e30f;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mbuf[w * (8 * D + 16) + g]);
    float L = 0.0f;
    for (int w = 0; w < kWaves; ++w) {
      const float* r = mbuf + w * (8 * D + 16);
      L += __builtin_amdgcn_exp2f(r[g] - M) * r[8 + g];
    }
    mg[g] = M;
    lg[g] = L;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G * D; t += blockDim.x) {
    const int g = t / D, i = t % D;
    float s = 0.0f;
    for (int w = 0; w < kWaves; ++w) {
      const float* r = mbuf + w * (8 * D + 16);
      s += __builtin_amdgcn_exp2f(r[g] - mg[g]) * r[16 + g * D + i];
    }
    res[t] = s;
  }
  __syncthreads();
  const int64_t head0 = ((int64_t)layer * a.batch + b) * a.q_heads + (int64_t)kv * G;
  if (a.splits == 1) {
    lds_fwht<D>(res, G);
    for (int t = threadIdx.x; t < G * D; t += blockDim.x) {
      const int g = t / D, i = t % D;
      const float L = lg[g];
      float v = L > 0.0f ? res[t] * a.oscale / L : 0.0f;
      if ((sb[i >> 3] >> (i & 7)) & 1) v = -v;
      a.out[head0 * D + t] = v;
    }
  } else {
    /* partial record per (head, split): {m, l, acc[D]} */
    for (int t = threadIdx.x; t < G * (D + 2); t += blockDim.x) {
      const int g = t / (D + 2), k = t % (D + 2);
      float* rec = a.ws + ((head0 + g) * a.splits + split) * (D + 2);
      rec[k] = k == 0 ? mg[g] : (k == 1 ? lg[g] : res[g * D + (k - 2)]);
    }
  }
}

/* Merge the split records of one head and rotate back: one block per head. */
template <int D>
__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ ws, int splits, const uint8_t* __restrict__ sign_bits,
               int heads_per_layer, float oscale, float* __restrict__ out) {
  __shared__ float buf[D];
  __shared__ float ML[2];
  const int64_t head = blockIdx.x;
  const int layer = (int)(head / heads_per_layer);
  const float* rec = ws + head * splits * (D + 2);
  if (threadIdx.x == 0) {
    float M = -1e30f;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, rec[s * (D + 2)]);
    float L = 0.0f;
    for (int s = 0; s < splits; ++s)
      L += __builtin_amdgcn_exp2f(rec[s * (D + 2)] - M) * rec[s * (D + 2) + 1];
    ML[0] = M;
    ML[1] = L;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < D; i += blockDim.x) {
    float acc = 0.0f;
    for (int s = 0; s < splits; ++s)
      acc += __builtin_amdgcn_exp2f(rec[s * (D + 2)] - ML[0]) * rec[s * (D + 2) + 2 + i];
    buf[i] = acc;
  }
  __syncthreads();
  lds_fwht<D>(buf, 1);
  const uint8_t* sb = sign_bits + (int64_t)layer * (D / 8);
  for (int i = threadIdx.x; i < D; i += blockDim.x) {
    float v = ML[1] > 0.0f ? buf[i] * oscale / ML[1] : 0.0f;
    if ((sb[i >> 3] >> (i & 7)) & 1) v = -v;
    out[head * D + i] = v;
  }
}

template <int D, int BK, int BV>
tq_status launch_decode_t(const DecArgs& a, hipStream_t s) {
  const int lut_bytes = Lut<BK>::BYTES + Lut<BV>::BYTES;
  const int merge_bytes = kWaves * (8 * D + 16) * 4;
  const size_t lds = (size_t)(lut_bytes > merge_bytes ? lut_bytes : merge_bytes) + 8 * D * 4;
  const int64_t blocks = (int64_t)a.n_layers * a.batch * a.kv_heads * a.splits;
  hipLaunchKernelGGL((decode_kernel<D, BK, BV>), dim3((unsigned)blocks), dim3(64 * kWaves), lds, s,
                     a);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_DEVICE;
  if (a.splits > 1) {
    const int64_t heads = (int64_t)a.n_layers * a.batch * a.q_heads;
    hipLaunchKernelGGL((combine_kernel<D>), dim3((unsigned)heads), dim3(256), 0, s, a.ws,
                       a.splits, a.sign_bits, a.batch * a.q_heads, a.oscale, a.out);
    if (hipGetLastError() != hipSuccess) return TQ_ERR_DEVICE;
  }
  return TQ_OK;
}

}  // namespace

tq_decode_plan tq_plan_decode(const tq_kv_cache* c, int q_heads, int max_len, int n_layers) {
  tq_decode_plan p;
  const int64_t units = (int64_t)n_layers * c->batch * c->kv_heads;
  const int tiles = (max_len + 31) / 32;
  const int64_t target_blocks = 1024;
  int splits = (int)((target_blocks + units - 1) / units);
  const int max_splits = tiles / (4 * kWaves);
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  p.splits = splits;
  p.tiles_per_split = tiles > 0 ? (tiles + splits - 1) / splits : 0;
  p.ws_bytes = splits > 1 ? (size_t)n_layers * c->batch * q_heads * splits *
                                (c->head_dim + 2) * sizeof(float)
                          : 0;
  return p;
}

tq_status tq_launch_decode(const tq_kv_cache* c, const tq_codebook_s* cbk,
                           const tq_codebook_s* cbv, const uint8_t* sign_bits,
                           const uint16_t* q, int q_heads, const int32_t* seq_lens,
                           int max_len, int n_layers, float* out, void* ws,
                           const tq_decode_plan& plan, hipStream_t s) {
  DecArgs a;
  a.k_codes = c->k_codes;
  a.v_codes = c->v_codes;
  a.k_norms = (const uint8_t*)c->k_norms;
  a.v_norms = (const uint8_t*)c->v_norms;
  a.ls_kc = c->layer_stride_k_codes;
  a.ls_vc = c->layer_stride_v_codes;
  a.ls_kn = c->layer_stride_k_norms;
  a.ls_vn = c->layer_stride_v_norms;
  a.batch = c->batch;
  a.kv_heads = c->kv_heads;
  a.capacity = c->capacity;
  a.q_heads = q_heads;
  a.group = q_heads / c->kv_heads;
  a.n_layers = n_layers;
  a.max_len = max_len;
  a.splits = plan.splits;
  a.tiles_per_split = plan.tiles_per_split;
  a.sign_bits = sign_bits;
  a.q = q;
  a.seq_lens = seq_lens;
  a.lut_k = cbk->dec_lut;
  a.lut_v = cbv->dec_lut;
  const double d = c->head_dim;
  a.qscale = (float)(1.4426950408889634 / (d * cbk->sigma));
  a.oscale = (float)(1.0 / (sqrt(d) * cbv->sigma));
  a.out = out;
  a.ws = (float*)ws;
#define TQ_DEC(DD, KK, VV) \
  if (c->head_dim == DD && c->bits_k == KK && c->bits_v == VV) return launch_decode_t<DD, KK, VV>(a, s);
#define TQ_DEC_D(DD) \
  TQ_DEC(DD, 2, 2) TQ_DEC(DD, 2, 3) TQ_DEC(DD, 2, 4) TQ_DEC(DD, 3, 2) TQ_DEC(DD, 3, 3) \
  TQ_DEC(DD, 3, 4) TQ_DEC(DD, 4, 2) TQ_DEC(DD, 4, 3) TQ_DEC(DD, 4, 4)
  TQ_DEC_D(64) TQ_DEC_D(128) TQ_DEC_D(256)
#undef TQ_DEC_D
#undef TQ_DEC
  return TQ_ERR_UNSUPPORTED;
}
