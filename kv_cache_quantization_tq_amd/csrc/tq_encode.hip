/*
 * gfx950 encode kernels: fp16 vector -> fp16 norm + b-bit codes.
 *
 * Per vector ("We Built a Python Library That Cuts LLM Memory Usage by 80%",
 * "The Paper"; AdapTQ page, "How it works (HAR + VQ)", steps 1-2):
 *   n   = ||x|| (fp16, correctly rounded)
 *   h   = H D x (fast Walsh-Hadamard transform, unnormalised)
 *   y_i = h_i / (sqrt(d) n)            rotated unit vector, ~N(0, 1/d)
 *   code_i = #{k : t_k < y_i}          Lloyd-Max thresholds t_k
 *
 * Work layout: 32 coordinates per lane, d/32 lanes per vector, 2048/d
 * vectors per wave pass.  A pass reads its vectors with fully coalesced
 * 128-bit loads, XORs the sign flip D into the fp16 sign bits and writes them
 * to a padded LDS stage, from which each lane reads back its own 64 bytes; the
 * next pass's loads are issued before this pass is computed.  The FWHT runs
 * five stages inside the lane's registers and the rest across the lanes of a
 * vector (DPP quad permutes, ds_swizzle for the eighth-lane stage).
 *
 * Norm: sum of exact fp32 squares (4 chains of 8, then a tree), <= 13 roundings,
 * so |S32 - S| <= 13 * 2^-24 S.  The fp16 candidate is accepted when S32 is
 * far enough from both rounding midpoints; otherwise the vector's fp16 inputs
 * are re-summed in fp64 and, if still ambiguous, exactly in 128-bit integers.
 *
 * Quantizer: u = (y + 1) * nb_half + 1 = fma(h, scale, nb_half + 1) selects one of the
 * codebook's buckets in LDS (at most one threshold per bucket), code = base +
 * (u > thr).  The comparison happens in fp32 on u; it differs from the exact
 * decision only for coordinates within ~1e-7 of a threshold.
 */
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace {

#ifndef TQ_ENC_WPE
#define TQ_ENC_WPE 3 /* registers for at least this many waves per SIMD */
#endif
constexpr int kPitch = 80;   /* LDS bytes per lane's 64-byte chunk, padded */
constexpr int kEncRep = 16;  /* copies of the bucket table (lane % 16): conflict-free 64-bit reads */

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

/* Butterfly partners: DPP quad permutes for lane xor 1 and xor 2, ds_swizzle
 * (bit mode) for lane xor 4. */
__device__ inline float xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ inline float xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
}
__device__ inline float xor4(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (4 << 10) | 0x1F));
}

__device__ inline float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ inline float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ inline float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int D>
struct Geo {
  static constexpr int LPV = D / 32;   /* lanes per vector */
  static constexpr int VPW = 64 / LPV; /* vectors per wave pass */
  static constexpr int CPR = D / 8;    /* 16-byte chunks per vector */
};

/* Per-lane XOR masks for the sign flip: every staging load of this lane
 * handles chunk (lane % CPR), coordinates 8*ch .. 8*ch+7. */
template <int D>
__device__ inline void sign_masks(const uint8_t* sign_bits, int lane, uint32_t (&m)[4]) {
  const int ch = lane % Geo<D>::CPR;
  const uint32_t b = sign_bits[ch];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    m[j] = (((b >> (2 * j)) & 1u) << 15) | (((b >> (2 * j + 1)) & 1u) << 31);
}

/* Global loads of one pass: vectors v in [vlo, vhi) at base + v * stride
 * elements; chunk c = 64 k + lane.  Vectors outside the range read as zero. */
template <int D>
__device__ inline void pass_load(const uint16_t* base, int64_t stride, int vlo, int vhi,
                                 uint4 (&g)[4], int lane) {
  using G = Geo<D>;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = 64 * k + lane;
    const int v = c / G::CPR, ch = c % G::CPR;
    g[k] = make_uint4(0u, 0u, 0u, 0u);
    if (v >= vlo && v < vhi) g[k] = *(const uint4*)(base + (int64_t)v * stride + ch * 8);
  }
}

/* Sign-flip the loaded chunks and put them in the wave's stage: lane
 * owner = v * LPV + ch / 4 receives chunk ch at (ch % 4) * 16. */
template <int D>
__device__ inline void pass_stage(const uint4 (&g)[4], const uint32_t (&sm)[4], char* stage,
                                  int lane) {
  using G = Geo<D>;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = 64 * k + lane;
    const int v = c / G::CPR, ch = c % G::CPR;
    uint4 val = g[k];
    val.x ^= sm[0];
    val.y ^= sm[1];
    val.z ^= sm[2];
    val.w ^= sm[3];
    *(uint4*)(stage + (v * G::LPV + ch / 4) * kPitch + (ch % 4) * 16) = val;
  }
}

/* fp16 value of a non-negative pattern; 0x7C00 stands for 65536 here. */
__device__ inline float half_pos(uint32_t p) {
  return p >= 0x7C00u ? 65536.0f : half_bits_to_float(p);
}

/* Accept the candidate RNE(sqrt(S)) only if S (with relative error below
 * del) lies strictly inside its rounding interval. */
__device__ inline bool norm16_check_f32(float S, uint32_t* out) {
  const float del = 4.0e-6f;
  if (S == 0.0f) { *out = 0; return true; }
  uint32_t p = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)__builtin_sqrtf(S));
  if (p > 0x7C00u) p = 0x7C00u;
  const float lo = p == 0 ? 0.0f : half_pos(p - 1), a = half_pos(p);
  const float mlo = 0.5f * (lo + a);
  bool ok = (p == 0) || (mlo * mlo < S * (1.0f - del));
  if (p < 0x7C00u) {
    const float mhi = 0.5f * (a + half_pos(p + 1));
    ok = ok && (S * (1.0f + del) < mhi * mhi);
  }
  *out = p;
  return ok;
}

__device__ inline bool norm16_check_f64(double S, uint32_t* out) {
  const double del = 1e-13;
  if (S == 0.0) { *out = 0; return true; }
  uint32_t p = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(float)__builtin_sqrt(S));
  if (p > 0x7C00u) p = 0x7C00u;
  /* walk to the interval that contains sqrt(S) (the fp32 detour can be off) */
  for (int it = 0; it < 4; ++it) {
    if (p < 0x7C00u) {
      double mhi = 0.5 * ((double)half_pos(p) + (double)half_pos(p + 1));
      if (S > mhi * mhi) { ++p; continue; }
    }
    if (p > 0) {
      double mlo = 0.5 * ((double)half_pos(p - 1) + (double)half_pos(p));
      if (S < mlo * mlo) { --p; continue; }
    }
    break;
  }
  bool ok = true;
  if (p > 0) {
    double mlo = 0.5 * ((double)half_pos(p - 1) + (double)half_pos(p));
    ok = mlo * mlo < S * (1.0 - del);
  }
  if (p < 0x7C00u) {
    double mhi = 0.5 * ((double)half_pos(p) + (double)half_pos(p + 1));
    ok = ok && (S * (1.0 + del) < mhi * mhi);
  }
  *out = p;
  return ok;
}

/* |x| in units of 2^-24 for a finite fp16 pattern. */
__device__ inline uint64_t half_units(uint32_t h) {
  const uint32_t e = (h >> 10) & 31u, f = h & 1023u;
  return e == 0 ? (uint64_t)f : ((uint64_t)(1024u + f) << (e - 1));
}

/* Exact RNE of the norm from 128-bit integer sums: 4 S compared with the
 * squared sums of neighbouring fp16 values (units of 2^-24). */
__device__ inline uint32_t norm16_exact(unsigned __int128 S, uint32_t p) {
  const unsigned __int128 S4 = S * 4u;
  for (int it = 0; it < 64; ++it) {
    const unsigned __int128 a = p >= 0x7C00u ? ((unsigned __int128)65536u << 24) : half_units(p);
    if (p < 0x7C00u) {
      const unsigned __int128 b = p + 1 >= 0x7C00u ? ((unsigned __int128)65536u << 24)
                                                   : half_units(p + 1);
      const unsigned __int128 m = (a + b) * (a + b);
      if (S4 > m || (S4 == m && (p & 1u))) { ++p; continue; }
    }
    if (p > 0) {
      const unsigned __int128 b = half_units(p - 1);
      const unsigned __int128 m = (a + b) * (a + b);
      if (S4 < m || (S4 == m && (p & 1u))) { --p; continue; }
    }
    break;
  }
  return p;
}

/* Exact fp16 norm of vector v of the pass from the LDS stage, by 128-bit
 * integer sums; reached only when even the fp64 sum sits within 1e-13 of a
 * rounding midpoint (exact ties).  Kept out of line: it needs registers the
 * hot path should not reserve.  Signs were flipped during staging; squares
 * do not care. */
template <int D>
__device__ __attribute__((noinline)) uint32_t norm16_exact_stage(const char* stage, int v,
                                                                 uint32_t guess) {
  using G = Geo<D>;
  unsigned __int128 E = 0;
  for (int p = 0; p < G::LPV; ++p)
    for (int j = 0; j < 16; ++j) {
      const uint32_t w = *(const uint32_t*)(stage + (v * G::LPV + p) * kPitch + 4 * j);
      const unsigned __int128 a = half_units(w & 0x7FFFu), b = half_units((w >> 16) & 0x7FFFu);
      E += a * a + b * b;
    }
  return norm16_exact(E, guess);
}

/* fp64 re-sum of vector v from the stage (rare), then the exact fallback. */
template <int D>
__device__ inline uint32_t norm16_slow(const char* stage, int v) {
  using G = Geo<D>;
  double S = 0.0;
#pragma unroll 1
  for (int k = 0; k < 16 * G::LPV; ++k) {
    const uint32_t w = *(const uint32_t*)(stage + (v * G::LPV + k / 16) * kPitch + 4 * (k % 16));
    const double a = (double)half_lo(w), b = (double)half_hi(w);
    S = __builtin_fma(a, a, S);
    S = __builtin_fma(b, b, S);
  }
  uint32_t n16;
  if (norm16_check_f64(S, &n16)) return n16;
  return norm16_exact_stage<D>(stage, v, n16);
}

/* a + b and a - b of the two fp16 halves of w, in fp32 (one mixed-precision
 * FMA each: a * 1 + (+-b)). */
__device__ inline void half_pair_sum_diff(uint32_t w, float* sum, float* diff) {
  float s, d;
  asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(s) : "v"(w));
  asm("v_fma_mix_f32 %0, %1, 1.0, -%1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(d) : "v"(w));
  *sum = s;
  *diff = d;
}

/* Encode the lane's 32 coordinates of its vector (data in the LDS stage).
 * Returns the packed codes (BITS words) and the vector's fp16 norm, the same
 * on all lanes of the vector.
 *
 * Cross-lane butterflies: each lane computes own + c * partner with
 * c = -1 on the lane whose index bit is set, one DPP-fused FMA per value; the
 * upper lane then holds the negated a - b, so lane values carry the sign
 * (-1)^popcount(lane bits), folded into the quantizer scale. */
template <int D, int BITS>
__device__ inline void encode_lane(const char* stage, const tq_enc_entry* table, float nbh,
                                   int lane, uint32_t (&packed)[BITS], uint32_t* n16_out,
                                   bool* sure_out) {
  using G = Geo<D>;
  uint32_t w[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 t = *(const uint4*)(stage + lane * kPitch + 16 * j);
    w[4 * j] = t.x;
    w[4 * j + 1] = t.y;
    w[4 * j + 2] = t.z;
    w[4 * j + 3] = t.w;
  }
  float v[32];
  float sq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    half_pair_sum_diff(w[j], &v[2 * j], &v[2 * j + 1]);
    const float a = half_lo(w[j]), b = half_hi(w[j]);
    sq[j & 3] = __builtin_fmaf(a, a, sq[j & 3]);
    sq[j & 3] = __builtin_fmaf(b, b, sq[j & 3]);
  }
#pragma unroll
  for (int h = 2; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!(i & h)) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  float S = (sq[0] + sq[1]) + (sq[2] + sq[3]);
  float sigma = 1.0f;
  if constexpr (G::LPV >= 2) {
    const float c = (lane & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(xor1(v[i]), c, v[i]);
    S += xor1(S);
    sigma *= c;
  }
  if constexpr (G::LPV >= 4) {
    const float c = (lane & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(xor2(v[i]), c, v[i]);
    S += xor2(S);
    sigma *= c;
  }
  if constexpr (G::LPV >= 8) {
    const float c = (lane & 4) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(xor4(v[i]), c, v[i]);
    S += xor4(S);
    sigma *= c;
  }
  uint32_t n16;
  const bool sure = norm16_check_f32(S, &n16);

  /* u = (y + 1) * nbh + 1 with y = h / (sqrt(d) * ||x||); bucket floor(u) */
  const float scale = S > 0.0f ? sigma * nbh * __builtin_amdgcn_rsqf(S * (float)D) : 0.0f;
  const float off = nbh + 1.0f;
  const char* tab = (const char*)table + (lane & (kEncRep - 1)) * sizeof(tq_enc_entry);
#pragma unroll
  for (int k = 0; k < BITS; ++k) packed[k] = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    /* bound how far the scheduler hoists table reads (registers) */
    if (i % 8 == 0) __builtin_amdgcn_sched_barrier(0);
    const float u = __builtin_fmaf(v[i], scale, off);
    const uint32_t b = (uint32_t)u;
    const tq_enc_entry e = *(const tq_enc_entry*)(tab + b * (kEncRep * sizeof(tq_enc_entry)));
    const uint32_t code = e.base + (u > e.thr ? 1u : 0u);
    const int bit = BITS * i;
    packed[bit / 32] |= code << (bit % 32);
    if ((bit % 32) + BITS > 32) packed[bit / 32 + 1] |= code >> (32 - bit % 32);
  }
  *n16_out = n16;
  *sure_out = sure;
}

/* The vector's fp16 norm once its codes are stored (the codes do not depend
 * on it): the rare undecided candidates are settled here, where the
 * coordinates are no longer live. */
template <int D>
__device__ inline uint32_t settle_norm(const char* stage, int lane, uint32_t n16, bool sure) {
  return sure ? n16 : norm16_slow<D>(stage, lane / Geo<D>::LPV);
}

/* Copy the bucket table into LDS, kEncRep interleaved copies. */
__device__ inline void load_table(tq_enc_entry* dst, const tq_enc_entry* src, int entries) {
  for (int i = threadIdx.x; i < entries * kEncRep; i += blockDim.x) dst[i] = src[i / kEncRep];
}

/* Store a lane's 4*BITS bytes of codes at dst (4-byte aligned; 8 for BITS 2,
 * 16 for BITS 4). */
template <int BITS>
__device__ inline void store_packed(uint8_t* dst, const uint32_t (&p)[BITS]) {
  if constexpr (BITS == 4) {
    *(uint4*)dst = make_uint4(p[0], p[1], p[2], p[3]);
  } else if constexpr (BITS == 2) {
    *(uint2*)dst = make_uint2(p[0], p[1]);
  } else {
    uint32_t* d = (uint32_t*)dst;
    d[0] = p[0];
    d[1] = p[1];
    d[2] = p[2];
  }
}

__host__ __device__ inline int table_bytes(int entries) {
  return (entries * kEncRep * (int)sizeof(tq_enc_entry) + 15) & ~15;
}

constexpr int kRowsWaves = 4;

/* tq_encode: n vectors, row layout.  Each wave takes passes grid-stride and
 * loads the next pass while it encodes the current one. */
template <int D, int BITS>
__global__ void __launch_bounds__(64 * kRowsWaves) __attribute__((amdgpu_waves_per_eu(TQ_ENC_WPE)))
encode_rows_kernel(const uint16_t* __restrict__ x, int64_t n, int64_t stride,
                   const uint8_t* __restrict__ sign_bits, const tq_enc_entry* __restrict__ table,
                   int entries, float nbh, uint8_t* __restrict__ codes,
                   uint16_t* __restrict__ norms) {
  using G = Geo<D>;
  extern __shared__ __align__(16) char smem[];
  tq_enc_entry* tab = (tq_enc_entry*)smem;
  const int lane = threadIdx.x % 64;
  char* stage = smem + table_bytes(entries) + (threadIdx.x / 64) * 64 * kPitch;
  load_table(tab, table, entries);
  __syncthreads();
  uint32_t sm[4];
  sign_masks<D>(sign_bits, lane, sm);
  const int64_t passes = (n + G::VPW - 1) / G::VPW;
  const int64_t wstride = (int64_t)gridDim.x * kRowsWaves;
  int64_t ps = (int64_t)blockIdx.x * kRowsWaves + threadIdx.x / 64;
  uint4 g[4];
  if (ps < passes) {
    const int64_t r0 = ps * G::VPW;
    pass_load<D>(x + r0 * stride, stride, 0, (int)(n - r0 < G::VPW ? n - r0 : G::VPW), g, lane);
  }
  for (; ps < passes; ps += wstride) {
    const int64_t row0 = ps * G::VPW;
    const int nv = (int)(n - row0 < G::VPW ? n - row0 : G::VPW);
    pass_stage<D>(g, sm, stage, lane);
    wave_lds_sync();
    const int64_t nx = ps + wstride;
    if (nx < passes) {
      const int64_t r1 = nx * G::VPW;
      pass_load<D>(x + r1 * stride, stride, 0, (int)(n - r1 < G::VPW ? n - r1 : G::VPW), g, lane);
    }
    uint32_t packed[BITS], n16;
    bool sure;
    encode_lane<D, BITS>(stage, tab, nbh, lane, packed, &n16, &sure);
    const int v = lane / G::LPV, part = lane % G::LPV;
    if (v < nv) store_packed<BITS>(codes + (row0 + v) * (D * BITS / 8) + part * (4 * BITS), packed);
    n16 = settle_norm<D>(stage, lane, n16, sure);
    if (v < nv && part == 0) norms[row0 + v] = (uint16_t)n16;
    wave_lds_sync(); /* the next pass overwrites the stage */
  }
}

/* ------------------------------------------------------------- append -- */

__device__ inline int tile_token(int q, int u) { return u < 4 ? 4 * q + u : 16 + 4 * q + (u - 4); }

struct AppendArgs {
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint16_t* k_norms;
  uint16_t* v_norms;
  int64_t ls_kc, ls_vc, ls_kn, ls_vn; /* layer strides, bytes */
  int batch, heads, capacity, t_new, n_layers, slots;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint8_t* sign_bits;
  const int32_t* pos;
  const tq_enc_entry* tab_k;
  const tq_enc_entry* tab_v;
  int ent_k, ent_v;
  float nbh_k, nbh_v;
};

/* A 32-token tile takes WPT waves (VPW vectors each); a block of 4 waves
 * works on TPB tiles side by side. */
template <int D>
struct AppendGeo {
  static constexpr int WPT = 32 / Geo<D>::VPW < 1 ? 1 : 32 / Geo<D>::VPW;
  static constexpr int TPB = 4 / WPT;
};
constexpr int kAppendWaves = 4;

/* Rows of tile `tile` receiving tokens of this append, [jlo, jhi). */
__device__ inline bool tile_range(const AppendArgs& a, int p0, int tile, int* jlo, int* jhi) {
  int lo = p0 - 32 * tile, hi = p0 + a.t_new - 32 * tile;
  if (lo < 0) lo = 0;
  if (hi > 32) hi = 32;
  if (32 * tile + hi > a.capacity) hi = a.capacity - 32 * tile;
  *jlo = lo;
  *jhi = hi;
  return hi > lo;
}

/* Task t of a role: (layer, seq, head, slot) with slot the tile offset from
 * the first tile touched by the append. */
__device__ inline void task_coords(const AppendArgs& a, int64_t task, int* layer, int* b, int* h,
                                   int* slot) {
  *slot = (int)(task % a.slots);
  int64_t r = task / a.slots;
  *h = (int)(r % a.heads);
  r /= a.heads;
  *b = (int)(r % a.batch);
  *layer = (int)(r / a.batch);
}

/* blockIdx.y = 0: keys (rows); 1: values (tiles).  Every wave loops over its
 * tasks grid-stride, loading the next task's vectors while encoding. */
template <int D, int BK, int BV>
__global__ void __launch_bounds__(64 * kAppendWaves) __attribute__((amdgpu_waves_per_eu(TQ_ENC_WPE)))
append_kernel(AppendArgs a) {
  using G = Geo<D>;
  using AG = AppendGeo<D>;
  extern __shared__ __align__(16) char smem[];
  const bool is_v = blockIdx.y == 1;
  const int ent = is_v ? a.ent_v : a.ent_k;
  const int tb = table_bytes(a.ent_k > a.ent_v ? a.ent_k : a.ent_v);
  tq_enc_entry* tab = (tq_enc_entry*)smem;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int slot_in_block = wave / AG::WPT, sub = wave % AG::WPT;
  char* stage = smem + tb + wave * 64 * kPitch;
  uint8_t* vbuf = (uint8_t*)(smem + tb + kAppendWaves * 64 * kPitch) + slot_in_block * 32 * D;
  load_table(tab, is_v ? a.tab_v : a.tab_k, ent);
  __syncthreads();
  const float nbh = is_v ? a.nbh_v : a.nbh_k;
  const uint16_t* src_all = is_v ? a.v_new : a.k_new;
  const int64_t tasks = (int64_t)a.n_layers * a.batch * a.heads * a.slots;
  const int64_t step = (int64_t)gridDim.x * AG::TPB;
  const int j0 = sub * G::VPW; /* this wave's first tile row */

  /* per-task geometry of this wave, and its prefetch */
  auto setup = [&](int64_t task, int* layer, int* b, int* h, int* tile, int* jlo, int* jhi,
                   const uint16_t** src) -> bool {
    int slot;
    task_coords(a, task, layer, b, h, &slot);
    const int p0 = a.pos[*b];
    if (p0 < 0) return false;
    *tile = p0 / 32 + slot;
    if (!tile_range(a, p0, *tile, jlo, jhi)) return false;
    const int64_t stream = ((int64_t)*layer * a.batch + *b) * a.heads + *h;
    *src = src_all + (stream * a.t_new + 32 * (int64_t)*tile + j0 - p0) * D;
    return true;
  };

  int64_t task = (int64_t)blockIdx.x * AG::TPB + slot_in_block;
  uint4 g[4];
  {
    int layer, b, h, tile, jlo, jhi;
    const uint16_t* src;
    if (task < tasks && setup(task, &layer, &b, &h, &tile, &jlo, &jhi, &src))
      pass_load<D>(src, D, jlo - j0, jhi - j0, g, lane);
  }
  /* every wave runs the same number of iterations (barriers inside) */
  const int64_t iters = (tasks + step - 1) / step;
  for (int64_t it = 0; it < iters; ++it, task += step) {
    int layer = 0, b = 0, h = 0, tile = 0, jlo = 0, jhi = 0;
    const uint16_t* src = nullptr;
    const bool live = task < tasks && setup(task, &layer, &b, &h, &tile, &jlo, &jhi, &src);
    uint32_t n16 = 0;
    uint32_t pk[BK > BV ? BK : BV];
    if (live) {
      uint32_t sm[4];
      sign_masks<D>(a.sign_bits + (int64_t)layer * (D / 8), lane, sm);
      pass_stage<D>(g, sm, stage, lane);
      wave_lds_sync();
    }
    {
      int l2, b2, h2, t2, lo2, hi2;
      const uint16_t* s2;
      const int64_t nt = task + step;
      if (nt < tasks && setup(nt, &l2, &b2, &h2, &t2, &lo2, &hi2, &s2))
        pass_load<D>(s2, D, lo2 - j0, hi2 - j0, g, lane);
    }
    const int v = lane / G::LPV, part = lane % G::LPV;
    const int jrow = j0 + v;
    const bool mine = live && jrow >= jlo && jrow < jhi;
    const int64_t row = ((int64_t)b * a.heads + h) * a.capacity + 32 * (int64_t)tile + jrow;
    if (live && !is_v) {
      uint32_t p4[BK];
      bool sure;
      encode_lane<D, BK>(stage, tab, nbh, lane, p4, &n16, &sure);
      if (mine)
        store_packed<BK>(a.k_codes + layer * a.ls_kc + row * (D * BK / 8) + part * (4 * BK), p4);
      n16 = settle_norm<D>(stage, lane, n16, sure);
      if (mine && part == 0)
        *(uint16_t*)((uint8_t*)a.k_norms + layer * a.ls_kn + row * 2) = (uint16_t)n16;
    } else if (live) {
      uint32_t pv[BV];
      bool sure;
      encode_lane<D, BV>(stage, tab, nbh, lane, pv, &n16, &sure);
      /* unpacked codes of this lane's 32 coordinates -> vbuf[jrow][part*32 ..] */
      if (jrow < 32) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          uint32_t word = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * k + e, bit = BV * i;
            uint32_t c = pv[bit / 32] >> (bit % 32);
            if ((bit % 32) + BV > 32) c |= pv[bit / 32 + 1] << (32 - bit % 32);
            word |= (c & ((1u << BV) - 1u)) << (8 * e);
          }
          *(uint32_t*)(vbuf + jrow * D + part * 32 + 4 * k) = word;
        }
      }
      n16 = settle_norm<D>(stage, lane, n16, sure);
      if (mine && part == 0)
        *(uint16_t*)((uint8_t*)a.v_norms + layer * a.ls_vn + row * 2) = (uint16_t)n16;
    }
    (void)pk;
    if (is_v) {
      __syncthreads();
      /* the first wave of each tile builds the 64 segments of its tile */
      if (live && sub == 0) {
        const int q = lane / 16, rr = lane % 16;
        constexpr int M = D / 16;
        constexpr int SW = D * BV / 64; /* segment words */
        uint32_t seg[SW], mask[SW];
#pragma unroll
        for (int k = 0; k < SW; ++k) {
          seg[k] = 0u;
          mask[k] = 0u;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int tj = tile_token(q, u);
          const bool valid = tj >= jlo && tj < jhi;
          uint8_t cb[M];
#pragma unroll
          for (int m = 0; m < M; ++m) cb[m] = vbuf[tj * D + rr * M + m];
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const int bit = (8 * m + u) * BV;
            const uint32_t c = valid ? cb[m] : 0u;
            const uint32_t f = valid ? ((1u << BV) - 1u) : 0u;
            seg[bit / 32] |= c << (bit % 32);
            mask[bit / 32] |= f << (bit % 32);
            if ((bit % 32) + BV > 32) {
              seg[bit / 32 + 1] |= c >> (32 - bit % 32);
              mask[bit / 32 + 1] |= f >> (32 - bit % 32);
            }
          }
        }
        const int64_t tile_base = (((int64_t)b * a.heads + h) * (a.capacity / 32) + tile) *
                                  (32 * D * BV / 8);
        uint32_t* dst = (uint32_t*)(a.v_codes + layer * a.ls_vc + tile_base +
                                    (int64_t)lane * (D * BV / 16));
        const bool full = (jlo == 0 && jhi == 32);
#pragma unroll
        for (int k = 0; k < SW; ++k) {
          uint32_t val = seg[k];
          if (!full) val = (dst[k] & ~mask[k]) | (seg[k] & mask[k]);
          dst[k] = val;
        }
      }
      __syncthreads(); /* vbuf is reused by the next task */
    } else {
      wave_lds_sync(); /* the stage is reused by the next task */
    }
  }
}

template <int D, int BITS>
tq_status launch_rows_t(const tq_codebook_s* cb, const uint16_t* x, int64_t n, int64_t stride,
                        const uint8_t* sb, uint8_t* codes, uint16_t* norms, hipStream_t s) {
  using G = Geo<D>;
  const int64_t passes = (n + G::VPW - 1) / G::VPW;
  int64_t blocks = (passes + kRowsWaves - 1) / kRowsWaves;
  if (blocks > 4096) blocks = 4096;
  const size_t lds = table_bytes(cb->enc_entries) + (size_t)kRowsWaves * 64 * kPitch;
  hipLaunchKernelGGL((encode_rows_kernel<D, BITS>), dim3((unsigned)blocks), dim3(64 * kRowsWaves),
                     lds, s, x, n, stride, sb, cb->enc_table, cb->enc_entries,
                     (float)cb->nb_half, codes, norms);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

template <int D, int BK, int BV>
tq_status launch_append_t(const AppendArgs& a, hipStream_t s) {
  using AG = AppendGeo<D>;
  const int64_t tasks = (int64_t)a.n_layers * a.batch * a.heads * a.slots;
  int64_t blocks = (tasks + AG::TPB - 1) / AG::TPB;
  if (blocks > 2048) blocks = 2048;
  const size_t lds = table_bytes(a.ent_k > a.ent_v ? a.ent_k : a.ent_v) +
                     (size_t)kAppendWaves * 64 * kPitch + (size_t)AG::TPB * 32 * D;
  hipLaunchKernelGGL((append_kernel<D, BK, BV>), dim3((unsigned)blocks, 2), dim3(64 * kAppendWaves),
                     lds, s, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

}  // namespace

tq_status tq_launch_encode_rows(const tq_codebook_s* cb, const uint16_t* x, int64_t n,
                                int64_t x_stride, const uint8_t* sign_bits, uint8_t* codes,
                                uint16_t* norms, hipStream_t s) {
#define TQ_ROWS(DD, BB) \
  if (cb->d == DD && cb->bits == BB) \
    return launch_rows_t<DD, BB>(cb, x, n, x_stride, sign_bits, codes, norms, s);
  TQ_ROWS(64, 2) TQ_ROWS(64, 3) TQ_ROWS(64, 4)
  TQ_ROWS(128, 2) TQ_ROWS(128, 3) TQ_ROWS(128, 4)
  TQ_ROWS(256, 2) TQ_ROWS(256, 3) TQ_ROWS(256, 4)
#undef TQ_ROWS
  return TQ_ERR_UNSUPPORTED;
}

tq_status tq_launch_append(const tq_kv_cache* c, const tq_codebook_s* cbk,
                           const tq_codebook_s* cbv, const uint8_t* sign_bits,
                           const uint16_t* k_new, const uint16_t* v_new, int t_new,
                           const int32_t* pos, int n_layers, hipStream_t s) {
  AppendArgs a;
  a.k_codes = c->k_codes;
  a.v_codes = c->v_codes;
  a.k_norms = c->k_norms;
  a.v_norms = c->v_norms;
  a.ls_kc = c->layer_stride_k_codes;
  a.ls_vc = c->layer_stride_v_codes;
  a.ls_kn = c->layer_stride_k_norms;
  a.ls_vn = c->layer_stride_v_norms;
  a.batch = c->batch;
  a.heads = c->kv_heads;
  a.capacity = c->capacity;
  a.t_new = t_new;
  a.n_layers = n_layers;
  a.slots = (t_new + 31) / 32 + 1;
  a.k_new = k_new;
  a.v_new = v_new;
  a.sign_bits = sign_bits;
  a.pos = pos;
  a.tab_k = cbk->enc_table;
  a.tab_v = cbv->enc_table;
  a.ent_k = cbk->enc_entries;
  a.ent_v = cbv->enc_entries;
  a.nbh_k = (float)cbk->nb_half;
  a.nbh_v = (float)cbv->nb_half;
#define TQ_APP(DD, KK, VV) \
  if (c->head_dim == DD && c->bits_k == KK && c->bits_v == VV) return launch_append_t<DD, KK, VV>(a, s);
#define TQ_APP_D(DD) \
  TQ_APP(DD, 2, 2) TQ_APP(DD, 2, 3) TQ_APP(DD, 2, 4) TQ_APP(DD, 3, 2) TQ_APP(DD, 3, 3) \
  TQ_APP(DD, 3, 4) TQ_APP(DD, 4, 2) TQ_APP(DD, 4, 3) TQ_APP(DD, 4, 4)
  TQ_APP_D(64) TQ_APP_D(128) TQ_APP_D(256)
#undef TQ_APP_D
#undef TQ_APP
  return TQ_ERR_UNSUPPORTED;
}
