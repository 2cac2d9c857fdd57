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
 * Work layout: 64 coordinates per lane, d/64 lanes per vector, 64/(d/64)
 * vectors per wave pass.  A pass reads its vectors with fully coalesced
 * 128-bit loads into a padded LDS stage, then each lane reads back its own
 * 128 bytes.  The sign flip D is an XOR on the fp16 sign bits during staging.
 * The FWHT runs its first six stages inside the lane's registers and the rest
 * across the lanes of a vector with DPP quad permutes.
 *
 * Norm: sum of exact fp32 squares (8 chains of 8, then a tree), ~13 roundings,
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

constexpr int kStagePitch = 144; /* LDS bytes per lane's 128-byte chunk, padded */
constexpr int kEncRep = 4;       /* copies of the bucket table (lane % kEncRep) */

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

/* DPP quad permutes: xor 1 = [1,0,3,2], xor 2 = [2,3,0,1]. */
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;
constexpr int kQuadXor2 = 0x4E;

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
  static constexpr int LPV = D / 64;       /* lanes per vector */
  static constexpr int VPW = 64 / LPV;     /* vectors per wave pass */
  static constexpr int CPR = D / 8;        /* 16-byte chunks per vector */
};

/* Per-lane XOR masks for the sign flip: every staging load of this lane
 * handles chunk (lane % CPR), coordinates 8*ch .. 8*ch+7. */
template <int D>
__device__ inline void sign_masks(const uint8_t* sign_bits, int lane, uint32_t (&m)[4]) {
  const int ch = lane % Geo<D>::CPR;
  uint32_t b = sign_bits[ch];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    m[j] = (((b >> (2 * j)) & 1u) << 15) | (((b >> (2 * j + 1)) & 1u) << 31);
}

/* Coalesced load of vectors v in [vlo, vhi) of a pass (vector v at
 * base + v * stride elements) into the wave's LDS stage, sign-flipped.
 * Vectors outside the range are staged as zeros. */
template <int D>
__device__ inline void stage_pass(const uint16_t* base, int64_t stride, int vlo, int vhi,
                                  const uint32_t (&sm)[4], char* stage, int lane) {
  using G = Geo<D>;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = 64 * k + lane;
    const int v = c / G::CPR, ch = c % G::CPR;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (v >= vlo && v < vhi) val = *(const uint4*)(base + (int64_t)v * stride + ch * 8);
    val.x ^= sm[0];
    val.y ^= sm[1];
    val.z ^= sm[2];
    val.w ^= sm[3];
    const int owner = v * G::LPV + ch / 8;
    *(uint4*)(stage + owner * kStagePitch + (ch % 8) * 16) = val;
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

/* Slow norm of vector v of the pass from the LDS stage (every lane of the
 * vector reads all of it).  Signs were flipped during staging; squares do not
 * care. */
template <int D>
__device__ __attribute__((noinline)) uint32_t norm16_slow(const char* stage, int v) {
  using G = Geo<D>;
  double S = 0.0;
  for (int p = 0; p < G::LPV; ++p)
    for (int j = 0; j < 32; ++j) {
      uint32_t w = *(const uint32_t*)(stage + (v * G::LPV + p) * kStagePitch + 4 * j);
      double a = (double)half_lo(w), b = (double)half_hi(w);
      S += a * a;
      S += b * b;
    }
  uint32_t n16;
  if (norm16_check_f64(S, &n16)) return n16;
  unsigned __int128 E = 0;
  for (int p = 0; p < G::LPV; ++p)
    for (int j = 0; j < 32; ++j) {
      uint32_t w = *(const uint32_t*)(stage + (v * G::LPV + p) * kStagePitch + 4 * j);
      unsigned __int128 a = half_units(w & 0x7FFFu), b = half_units((w >> 16) & 0x7FFFu);
      E += a * a + b * b;
    }
  return norm16_exact(E, n16);
}

/* Encode the lane's 64 coordinates of one vector of a pass whose data sits
 * in the LDS stage.  Returns the packed codes (64*BITS/32 words) and the
 * vector's fp16 norm (the same on all lanes of the vector). */
template <int D, int BITS>
__device__ inline void encode_lane(const char* stage, const tq_enc_entry* table, float nbh,
                                   int lane, uint32_t (&packed)[2 * BITS], uint32_t* n16_out) {
  using G = Geo<D>;
  uint32_t w[32];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint4 t = *(const uint4*)(stage + lane * kStagePitch + 16 * j);
    w[4 * j] = t.x;
    w[4 * j + 1] = t.y;
    w[4 * j + 2] = t.z;
    w[4 * j + 3] = t.w;
  }
  float v[64];
  float sq[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) sq[k] = 0.0f;
  /* first butterfly stage straight from fp16; squares from the same values */
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float a = half_lo(w[j]), b = half_hi(w[j]);
    v[2 * j] = a + b;
    v[2 * j + 1] = a - b;
    sq[j & 7] = __builtin_fmaf(a, a, sq[j & 7]);
    sq[j & 7] = __builtin_fmaf(b, b, sq[j & 7]);
  }
#pragma unroll
  for (int h = 2; h < 64; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (!(i & h)) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  float S = ((sq[0] + sq[1]) + (sq[2] + sq[3])) + ((sq[4] + sq[5]) + (sq[6] + sq[7]));
  if constexpr (G::LPV >= 2) {
    const float sg = (lane & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = __builtin_fmaf(sg, v[i], dpp_f<kQuadXor1>(v[i]));
    S += dpp_f<kQuadXor1>(S);
  }
  if constexpr (G::LPV >= 4) {
    const float sg = (lane & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = __builtin_fmaf(sg, v[i], dpp_f<kQuadXor2>(v[i]));
    S += dpp_f<kQuadXor2>(S);
  }
  uint32_t n16;
  if (!norm16_check_f32(S, &n16)) n16 = norm16_slow<D>(stage, lane / G::LPV);
  *n16_out = n16;

  /* u = (y + 1) * nbh with y = h / (sqrt(d) * ||x||) */
  const float scale = S > 0.0f ? nbh * __builtin_amdgcn_rsqf(S * (float)D) : 0.0f;
  const float off = nbh + 1.0f; /* bucket 0 stays unused, so u > 0 */
  const tq_enc_entry* tab = table + (lane % kEncRep);
#pragma unroll
  for (int k = 0; k < 2 * BITS; ++k) packed[k] = 0u;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const float u = __builtin_fmaf(v[i], scale, off);
    const uint32_t b = (uint32_t)u;
    const tq_enc_entry e = tab[b * kEncRep];
    const uint32_t code = e.base + (u > e.thr ? 1u : 0u);
    const int bit = BITS * i;
    packed[bit / 32] |= code << (bit % 32);
    if ((bit % 32) + BITS > 32) packed[bit / 32 + 1] |= code >> (32 - bit % 32);
  }
}

/* Copy the bucket table into LDS, kEncRep interleaved copies. */
__device__ inline void load_table(tq_enc_entry* dst, const tq_enc_entry* src, int entries) {
  for (int i = threadIdx.x; i < entries * kEncRep; i += blockDim.x) dst[i] = src[i / kEncRep];
}

/* Store a lane's packed codes at byte address dst (8-byte aligned). */
template <int BITS>
__device__ inline void store_packed(uint8_t* dst, const uint32_t (&p)[2 * BITS]) {
  if constexpr (BITS == 4) {
    *(uint4*)dst = make_uint4(p[0], p[1], p[2], p[3]);
    *(uint4*)(dst + 16) = make_uint4(p[4], p[5], p[6], p[7]);
  } else if constexpr (BITS == 2) {
    *(uint4*)dst = make_uint4(p[0], p[1], p[2], p[3]);
  } else {
    *(uint2*)dst = make_uint2(p[0], p[1]);
    *(uint2*)(dst + 8) = make_uint2(p[2], p[3]);
    *(uint2*)(dst + 16) = make_uint2(p[4], p[5]);
  }
}

constexpr int kRowsWaves = 4;

/* tq_encode: n vectors, row layout.  Waves take passes grid-stride. */
template <int D, int BITS>
__global__ void __launch_bounds__(64 * kRowsWaves)
encode_rows_kernel(const uint16_t* __restrict__ x, int64_t n, int64_t stride,
                   const uint8_t* __restrict__ sign_bits, const tq_enc_entry* __restrict__ table,
                   int entries, float nbh, uint8_t* __restrict__ codes,
                   uint16_t* __restrict__ norms) {
  using G = Geo<D>;
  extern __shared__ __align__(16) char smem[];
  tq_enc_entry* tab = (tq_enc_entry*)smem;
  char* stage = smem + ((entries * kEncRep * (int)sizeof(tq_enc_entry) + 15) & ~15) +
                (threadIdx.x / 64) * 64 * kStagePitch;
  load_table(tab, table, entries);
  __syncthreads();
  const int lane = threadIdx.x % 64;
  uint32_t sm[4];
  sign_masks<D>(sign_bits, lane, sm);
  const int64_t passes = (n + G::VPW - 1) / G::VPW;
  const int64_t wave0 = (int64_t)blockIdx.x * kRowsWaves + threadIdx.x / 64;
  const int64_t wstride = (int64_t)gridDim.x * kRowsWaves;
  const int rowbytes = D * BITS / 8;
  for (int64_t ps = wave0; ps < passes; ps += wstride) {
    const int64_t row0 = ps * G::VPW;
    const int nv = (int)(n - row0 < G::VPW ? n - row0 : G::VPW);
    stage_pass<D>(x + row0 * stride, stride, 0, nv, sm, stage, lane);
    wave_lds_sync();
    uint32_t packed[2 * BITS], n16;
    encode_lane<D, BITS>(stage, tab, nbh, lane, packed, &n16);
    const int v = lane / G::LPV, part = lane % G::LPV;
    if (v < nv) {
      store_packed<BITS>(codes + (row0 + v) * rowbytes + part * (8 * BITS), packed);
      if (part == 0) norms[row0 + v] = (uint16_t)n16;
    }
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

template <int D>
struct AppendGeo {
  static constexpr int WPK = D >= 256 ? 2 : 1;  /* waves per kind for a 32-token tile */
  static constexpr int WAVES = 2 * WPK;
};

/* One task = one 32-token tile of one (layer, seq, kv head) stream: keys go
 * to rows, values are assembled into the tile layout in LDS and merged with
 * the tile's existing bits when the append covers it only partly. */
template <int D, int BK, int BV>
__global__ void __launch_bounds__(64 * AppendGeo<D>::WAVES)
append_kernel(AppendArgs a) {
  using G = Geo<D>;
  using AG = AppendGeo<D>;
  extern __shared__ __align__(16) char smem[];
  const int tk_bytes = (a.ent_k * kEncRep * (int)sizeof(tq_enc_entry) + 15) & ~15;
  const int tv_bytes = (a.ent_v * kEncRep * (int)sizeof(tq_enc_entry) + 15) & ~15;
  tq_enc_entry* tab_k = (tq_enc_entry*)smem;
  tq_enc_entry* tab_v = (tq_enc_entry*)(smem + tk_bytes);
  uint8_t* vbuf = (uint8_t*)(smem + tk_bytes + tv_bytes);  /* [32][D] value codes */
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  char* stage = smem + tk_bytes + tv_bytes + 32 * D + wave * 64 * kStagePitch;
  load_table(tab_k, a.tab_k, a.ent_k);
  load_table(tab_v, a.tab_v, a.ent_v);
  __syncthreads();

  const int kind = wave / AG::WPK, sub = wave % AG::WPK;
  const int64_t tasks = (int64_t)a.n_layers * a.batch * a.heads * a.slots;
  const int64_t seg_bytes = D * BV / 16;
  for (int64_t task = blockIdx.x; task < tasks; task += gridDim.x) {
    const int slot = (int)(task % a.slots);
    int64_t r = task / a.slots;
    const int h = (int)(r % a.heads);
    r /= a.heads;
    const int b = (int)(r % a.batch);
    const int layer = (int)(r / a.batch);
    const int p0 = a.pos[b];
    if (p0 < 0) continue; /* uniform over the block */
    const int tile = p0 / 32 + slot;
    /* rows 32*tile + j, j in [jlo, jhi), receive tokens 32*tile + j - p0 */
    int jlo = p0 - 32 * tile, jhi = p0 + a.t_new - 32 * tile;
    if (jlo < 0) jlo = 0;
    if (jhi > 32) jhi = 32;
    if (32 * tile + jhi > a.capacity) jhi = a.capacity - 32 * tile;
    if (jhi <= jlo) continue; /* uniform over the block */

    const uint8_t* sb = a.sign_bits + (int64_t)layer * (D / 8);
    uint32_t sm[4];
    sign_masks<D>(sb, lane, sm);
    const int64_t stream = ((int64_t)layer * a.batch + b) * a.heads + h;
    const uint16_t* src = (kind == 0 ? a.k_new : a.v_new) + stream * a.t_new * D;
    /* this wave's vectors: tile rows j = sub * VPW + v */
    const int j0 = sub * G::VPW;
    const int64_t tok0 = 32 * (int64_t)tile + j0 - p0; /* source token of v = 0 */
    const int vlo = jlo - j0, vhi = jhi - j0;
    const bool active = (vhi > 0) && (vlo < G::VPW) && (j0 < 32);
    if (active) {
      stage_pass<D>(src + tok0 * D, D, vlo, vhi, sm, stage, lane);
      wave_lds_sync();
      uint32_t n16;
      const int v = lane / G::LPV, part = lane % G::LPV;
      const int jrow = j0 + v;
      const bool mine = v >= vlo && v < vhi && jrow < 32;
      const int64_t row = ((int64_t)b * a.heads + h) * a.capacity + 32 * (int64_t)tile + jrow;
      if (kind == 0) {
        uint32_t pk[2 * BK];
        encode_lane<D, BK>(stage, tab_k, a.nbh_k, lane, pk, &n16);
        if (mine) {
          store_packed<BK>(a.k_codes + layer * a.ls_kc + row * (D * BK / 8) + part * (8 * BK), pk);
          if (part == 0)
            *(uint16_t*)((uint8_t*)a.k_norms + layer * a.ls_kn + row * 2) = (uint16_t)n16;
        }
      } else {
        uint32_t pv[2 * BV];
        encode_lane<D, BV>(stage, tab_v, a.nbh_v, lane, pv, &n16);
        if (mine && part == 0)
          *(uint16_t*)((uint8_t*)a.v_norms + layer * a.ls_vn + row * 2) = (uint16_t)n16;
        /* unpacked codes of this lane's 64 coordinates -> vbuf[jrow][part*64 ..] */
        if (jrow < 32) {
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * k + e, bit = BV * i;
              uint32_t c = pv[bit / 32] >> (bit % 32);
              if ((bit % 32) + BV > 32) c |= pv[bit / 32 + 1] << (32 - bit % 32);
              word |= (c & ((1u << BV) - 1u)) << (8 * e);
            }
            *(uint32_t*)(vbuf + jrow * D + part * 64 + 4 * k) = word;
          }
        }
      }
    }
    __syncthreads();
    /* value tile assembly: lane l of the first value wave builds segment l */
    if (kind == 1 && sub == 0) {
      const int q = lane / 16, rr = lane % 16;
      constexpr int M = D / 16;
      constexpr int SW = D * BV / 64; /* segment words */
      uint32_t seg[SW], mask[SW];
#pragma unroll
      for (int k = 0; k < SW; ++k) { seg[k] = 0u; mask[k] = 0u; }
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
      uint32_t* dst = (uint32_t*)(a.v_codes + layer * a.ls_vc + tile_base + lane * seg_bytes);
      const bool full = (jlo == 0 && jhi == 32);
#pragma unroll
      for (int k = 0; k < SW; ++k) {
        uint32_t val = seg[k];
        if (!full) val = (dst[k] & ~mask[k]) | (seg[k] & mask[k]);
        dst[k] = val;
      }
    }
    __syncthreads(); /* vbuf and stages are reused by the next task */
  }
}

template <int D, int BITS>
tq_status launch_rows_t(const tq_codebook_s* cb, const uint16_t* x, int64_t n, int64_t stride,
                        const uint8_t* sb, uint8_t* codes, uint16_t* norms, hipStream_t s) {
  using G = Geo<D>;
  const int64_t passes = (n + G::VPW - 1) / G::VPW;
  int64_t blocks = (passes + kRowsWaves - 1) / kRowsWaves;
  if (blocks > 2048) blocks = 2048;
  const size_t lds = ((cb->enc_entries * kEncRep * sizeof(tq_enc_entry) + 15) & ~(size_t)15) +
                     (size_t)kRowsWaves * 64 * kStagePitch;
  hipLaunchKernelGGL((encode_rows_kernel<D, BITS>), dim3((unsigned)blocks), dim3(64 * kRowsWaves),
                     lds, s, x, n, stride, sb, cb->enc_table, cb->enc_entries,
                     (float)cb->nb_half, codes, norms);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

template <int D, int BK, int BV>
tq_status launch_append_t(const AppendArgs& a, hipStream_t s) {
  using AG = AppendGeo<D>;
  const int64_t tasks = (int64_t)a.n_layers * a.batch * a.heads * a.slots;
  int64_t blocks = tasks < 4096 ? tasks : 4096;
  const size_t lds = ((a.ent_k * kEncRep * sizeof(tq_enc_entry) + 15) & ~(size_t)15) +
                     ((a.ent_v * kEncRep * sizeof(tq_enc_entry) + 15) & ~(size_t)15) +
                     32 * D + (size_t)AG::WAVES * 64 * kStagePitch;
  hipLaunchKernelGGL((append_kernel<D, BK, BV>), dim3((unsigned)blocks), dim3(64 * AG::WAVES),
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
