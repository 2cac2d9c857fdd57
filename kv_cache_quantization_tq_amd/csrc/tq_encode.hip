/*
 * gfx950 encode kernels: fp16 vector -> fp16 norm + b-bit codes.
 *
 * Per vector ("We Built a Python Library That Cuts LLM Memory Usage by 80%",
 * "The Paper"; AdapTQ page, "How it works (HAR + VQ)", steps 1-2):
 *   n   = ||x|| (fp16, correctly rounded)
 *   h   = H D x (Walsh-Hadamard transform of the sign-flipped vector,
 *         unnormalised)
 *   y_i = h_i / (sqrt(d) n)            rotated unit vector, ~N(0, 1/d)
 *   code_i = #{k : t_k < y_i}          Lloyd-Max thresholds t_k
 *
 * Work layout.  A wave pass encodes 16 vectors.  Lane (q4, n) = (lane / 16,
 * lane % 16) holds coordinates 32 j + 8 q4 .. 32 j + 8 q4 + 7 of vector n for
 * every 32-coordinate block j (one 16-byte load per block), XORs the sign
 * flip D into their fp16 sign bits and squares them for the norm.
 *
 * The transform runs on the matrix cores (v_mfma_f32_16x16x32_f16) as the
 * product H_d X, X the pass's 16 vectors as columns.  A 16 x 32 tile of H_d
 * (output rows 16 ob .. 16 ob + 15, input columns 32 j .. 32 j + 31) is, with
 * Sylvester's H[r][c] = (-1)^popcount(r & c),
 *   (-1)^popcount((ob >> 1) & j) * T_(ob & 1),
 *   T_h[r][k] = (-1)^(popcount(r & k) + h * (k >> 4)),  r < 16, k < 32,
 * so two constant +-1 operands (and their negations) serve the whole matrix:
 * d/16 * d/32 products per pass, accumulated in fp32 from exact fp16 inputs.
 * Lane (q4, n) then holds transformed coordinates 16 ob + 4 q4 + i (i < 4) of
 * vector n.
 *
 * Norm: sum of exact fp32 squares (4 chains, then a tree and a 4-lane sum),
 * at most 2 d/32 + 3 roundings, so |S32 - S| stays below norm_del(d) S.  The
 * fp16 candidate is accepted when S32 is far enough from both rounding
 * midpoints; otherwise the inputs are re-summed in fp64 and, if still
 * ambiguous, exactly in 128-bit integers.
 *
 * Quantizer: u = (y + 1) * nb_half + 1/2 + shift = fma(h, scale, off)
 * selects, rounded to an integer, one of the codebook's buckets in LDS (at
 * most one threshold t per bucket, kept clear of the bucket edges by the
 * shift), code = base + (fma(h, scale, -t nb_half) > 0).  That fma rounds
 * once, so its sign is the exact sign of y nb_half - t nb_half for the fp32
 * h and scale: the decision differs from the exact one only through the
 * rounding of the transform sums and of the norm (~1e-8 in y), not through
 * the ~1e-7 spacing of fp32 values near u.
 *
 * Output.  Key rows: the four lanes of a vector exchange their 4-code pieces
 * with 4 x 4 word transposes (permlane swaps), after which each lane owns d/4
 * consecutive coordinates and stores them packed.  Value tiles: a wave's 16
 * tokens are one contiguous half of a tile; their code bytes go to the wave's
 * own LDS rows, from which each lane packs half a segment (no block barrier).
 */
#include <hip/hip_runtime.h>

#include "tq_append_rows.h"
#include "tq_internal.h"

namespace {

#ifndef TQ_ENC_WPE
#define TQ_ENC_WPE 3 /* registers for at least this many waves per SIMD */
#endif

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kVec = 16;     /* vectors per wave pass (the matrix-core N) */
constexpr int kEncRep = 32;  /* copies of the bucket table (lane % 32): a 64-bit LDS read
                                serves 32 lanes per cycle, each on its own pair of banks */

template <int D>
struct EGeo {
  static constexpr int J = D / 32;  /* 32-coordinate input blocks */
  static constexpr int OB = D / 16; /* 16-coordinate output blocks */
  static constexpr int T = OB / 4;  /* output blocks per lane of a row chunk */
};

/* Relative error bound used by the fp32 norm test: the sum has at most
 * 2 J + 3 roundings (chains of 2 J fmas, a 2-level tree, a 4-lane sum); one
 * more for the scaled comparison, and a margin. */
template <int D>
constexpr float norm_del() { return (float)(2 * (D / 32) + 6) * 5.9604645e-8f; }

/* Sums over the four lanes n, n + 16, n + 32, n + 48 (one vector's lanes). */
__device__ inline float col_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ inline double col_sum_f64(double v) {
  uint64_t u = __builtin_bit_cast(uint64_t, v);
  uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  v = __builtin_bit_cast(double, (uint64_t)a[0] | ((uint64_t)b[0] << 32)) +
      __builtin_bit_cast(double, (uint64_t)a[1] | ((uint64_t)b[1] << 32));
  u = __builtin_bit_cast(uint64_t, v);
  lo = (uint32_t)u;
  hi = (uint32_t)(u >> 32);
  auto c = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  auto e = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  return __builtin_bit_cast(double, (uint64_t)c[0] | ((uint64_t)e[0] << 32)) +
         __builtin_bit_cast(double, (uint64_t)c[1] | ((uint64_t)e[1] << 32));
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

/* fp16 value of a non-negative pattern; 0x7C00 stands for 65536 here. */
__device__ inline float half_pos(uint32_t p) {
  return p >= 0x7C00u ? 65536.0f : half_bits_to_float(p);
}

/* Accept the candidate RNE(sqrt(S)) only if S (with relative error below
 * del) lies strictly inside its rounding interval.  Midpoints of fp16
 * neighbours have at most 12 significant bits, so their squares are exact. */
__device__ inline bool norm16_check_f32(float S, float del, uint32_t* out) {
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

/* Exact fp16 norm of the D fp16 values at vec (global memory), by 128-bit
 * integer sums; reached only when even the fp64 sum sits within 1e-13 of a
 * rounding midpoint (exact ties).  Kept out of line. */
template <int D>
__device__ __attribute__((noinline)) uint32_t norm16_exact_global(const uint16_t* vec,
                                                                  uint32_t guess) {
  unsigned __int128 E = 0;
  for (int i = 0; i < D; ++i) {
    const unsigned __int128 a = half_units(vec[i] & 0x7FFFu);
    E += a * a;
  }
  return norm16_exact(E, guess);
}

/* Word w of a uint4. */
__device__ inline uint32_t u4w(const uint4& u, int w) {
  return w == 0 ? u.x : (w == 1 ? u.y : (w == 2 ? u.z : u.w));
}

/* Matrix operands T_0, T_1 of the transform and their negations, as held by
 * lane (q4, n): row n, columns 8 q4 .. 8 q4 + 7. */
struct HTiles {
  half8 p[2], m[2];
};
__device__ inline HTiles h_tiles(int n, int q4) {
  HTiles t;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int k = 8 * q4 + r;
      const int par = (__builtin_popcount(n & k & 15) + h * (k >> 4)) & 1;
      t.p[h][r] = par ? (_Float16)-1.0f : (_Float16)1.0f;
      t.m[h][r] = par ? (_Float16)1.0f : (_Float16)-1.0f;
    }
  return t;
}

/* Read-only kernel inputs read through the constant address space, so that
 * uniform reads become scalar loads (the kernel never writes them). */
template <class T>
__device__ inline T ld_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

/* Sign-flip masks of lane (q4, .): block j's coordinates 32 j + 8 q4 .. +7
 * are byte 4 j + q4 of the layer's sign bits (word j, read with a scalar
 * load; sb is 4-byte aligned); word w of the masks holds two of them. */
template <int D>
__device__ inline void sign_masks(const uint8_t* sb, int q4, uint32_t (&m)[EGeo<D>::J][4]) {
#pragma unroll
  for (int j = 0; j < EGeo<D>::J; ++j) {
    const uint32_t sw = ld_const((const uint32_t*)sb + j);
    const uint32_t b = (sw >> (8 * q4)) & 0xFFu;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      m[j][w] = (((b >> (2 * w)) & 1u) << 15) | (((b >> (2 * w + 1)) & 1u) << 31);
  }
}

/* One pass's input registers: block j's 8 fp16 values of the lane's vector. */
template <int D>
struct XRegs {
  uint4 w[EGeo<D>::J];
};

template <int D>
__device__ inline void load_x(XRegs<D>& x, const uint16_t* vec, int q4) {
#pragma unroll
  for (int j = 0; j < EGeo<D>::J; ++j) x.w[j] = *(const uint4*)(vec + 32 * j + 8 * q4);
}

/* Encode the pass held in xr.  Columns without a vector of their own hold a
 * copy of a real row (loads are clamped), which is encoded and discarded, so
 * the pass needs no masking; vec: the column's fp16 values in global memory
 * (read only by the exact-tie fallback).  piece[ob] receives the codes of
 * coordinates 16 ob + 4 q4 + i, i < 4: BITS bits each (first lowest), or one
 * byte each when BYTES.  Returns the fp16 norm (the same on the vector's four
 * lanes). */
template <int D, int BITS, bool BYTES>
__device__ inline uint32_t encode_pass(const XRegs<D>& xr,
                                       const uint32_t (&sm)[EGeo<D>::J][4], const HTiles& ht,
                                       const char* tab, uint32_t lane_off, float nbh,
                                       float off, const uint16_t* vec,
                                       uint32_t (&piece)[EGeo<D>::OB]) {
  using G = EGeo<D>;
  uint32_t x[G::J][4];
#pragma unroll
  for (int j = 0; j < G::J; ++j)
#pragma unroll
    for (int w = 0; w < 4; ++w) x[j][w] = u4w(xr.w[j], w) ^ sm[j][w];

  /* norm: exact fp32 squares, 4 chains */
  float sq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < G::J; ++j)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = half_lo(x[j][w]), b = half_hi(x[j][w]);
      sq[w] = __builtin_fmaf(a, a, sq[w]);
      sq[w] = __builtin_fmaf(b, b, sq[w]);
    }
  const float S = col_sum((sq[0] + sq[1]) + (sq[2] + sq[3]));
  uint32_t n16;
  const bool sure = norm16_check_f32(S, norm_del<D>(), &n16);
  if (__builtin_expect(__any(!sure), 0)) {
    /* rare: fp64 from the registers, then exact integers from memory */
    double s64 = 0.0;
#pragma unroll
    for (int j = 0; j < G::J; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const double a = (double)half_lo(x[j][w]), b = (double)half_hi(x[j][w]);
        s64 = __builtin_fma(a, a, s64);
        s64 = __builtin_fma(b, b, s64);
      }
    s64 = col_sum_f64(s64);
    if (!sure) {
      uint32_t p64;
      if (norm16_check_f64(s64, &p64))
        n16 = p64;
      else
        n16 = norm16_exact_global<D>(vec, p64);
    }
  }

  /* H_d X on the matrix cores, one 16-coordinate output block at a time */
  half8 b[G::J];
#pragma unroll
  for (int j = 0; j < G::J; ++j)
    b[j] = __builtin_bit_cast(half8, u32x4{x[j][0], x[j][1], x[j][2], x[j][3]});
  const float scale = S > 0.0f ? nbh * __builtin_amdgcn_rsqf(S * (float)D) : 0.0f;
  floatx4 y[G::OB];
#pragma unroll
  for (int ob = 0; ob < G::OB; ++ob) {
    y[ob] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < G::J; ++j) {
      const bool neg = __builtin_popcount((ob >> 1) & j) & 1;
      y[ob] = __builtin_amdgcn_mfma_f32_16x16x32_f16(neg ? ht.m[ob & 1] : ht.p[ob & 1], b[j],
                                                     y[ob], 0, 0, 0);
    }
  }
  /* quantize: u = (y + 1) * nb_half + 1/2 + shift; bucket r = u rounded to
   * the nearest integer.  One (saturating) conversion writes r into byte 1
   * of the lane's table offset, i.e. the address of row r, copy lane % 32.
   * The table reads of QB output blocks go out together; each code is then
   * decided by the sign of one fma against the bucket's threshold. */
  constexpr int QB = 2;
#pragma unroll
  for (int ob0 = 0; ob0 < G::OB; ob0 += QB) {
    float u[4 * QB];
    tq_enc_entry e[4 * QB];
#pragma unroll
    for (int k = 0; k < 4 * QB; ++k) u[k] = __builtin_fmaf(y[ob0 + k / 4][k % 4], scale, off);
#pragma unroll
    for (int k = 0; k < 4 * QB; ++k)
      e[k] = *(const tq_enc_entry*)(tab + __builtin_amdgcn_cvt_pk_u8_f32(u[k], 1, lane_off));
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      uint32_t pc = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float side = __builtin_fmaf(y[ob0 + q][i], scale, e[4 * q + i].neg_t);
        const uint32_t code = e[4 * q + i].base + (side > 0.0f ? 1u : 0u);
        pc |= code << (BYTES ? 8 * i : BITS * i);
      }
      piece[ob0 + q] = pc;
    }
  }
  return n16;
}

/* OR the w-bit value v into the bit string out at bit position pos. */
template <int NW>
__device__ inline void put_bits(uint32_t (&out)[NW], int pos, uint32_t v, int w) {
  out[pos / 32] |= v << (pos % 32);
  if ((pos % 32) + w > 32 && pos / 32 + 1 < NW) out[pos / 32 + 1] |= v >> (32 - pos % 32);
}

/* 4 x 4 transpose of 32-bit words over a vector's four lanes: before, lane q
 * holds r[q'] for every q'; after, lane q' holds in r[q] what lane q held in
 * r[q']. */
__device__ inline void transpose4(uint32_t (&r)[4]) {
  auto s0 = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
  auto s1 = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
  r[0] = s0[0];
  r[2] = s0[1];
  r[1] = s1[0];
  r[3] = s1[1];
  auto s2 = __builtin_amdgcn_permlane16_swap(r[0], r[1], false, false);
  auto s3 = __builtin_amdgcn_permlane16_swap(r[2], r[3], false, false);
  r[0] = s2[0];
  r[1] = s2[1];
  r[2] = s3[0];
  r[3] = s3[1];
}

/* Words of a lane's packed row chunk (d/4 coordinates of BITS bits). */
template <int D, int BITS>
struct Chunk {
  static constexpr int BYTES = D * BITS / 32;
  static constexpr int NW = (BYTES + 3) / 4;
};

/* Key-row output: afterwards lane (q4, n) holds the packed codes of
 * coordinates q4 d/4 .. (q4 + 1) d/4 - 1 of vector n (first code lowest).
 * Lane q sends lane q' its pieces of output blocks q' T .. q' T + T - 1, two
 * per word. */
template <int D, int BITS>
__device__ inline void gather_row_chunk(const uint32_t (&piece)[EGeo<D>::OB],
                                        uint32_t (&out)[Chunk<D, BITS>::NW]) {
  constexpr int T = EGeo<D>::T, PB = 4 * BITS;
  constexpr int NWT = (T + 1) / 2; /* transposed words per lane pair */
#pragma unroll
  for (int k = 0; k < Chunk<D, BITS>::NW; ++k) out[k] = 0u;
#pragma unroll
  for (int k = 0; k < NWT; ++k) {
    uint32_t r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t0 = 2 * k, t1 = 2 * k + 1;
      r[q] = piece[q * T + t0] | (t1 < T ? piece[q * T + t1] << 16 : 0u);
    }
    transpose4(r);
    /* r[q]: lane q's pieces of blocks q' T + 2k (low half), + 2k + 1 (high);
     * coordinate 16 t + 4 q + i of the chunk sits at bit BITS (16 t + 4 q + i) */
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      put_bits(out, 16 * BITS * (2 * k) + PB * q, r[q] & 0xFFFFu, PB);
      if (2 * k + 1 < T) put_bits(out, 16 * BITS * (2 * k + 1) + PB * q, r[q] >> 16, PB);
    }
  }
}

/* Store a lane's packed row chunk at dst (dst aligned to 8 bytes when the
 * chunk size is a multiple of 8, else to 2; A16: aligned to 16, and then
 * 16-byte chunks go out as single non-temporal stores, since the cache is
 * written once and read back much later). */
template <int D, int BITS, bool A16 = false>
__device__ inline void store_chunk(uint8_t* dst, const uint32_t (&p)[Chunk<D, BITS>::NW]) {
  constexpr int NB = Chunk<D, BITS>::BYTES;
  if constexpr (A16 && NB % 16 == 0) {
#pragma unroll
    for (int k = 0; k < NB / 16; ++k)
      __builtin_nontemporal_store(u32x4{p[4 * k], p[4 * k + 1], p[4 * k + 2], p[4 * k + 3]},
                                  (u32x4*)(dst + 16 * k));
  } else if constexpr (NB % 8 == 0) {
#pragma unroll
    for (int k = 0; k < NB / 8; ++k) *(uint2*)(dst + 8 * k) = make_uint2(p[2 * k], p[2 * k + 1]);
  } else if constexpr (NB % 4 == 0) {
#pragma unroll
    for (int k = 0; k < NB / 4; ++k) *(uint32_t*)(dst + 4 * k) = p[k];
  } else {
#pragma unroll
    for (int k = 0; k < NB / 2; ++k)
      *(uint16_t*)(dst + 2 * k) = (uint16_t)(p[k / 2] >> (16 * (k & 1)));
  }
}

/* Copy the bucket table into LDS, kEncRep interleaved copies. */
__device__ inline void load_table(tq_enc_entry* dst, const tq_enc_entry* src, int entries) {
  for (int i = threadIdx.x; i < entries * kEncRep; i += blockDim.x) dst[i] = src[i / kEncRep];
}

constexpr int kRowsWaves = 4;

/* tq_encode: n vectors, row layout.  Each wave takes passes grid-stride and
 * loads the next pass while it encodes the current one (loads are issued
 * on every path, clamped to real rows, so waits cover only the pass in use). */
template <int D, int BITS>
__global__ void __launch_bounds__(64 * kRowsWaves) __attribute__((amdgpu_waves_per_eu(D == 256 ? 2 : TQ_ENC_WPE)))
encode_rows_kernel(const uint16_t* __restrict__ x, int64_t n, int64_t stride,
                   const uint8_t* __restrict__ sign_bits, const tq_enc_entry* __restrict__ table,
                   int entries, float nbh, float off, uint8_t* __restrict__ codes,
                   uint16_t* __restrict__ norms) {
  using G = EGeo<D>;
  /* static LDS: the table's address is a constant, folded into the reads */
  constexpr int kRows = tq_enc_rows_max(D, BITS);
  __shared__ __align__(16) tq_enc_entry tab[kRows * kEncRep];
  const int lane = threadIdx.x % 64, q4 = lane / 16, nl = lane % 16;
  const int64_t passes = (n + kVec - 1) / kVec;
  const int64_t wstride = (int64_t)gridDim.x * kRowsWaves;
  int64_t ps = (int64_t)blockIdx.x * kRowsWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  /* this lane's row in pass p, clamped to a real row */
  auto row_of = [&](int64_t p) -> int64_t {
    const int64_t r = p * kVec + nl;
    return r < n ? r : n - 1;
  };
  /* the first pass's loads go out before the table is built */
  XRegs<D> xa, xb;
  load_x<D>(xa, x + row_of(ps < passes ? ps : passes - 1) * stride, q4);
  load_table(tab, table, entries);
  __syncthreads();
  if (ps >= passes) return;
  const uint32_t tab_off = (uint32_t)(lane & (kEncRep - 1)) * sizeof(tq_enc_entry);
  uint32_t sm[G::J][4];
  sign_masks<D>(sign_bits, q4, sm);
  const HTiles ht = h_tiles(nl, q4);
  auto body = [&](const XRegs<D>& xr, int64_t p) {
    const int64_t r = p * kVec + nl;
    const bool valid = r < n;
    uint32_t piece[G::OB];
    const uint32_t n16 = encode_pass<D, BITS, false>(xr, sm, ht, (const char*)tab, tab_off, nbh,
                                                     off, x + row_of(p) * stride, piece);
    uint32_t out[Chunk<D, BITS>::NW];
    gather_row_chunk<D, BITS>(piece, out);
    if (valid) {
      store_chunk<D, BITS>(codes + r * (D * BITS / 8) + q4 * Chunk<D, BITS>::BYTES, out);
      if (q4 == 0) norms[r] = (uint16_t)n16;
    }
  };
  for (;;) {
    const int64_t p1 = ps + wstride;
    load_x<D>(xb, x + row_of(p1 < passes ? p1 : ps) * stride, q4);
    body(xa, ps);
    ps = p1;
    if (ps >= passes) break;
    const int64_t p2 = ps + wstride;
    load_x<D>(xa, x + row_of(p2 < passes ? p2 : ps) * stride, q4);
    body(xb, ps);
    ps = p2;
    if (ps >= passes) break;
  }
}

/* ------------------------------------------------------------- append -- */

/* Row pitch of a wave's value-code buffer (16 rows, one per token; the
 * padding puts the 64 lanes' 4-byte writes of one output block on distinct
 * banks). */
template <int D>
constexpr int kVPitch = D + 16;

/* N bytes (2, 4 or 8) of LDS as words. */
template <int N>
__device__ inline void read_codes(const uint8_t* p, uint32_t (&w)[(N + 3) / 4]) {
  if constexpr (N == 2) {
    w[0] = *(const uint16_t*)p;
  } else if constexpr (N == 4) {
    w[0] = *(const uint32_t*)p;
  } else {
    const uint2 v = *(const uint2*)p;
    w[0] = v.x;
    w[1] = v.y;
  }
}

/* Build this wave's half of a value tile.  The wave's 16 tokens are tile
 * tokens 16 sub .. 16 sub + 15, i.e. segments 32 sub .. 32 sub + 31 (the
 * segment l = 16 q + r holds, for m < d/16 and u < 8, the code of coordinate
 * r d/16 + m of tile token 8 q + u at bit (8 m + u) BV).  Lane L writes half
 * L % 2 of local segment L / 2: fields m in [h d/32, (h + 1) d/32), i.e. one
 * contiguous run of d/32 code bytes from each of the segment's 8 token rows
 * of vbuf (the wave's 16 rows of code bytes, kVPitch apart).  Tokens outside
 * [lo, hi) (wave-local rows) keep the bits already in memory; dst is the
 * wave's half tile. */
template <int D, int BV>
__device__ inline void build_value_half(const uint8_t* vbuf, int lane, int lo, int hi,
                                        uint8_t* dst) {
  constexpr int MH = D / 32;               /* fields (coordinates) per lane */
  constexpr int NW = (MH + 3) / 4;         /* words per token row read */
  constexpr int OB = MH * BV;              /* output bytes per lane (8 tokens x MH x BV bits) */
  constexpr int OW = (OB + 3) / 4;
  const int s = lane >> 1, h = lane & 1, ql = s >> 4, r = s & 15;
  uint32_t x[8][NW];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    read_codes<MH>(vbuf + (8 * ql + u) * kVPitch<D> + r * (D / 16) + h * MH, x[u]);
  uint32_t out[OW];
#pragma unroll
  for (int k = 0; k < OW; ++k) out[k] = 0u;
  if constexpr (BV == 2) {
    /* bytes of A (B): tokens 0..3 (4..7) of one field, two bits each; field
     * i = 16 bits [A_i, B_i] */
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t A = (x[0][w] | (x[1][w] << 2)) | ((x[2][w] | (x[3][w] << 2)) << 4);
      const uint32_t B = (x[4][w] | (x[5][w] << 2)) | ((x[6][w] | (x[7][w] << 2)) << 4);
      out[2 * w] = __builtin_amdgcn_perm(B, A, 0x05010400u);
      if (2 * w + 1 < OW) out[2 * w + 1] = __builtin_amdgcn_perm(B, A, 0x07030602u);
    }
  } else if constexpr (BV == 4) {
    /* bytes of t_k: tokens 2k, 2k + 1 of one field; field i = 32 bits
     * [t0_i, t1_i, t2_i, t3_i] */
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      uint32_t t[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) t[k] = x[2 * k][w] | (x[2 * k + 1][w] << 4);
      const uint32_t P = __builtin_amdgcn_perm(t[1], t[0], 0x05010400u);
      const uint32_t Q = __builtin_amdgcn_perm(t[3], t[2], 0x05010400u);
      const uint32_t R = __builtin_amdgcn_perm(t[1], t[0], 0x07030602u);
      const uint32_t S = __builtin_amdgcn_perm(t[3], t[2], 0x07030602u);
      const uint32_t f[4] = {__builtin_amdgcn_perm(Q, P, 0x05040100u),
                             __builtin_amdgcn_perm(Q, P, 0x07060302u),
                             __builtin_amdgcn_perm(S, R, 0x05040100u),
                             __builtin_amdgcn_perm(S, R, 0x07060302u)};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (4 * w + k < MH) out[4 * w + k] = f[k];
    }
  } else {
    /* 3 bits: field i = 24 bits, tokens u at 3 u.  Bytes of p_k: tokens 2k,
     * 2k + 1 (6 bits); the even and odd fields of a word then go to 16-bit
     * halves, where four tokens fit (12 bits), and two halves make a field. */
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      uint32_t p[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) p[k] = x[2 * k][w] | (x[2 * k + 1][w] << 3);
      const uint32_t e01 = (p[0] & 0x00FF00FFu) | ((p[1] & 0x00FF00FFu) << 6);
      const uint32_t e23 = (p[2] & 0x00FF00FFu) | ((p[3] & 0x00FF00FFu) << 6);
      const uint32_t o01 = ((p[0] >> 8) & 0x00FF00FFu) | (((p[1] >> 8) & 0x00FF00FFu) << 6);
      const uint32_t o23 = ((p[2] >> 8) & 0x00FF00FFu) | (((p[3] >> 8) & 0x00FF00FFu) << 6);
      const uint32_t f[4] = {(e01 & 0xFFFu) | ((e23 & 0xFFFu) << 12),
                             (o01 & 0xFFFu) | ((o23 & 0xFFFu) << 12),
                             (e01 >> 16) | ((e23 >> 16) << 12),
                             (o01 >> 16) | ((o23 >> 16) << 12)};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = 4 * w + k;
        if (i < MH) {
          const int bit = 24 * i;
          out[bit / 32] |= f[k] << (bit % 32);
          if ((bit % 32) + 24 > 32) out[bit / 32 + 1] |= f[k] >> (32 - bit % 32);
        }
      }
    }
  }
  uint8_t* d = dst + lane * OB;
  const int t0 = 8 * ql; /* wave-local row of token u = 0 */
  if (lo <= t0 && t0 + 8 <= hi) {
    if constexpr (OB % 16 == 0) {
#pragma unroll
      for (int k = 0; k < OB / 16; ++k)
        __builtin_nontemporal_store(u32x4{out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]},
                                    (u32x4*)(d + 16 * k));
    } else if constexpr (OB % 8 == 0) {
#pragma unroll
      for (int k = 0; k < OB / 8; ++k)
        __builtin_nontemporal_store(u32x2{out[2 * k], out[2 * k + 1]}, (u32x2*)(d + 8 * k));
    } else if constexpr (OB % 4 == 0) {
#pragma unroll
      for (int k = 0; k < OB / 4; ++k) __builtin_nontemporal_store(out[k], (uint32_t*)(d + 4 * k));
    } else {
#pragma unroll
      for (int k = 0; k < OB / 2; ++k)
        *(uint16_t*)(d + 2 * k) = (uint16_t)(out[k / 2] >> (16 * (k & 1)));
    }
  } else {
    /* partly covered: keep the other tokens' bits (16-bit pieces; OB is even) */
    uint32_t mask[OW];
#pragma unroll
    for (int k = 0; k < OW; ++k) mask[k] = 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t f = (t0 + u >= lo && t0 + u < hi) ? ((1u << BV) - 1u) : 0u;
#pragma unroll
      for (int i = 0; i < MH; ++i) {
        const int bit = (8 * i + u) * BV;
        mask[bit / 32] |= f << (bit % 32);
        if ((bit % 32) + BV > 32) mask[bit / 32 + 1] |= f >> (32 - bit % 32);
      }
    }
#pragma unroll
    for (int k = 0; k < OB / 2; ++k) {
      const uint32_t sh = 16 * (k & 1);
      const uint32_t m = (mask[k / 2] >> sh) & 0xFFFFu;
      uint16_t* p = (uint16_t*)(d + 2 * k);
      *p = (uint16_t)((*p & ~m) | ((out[k / 2] >> sh) & m));
    }
  }
}

struct AppendArgs {
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint16_t* k_norms;
  uint16_t* v_norms;
  int64_t ls_kc, ls_vc, ls_kn, ls_vn; /* layer strides, bytes */
  int batch, heads, capacity, t_new, n_layers, slots;
  int64_t chunk;                      /* tile pairs per block */
  const int32_t* block_table;         /* paged storage: [batch][max_pages], else null */
  int lg_tpp, max_pages, num_pages;   /* log2(tiles per page), table row, pool pages */
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint8_t* sign_bits;
  const int32_t* pos;
  const tq_enc_entry* tab_k;
  const tq_enc_entry* tab_v;
  int ent_k, ent_v;
  float nbh_k, nbh_v;
  float off_k, off_v; /* nb_half + 1/2 + the codebook's bucket shift */
};

/* A 32-token tile takes two waves (16 vectors each); a block of 4 waves
 * works on two tiles side by side. */
constexpr int kAppendWaves = 4;
constexpr int kTPB = 2;

/* Whether key and value blocks alternate in one grid dimension. */
template <int BV>
constexpr bool kMixKV = BV == 2;

/* Task coordinates (layer, seq, head, slot), slot the tile offset from the
 * first tile touched by the append; tasks are numbered with slot fastest.
 * The divisions happen once per block; later tasks advance by carries. */
struct TaskIter {
  int64_t task;
  int layer, b, h, slot;
};

__device__ inline TaskIter task_at(const AppendArgs& a, int64_t task) {
  TaskIter t;
  t.task = task;
  t.slot = (int)(task % a.slots);
  int64_t r = task / a.slots;
  t.h = (int)(r % a.heads);
  r /= a.heads;
  t.b = (int)(r % a.batch);
  t.layer = (int)(r / a.batch);
  return t;
}

/* The task `step` further on (step <= slots). */
__device__ inline TaskIter task_advance(const AppendArgs& a, TaskIter t, int step) {
  t.task += step;
  t.slot += step;
  if (t.slot >= a.slots) {
    t.slot -= a.slots;
    if (++t.h == a.heads) {
      t.h = 0;
      if (++t.b == a.batch) {
        t.b = 0;
        ++t.layer;
      }
    }
  }
  return t;
}

/* Geometry of one wave's part of a task. */
struct TaskGeo {
  bool live;
  int layer, b, h, tile, jlo, jhi;
  int full_end;        /* rows below this (and at or above p0) receive appended tokens */
  int64_t rbase;       /* row index (within the layer's rows) of the tile's row 0 */
  int64_t vt;          /* value-tile index within the layer's tiles */
  const uint16_t* src; /* fp16 input row of tile row j0 (the wave's first row) */
};

/* Key (row) and value (tile) blocks: with 2-bit values they alternate
 * (blockIdx.x odd: values), which mixes the two write streams evenly and
 * measured faster; otherwise blockIdx.y = 1 marks the value blocks, all
 * dispatched after the key blocks, which measured faster for 3- and 4-bit
 * values.  Block k of a kind takes the tile
 * pairs [k chunk, (k + 1) chunk) in order (consecutive tiles of a stream, so
 * the layer and its sign flip rarely change), loading the next pair's
 * vectors while encoding the current one. */
template <int D, int BK, int BV>
__global__ void __launch_bounds__(64 * kAppendWaves) __attribute__((amdgpu_waves_per_eu(D == 256 ? 2 : TQ_ENC_WPE)))
append_kernel(AppendArgs a) {
  using G = EGeo<D>;
  /* static LDS: the table's address is a constant, folded into the reads */
  constexpr int kRows = tq_enc_rows_max(D, BK) > tq_enc_rows_max(D, BV) ? tq_enc_rows_max(D, BK)
                                                                       : tq_enc_rows_max(D, BV);
  __shared__ __align__(16) tq_enc_entry tab[kRows * kEncRep];
  __shared__ __align__(16) uint8_t vbuf_all[kAppendWaves * kVec * kVPitch<D>];
  constexpr bool kMix = kMixKV<BV>;
  const bool is_v = kMix ? (blockIdx.x & 1) != 0 : blockIdx.y == 1;
  const int ent = is_v ? a.ent_v : a.ent_k; /* <= kRows (checked by the codebook build) */
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  const int q4 = lane / 16, nl = lane % 16;
  const int slot_in_block = wave / 2, sub = wave % 2;
  /* the wave's value codes [row][coord], one row per token of its pass */
  uint8_t* vbuf = vbuf_all + wave * kVec * kVPitch<D>;
  const uint32_t tab_off = (uint32_t)(lane & (kEncRep - 1)) * sizeof(tq_enc_entry);
  const float nbh = is_v ? a.nbh_v : a.nbh_k;
  const float off = is_v ? a.off_v : a.off_k;
  const uint16_t* src_all = is_v ? a.v_new : a.k_new;
  const int64_t tasks = (int64_t)a.n_layers * a.batch * a.heads * a.slots;
  const int j0 = sub * kVec; /* this wave's first tile row */
  const HTiles ht = h_tiles(nl, q4);

  auto setup = [&](const TaskIter& t) -> TaskGeo {
    TaskGeo g;
    g.live = false;
    g.layer = t.layer;
    g.b = t.b;
    g.h = t.h;
    g.tile = g.jlo = g.jhi = g.full_end = 0;
    g.rbase = g.vt = 0;
    g.src = src_all;
    if (t.task >= tasks) return g;
    const int slot = t.slot;
    /* a scalar load: the index is uniform (a vector load here would make the
     * wave wait for all its outstanding memory operations) */
    const int p0 = ld_const(a.pos + g.b);
    /* the tile of this slot and its appended rows below capacity (nothing
     * when p0 is negative or at or past capacity) */
    if (!tq_append_tile_rows(p0, a.t_new, a.capacity, slot, &g.tile, &g.jlo, &g.jhi)) return g;
    g.full_end = tq_append_full_end(p0, a.t_new, a.capacity);
    if (a.block_table) {
      /* paged: the pool page of this tile's page (rows of pages outside the
       * pool are skipped) */
      const int tpp = 1 << a.lg_tpp;
      const int phys = ld_const(a.block_table + (int64_t)g.b * a.max_pages + (g.tile >> a.lg_tpp));
      if (phys < 0 || phys >= a.num_pages) return g;
      const int64_t pb = (int64_t)phys * a.heads + g.h;
      g.rbase = pb * (32 * tpp) + 32 * (g.tile & (tpp - 1));
      g.vt = pb * tpp + (g.tile & (tpp - 1));
    } else {
      const int64_t sh = (int64_t)g.b * a.heads + g.h;
      g.rbase = sh * a.capacity + 32 * (int64_t)g.tile;
      g.vt = sh * (a.capacity / 32) + g.tile;
    }
    /* this wave's 16 rows must meet the appended ones */
    if (g.jhi <= j0 || g.jlo >= j0 + kVec) {
      g.src = src_all;
    } else {
      const int64_t stream = ((int64_t)g.layer * a.batch + g.b) * a.heads + g.h;
      g.src = src_all + (stream * a.t_new + 32 * (int64_t)g.tile + j0 - p0) * D;
    }
    g.live = true;
    return g;
  };
  /* the lane's input row of a task, clamped into the task's appended rows
   * that this wave covers (any real row when it covers none) */
  auto lane_src = [&](const TaskGeo& g) -> const uint16_t* {
    const int lo = g.jlo > j0 ? g.jlo : j0, hi = g.jhi < j0 + kVec ? g.jhi : j0 + kVec;
    if (!g.live || hi <= lo) return src_all;
    int j = j0 + nl;
    if (j < lo) j = lo;
    if (j >= hi) j = hi - 1;
    return g.src + (int64_t)(j - j0) * D;
  };

  const int64_t pairs = (tasks + kTPB - 1) / kTPB;
  const int64_t first = (int64_t)(kMix ? blockIdx.x >> 1 : blockIdx.x) * a.chunk;
  int64_t last = first + a.chunk;
  if (last > pairs) last = pairs;
  if (first >= last) return;

  uint32_t sm[G::J][4];
  int sm_layer = -1;

  auto body = [&](const XRegs<D>& xr, const TaskGeo& g) {
    if (g.live && g.layer != sm_layer) {
      sign_masks<D>(a.sign_bits + (int64_t)g.layer * (D / 8), q4, sm);
      sm_layer = g.layer;
    }
    const int jrow = j0 + nl;
    const bool mine = g.live && jrow >= g.jlo && jrow < g.jhi;
    const int64_t row = g.rbase + jrow;
    const uint16_t* vec = lane_src(g);
    uint32_t piece[G::OB];
    if (!is_v) {
      const uint32_t n16 = encode_pass<D, BK, false>(xr, sm, ht, (const char*)tab, tab_off, nbh,
                                                     off, vec, piece);
      uint32_t out[Chunk<D, BK>::NW];
      gather_row_chunk<D, BK>(piece, out);
      if (mine) {
        store_chunk<D, BK, true>(a.k_codes + g.layer * a.ls_kc + row * (D * BK / 8) +
                                     q4 * Chunk<D, BK>::BYTES, out);
        if (q4 == 0) *(uint16_t*)((uint8_t*)a.k_norms + g.layer * a.ls_kn + row * 2) = (uint16_t)n16;
      }
    } else {
      const uint32_t n16 = encode_pass<D, BV, true>(xr, sm, ht, (const char*)tab, tab_off, nbh,
                                                    off, vec, piece);
      /* code bytes of coordinates 16 ob + 4 q4 .. +3 -> the wave's row nl */
#pragma unroll
      for (int ob = 0; ob < G::OB; ++ob)
        *(uint32_t*)(vbuf + nl * kVPitch<D> + 16 * ob + 4 * q4) = piece[ob];
      if (mine && q4 == 0)
        *(uint16_t*)((uint8_t*)a.v_norms + g.layer * a.ls_vn + row * 2) = (uint16_t)n16;
      /* the wave's own rows only: a wave-level fence orders the writes and
       * the reads of other lanes (LDS operations of a wave run in order) */
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (g.live && g.jhi > j0 && g.jlo < j0 + kVec)
        build_value_half<D, BV>(vbuf, lane, g.jlo - j0, g.jhi - j0,
                                a.v_codes + g.layer * a.ls_vc + g.vt * (32 * D * BV / 8) +
                                    sub * (16 * D * BV / 8));
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  };

  /* every wave of the block runs the same iterations */
  /* the first pair's loads go out before the table is built */
  XRegs<D> xa, xb;
  TaskIter tnext = task_at(a, first * kTPB + slot_in_block);
  TaskGeo ga = setup(tnext);
  load_x<D>(xa, lane_src(ga), q4);
  load_table(tab, is_v ? a.tab_v : a.tab_k, ent);
  __syncthreads();
  /* the geometry of the pair after `it` (the same pair again at the end,
   * so the prefetch loads are issued on every path) */
  auto next_geo = [&](int64_t it, const TaskGeo& same) -> TaskGeo {
    if (it + 1 >= last) return same;
    const int slot0 = tnext.slot;
    tnext = task_advance(a, tnext, kTPB);
    /* the common case, the same stream's tile kTPB further on, with this
     * tile and that one wholly appended: the geometry moves by constants */
    if (!a.block_table && same.live && tnext.slot == slot0 + kTPB &&
        tq_append_next_full(same.tile, same.jlo, same.jhi, same.full_end, kTPB)) {
      TaskGeo g = same;
      g.tile += kTPB;
      g.rbase += 32 * kTPB;
      g.vt += kTPB;
      g.src += (int64_t)32 * kTPB * D;
      return g;
    }
    return setup(tnext);
  };
  int64_t it = first;
  for (;;) {
    const TaskGeo gb = next_geo(it, ga);
    load_x<D>(xb, lane_src(gb), q4);
    body(xa, ga);
    if (++it >= last) break;
    ga = next_geo(it, gb);
    load_x<D>(xa, lane_src(ga), q4);
    body(xb, gb);
    if (++it >= last) break;
  }
}

/* ------------------------------------------------- one-token append -- */

/* Sign-flip masks as sign_masks, for a layer that may differ between the
 * lanes of a wave (vector loads). */
template <int D>
__device__ inline void sign_masks_lane(const uint8_t* sb, int q4, uint32_t (&m)[EGeo<D>::J][4]) {
#pragma unroll
  for (int j = 0; j < EGeo<D>::J; ++j) {
    const uint32_t b = (((const uint32_t*)sb)[j] >> (8 * q4)) & 0xFFu;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      m[j][w] = (((b >> (2 * w)) & 1u) << 15) | (((b >> (2 * w + 1)) & 1u) << 31);
  }
}

/* An append of one token per stream (a decode step).  The n_layers batch
 * heads new vectors of a kind are then one row-major matrix, encoded 16 per
 * wave pass as in tq_encode (lanes of one pass may belong to different
 * layers and sequences).  Key codes and norms go straight to the stream's
 * row.  A value token owns BV bits of every field of 16 segments of its tile
 * (tile row 8 q + u: segments 16 q + r, field m at bit (8 m + u) BV); lane
 * (token, segment) pairs merge those bits into the words already in memory.
 * One token per stream means no two vectors of a launch share a tile, so no
 * two merges touch one word.  blockIdx.y = 1 marks the value blocks. */
template <int D, int BK, int BV>
__global__ void __launch_bounds__(64 * kRowsWaves) __attribute__((amdgpu_waves_per_eu(D == 256 ? 2 : TQ_ENC_WPE)))
append_token_kernel(AppendArgs a) {
  using G = EGeo<D>;
  constexpr int kRows = tq_enc_rows_max(D, BK) > tq_enc_rows_max(D, BV) ? tq_enc_rows_max(D, BK)
                                                                       : tq_enc_rows_max(D, BV);
  constexpr int MS = D / 16;      /* fields per value segment */
  constexpr int SB = D * BV / 16; /* bytes per value segment (a multiple of 4) */
  constexpr int SW = SB / 4;
  __shared__ __align__(16) tq_enc_entry tab[kRows * kEncRep];
  __shared__ __align__(16) uint8_t vbuf_all[kRowsWaves * kVec * kVPitch<D>];
  /* per wave and token: byte offset of the value tile (-1: nothing to
   * write) and the token's tile row */
  __shared__ int64_t tbase_all[kRowsWaves * kVec];
  __shared__ int trow_all[kRowsWaves * kVec];
  const bool is_v = blockIdx.y == 1;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  const int q4 = lane / 16, nl = lane % 16;
  uint8_t* vbuf = vbuf_all + wave * kVec * kVPitch<D>;
  int64_t* tbase = tbase_all + wave * kVec;
  int* trow = trow_all + wave * kVec;
  const uint32_t tab_off = (uint32_t)(lane & (kEncRep - 1)) * sizeof(tq_enc_entry);
  const float nbh = is_v ? a.nbh_v : a.nbh_k;
  const float off = is_v ? a.off_v : a.off_k;
  const uint16_t* src_all = is_v ? a.v_new : a.k_new;
  const int64_t per_layer = (int64_t)a.batch * a.heads;
  const int64_t n = (int64_t)a.n_layers * per_layer;
  const int64_t passes = (n + kVec - 1) / kVec;
  const int64_t wstride = (int64_t)gridDim.x * kRowsWaves;
  int64_t ps = (int64_t)blockIdx.x * kRowsWaves + wave;
  load_table(tab, is_v ? a.tab_v : a.tab_k, is_v ? a.ent_v : a.ent_k);
  __syncthreads();
  const HTiles ht = h_tiles(nl, q4);
  for (; ps < passes; ps += wstride) {
    /* the lane's vector, clamped to a real one */
    const int64_t v = ps * kVec + nl;
    const int64_t vc = v < n ? v : n - 1;
    const int layer = (int)(vc / per_layer);
    const int64_t sh = vc - (int64_t)layer * per_layer; /* b heads + h */
    const int b = (int)(sh / a.heads), h = (int)(sh - (int64_t)b * a.heads);
    const uint16_t* vec = src_all + vc * D;
    XRegs<D> xr;
    load_x<D>(xr, vec, q4);
    uint32_t sm[G::J][4];
    sign_masks_lane<D>(a.sign_bits + (int64_t)layer * (D / 8), q4, sm);
    /* the token's row: tile p0 / 32, tile row p0 % 32 (nothing when p0 is
     * outside [0, capacity) or, paged, its page is outside the pool) */
    const int p0 = a.pos[b];
    int tile = 0, jlo = 0, jhi = 0;
    bool mine = v < n && tq_append_tile_rows(p0, 1, a.capacity, 0, &tile, &jlo, &jhi);
    int64_t rbase = 0, vt = 0;
    if (mine) {
      if (a.block_table) {
        const int tpp = 1 << a.lg_tpp;
        const int phys = a.block_table[(int64_t)b * a.max_pages + (tile >> a.lg_tpp)];
        mine = phys >= 0 && phys < a.num_pages;
        const int64_t pb = (int64_t)phys * a.heads + h;
        rbase = pb * (32 * tpp) + 32 * (tile & (tpp - 1));
        vt = pb * tpp + (tile & (tpp - 1));
      } else {
        rbase = sh * a.capacity + 32 * (int64_t)tile;
        vt = sh * (a.capacity / 32) + tile;
      }
    }
    const int64_t row = rbase + jlo;
    uint32_t piece[G::OB];
    if (!is_v) {
      const uint32_t n16 = encode_pass<D, BK, false>(xr, sm, ht, (const char*)tab, tab_off, nbh,
                                                     off, vec, piece);
      uint32_t out[Chunk<D, BK>::NW];
      gather_row_chunk<D, BK>(piece, out);
      if (mine) {
        store_chunk<D, BK, true>(a.k_codes + layer * a.ls_kc + row * (D * BK / 8) +
                                     q4 * Chunk<D, BK>::BYTES, out);
        if (q4 == 0) *(uint16_t*)((uint8_t*)a.k_norms + layer * a.ls_kn + row * 2) = (uint16_t)n16;
      }
      continue;
    }
    const uint32_t n16 = encode_pass<D, BV, true>(xr, sm, ht, (const char*)tab, tab_off, nbh,
                                                  off, vec, piece);
#pragma unroll
    for (int ob = 0; ob < G::OB; ++ob)
      *(uint32_t*)(vbuf + nl * kVPitch<D> + 16 * ob + 4 * q4) = piece[ob];
    if (q4 == 0) {
      tbase[nl] = mine ? layer * a.ls_vc + vt * (32 * D * BV / 8) : (int64_t)-1;
      trow[nl] = jlo;
      if (mine) *(uint16_t*)((uint8_t*)a.v_norms + layer * a.ls_vn + row * 2) = (uint16_t)n16;
    }
    /* the wave's own LDS rows: a wave-level fence orders the writes and the
     * other lanes' reads (LDS operations of a wave run in order) */
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int r = lane % 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = lane / 16 + 4 * i; /* the pass's token */
      const int64_t base = tbase[t];
      if (base < 0) continue;
      const int j = trow[t], u = j % 8;
      /* the token's codes of segment r (coordinates r MS .. r MS + MS - 1)
       * at field bits 8 m BV, then moved up to token u's place: u BV < 32,
       * and each code stays inside its own field */
      uint32_t cw[MS / 4];
#pragma unroll
      for (int k = 0; k < MS / 4; ++k)
        cw[k] = *(const uint32_t*)(vbuf + t * kVPitch<D> + r * MS + 4 * k);
      uint32_t bits0[SW], mask0[SW];
#pragma unroll
      for (int w = 0; w < SW; ++w) bits0[w] = mask0[w] = 0u;
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        const uint32_t code = (cw[m / 4] >> (8 * (m % 4))) & ((1u << BV) - 1u);
        put_bits(bits0, 8 * m * BV, code, BV);
        put_bits(mask0, 8 * m * BV, (1u << BV) - 1u, BV);
      }
      const uint32_t s = (uint32_t)(u * BV);
      uint32_t* seg = (uint32_t*)(a.v_codes + base + (int64_t)(16 * (j / 8) + r) * SB);
#pragma unroll
      for (int w = 0; w < SW; ++w) {
        const uint32_t lo_b = w > 0 ? bits0[w - 1] : 0u, lo_m = w > 0 ? mask0[w - 1] : 0u;
        const uint32_t bw = (uint32_t)((((uint64_t)bits0[w] << 32) | lo_b) >> (32 - s));
        const uint32_t mw = (uint32_t)((((uint64_t)mask0[w] << 32) | lo_m) >> (32 - s));
        seg[w] = (seg[w] & ~mw) | bw;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template <int D, int BK, int BV>
tq_status launch_append_token_t(const AppendArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_layers * a.batch * a.heads;
  const int64_t passes = (n + kVec - 1) / kVec;
  int64_t blocks = (passes + kRowsWaves - 1) / kRowsWaves;
  if (blocks < 1) return TQ_OK;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL((append_token_kernel<D, BK, BV>), dim3((unsigned)blocks, 2),
                     dim3(64 * kRowsWaves), 0, s, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

template <int D, int BITS>
tq_status launch_rows_t(const tq_codebook_s* cb, const uint16_t* x, int64_t n, int64_t stride,
                        const uint8_t* sb, uint8_t* codes, uint16_t* norms, hipStream_t s) {
  const int64_t passes = (n + kVec - 1) / kVec;
  int64_t blocks = (passes + kRowsWaves - 1) / kRowsWaves;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL((encode_rows_kernel<D, BITS>), dim3((unsigned)blocks), dim3(64 * kRowsWaves),
                     0, s, x, n, stride, sb, cb->enc_table, cb->enc_entries,
                     (float)cb->nb_half, (float)cb->nb_half + 0.5f + cb->enc_shift, codes, norms);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

template <int D, int BK, int BV>
tq_status launch_append_t(AppendArgs a, hipStream_t s) {
  const int64_t tasks = (int64_t)a.n_layers * a.batch * a.heads * a.slots;
  const int64_t pairs = (tasks + kTPB - 1) / kTPB;
  int64_t blocks = pairs < 2048 ? pairs : 2048;
  a.chunk = (pairs + blocks - 1) / blocks;
  blocks = (pairs + a.chunk - 1) / a.chunk;
  const dim3 grid = kMixKV<BV> ? dim3((unsigned)(2 * blocks)) : dim3((unsigned)blocks, 2);
  hipLaunchKernelGGL((append_kernel<D, BK, BV>), grid, dim3(64 * kAppendWaves), 0, s, a);
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
  a.chunk = 1;
  a.block_table = c->block_table;
  a.lg_tpp = 0;
  if (c->block_table)
    while ((32 << a.lg_tpp) < c->page_tokens) ++a.lg_tpp;
  a.max_pages = c->block_table ? c->max_pages : 0;
  a.num_pages = c->block_table ? c->num_pages : 0;
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
  a.off_k = (float)cbk->nb_half + 0.5f + cbk->enc_shift;
  a.off_v = (float)cbv->nb_half + 0.5f + cbv->enc_shift;
#define TQ_APP(DD, KK, VV) \
  if (c->head_dim == DD && c->bits_k == KK && c->bits_v == VV) \
    return t_new == 1 ? launch_append_token_t<DD, KK, VV>(a, s) : launch_append_t<DD, KK, VV>(a, s);
#define TQ_APP_D(DD) \
  TQ_APP(DD, 2, 2) TQ_APP(DD, 2, 3) TQ_APP(DD, 2, 4) TQ_APP(DD, 3, 2) TQ_APP(DD, 3, 3) \
  TQ_APP(DD, 3, 4) TQ_APP(DD, 4, 2) TQ_APP(DD, 4, 3) TQ_APP(DD, 4, 4)
  TQ_APP_D(64) TQ_APP_D(128) TQ_APP_D(256)
#undef TQ_APP_D
#undef TQ_APP
  return TQ_ERR_UNSUPPORTED;
}
