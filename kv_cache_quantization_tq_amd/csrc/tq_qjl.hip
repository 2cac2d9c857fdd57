/*
 * gfx950 kernels of the QJL stage: the 1-bit residual sketch of keys and the
 * inner-product estimate that uses it ("We Built a Python Library That Cuts
 * LLM Memory Usage by 80%", "Why not both stages?": the method's second
 * stage, one bit per coordinate of the residual, so that inner-product
 * estimates are unbiased).
 *
 * For a key x with stage-1 codes (tq_encode) the residual in the rotated unit
 * domain is r = R x / ||x|| - c[codes]; its sketch is gamma = fp16(||r||) and
 * the signs of S r (m = d rows of the caller's fp16 matrix S, bit set iff the
 * projection is >= 0).  The estimate of <q, x> is
 *   n16 * ( <R q, c[codes]> + sqrt(pi/2) / d * gamma * <S R q, z> ).
 *
 * qjl_encode_kernel: a wave sketches 16 keys at a time.  For d <= 128 both
 * products run on the matrix cores (v_mfma_f32_16x16x32_f16): the rotation
 * as a row-reordered Hadamard matrix (exact in fp16, staged in LDS with S)
 * times the sign-flipped fp16 keys, which leaves each lane a contiguous
 * quarter of the rotated coordinates, and S r with the residual in two fp16
 * parts (S is exact in fp16).  For d = 256 the rotation is the butterfly
 * Walsh-Hadamard transform in registers (in-lane strides 1, 2, 4 and >= 32;
 * strides 8 and 16 through the permlane swaps) and S is read through the
 * caches.  Sign nibbles are joined by permlane swaps, not LDS.
 * qjl_scores_kernel: 16 keys per wave on the matrix cores, like the decode's
 * scores: A = the keys' fp16 levels (plus their fp16 remainders against
 * q 2^-11) and their signs as +-1, B = the group's rotated queries and their
 * projections split into two fp16 parts (columns 0..7 and 8..15).  A lane
 * takes a contiguous quarter of a key's coordinates, so a tile's codes and
 * signs arrive in a few wide loads, and the next tile's are in flight while
 * one is scored.
 */
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kSqrtHalfPi = 1.2533141373155003f; /* sqrt(pi / 2) */

struct QjlEncArgs {
  const uint16_t* x;
  int64_t n, stride;
  const uint8_t* sign_bits;
  const uint16_t* S; /* fp16 [d][d] */
  const uint8_t* codes;
  uint8_t* signs;
  uint16_t* gamma;
  int vec_signs; /* signs 16-byte aligned: a key's sign row goes out in vector stores */
  float levels[16];
};

__device__ inline float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ inline uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

/* sum over the four 16-lane rows (lanes n, n+16, n+32, n+48) */
__device__ inline float rows_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

/* r0, r1 as fp16 pairs: hi = (fp16(r0), fp16(r1)) and lo = the fp16 of the
 * exact fp32 remainders r - hi (one pair conversion each, and one
 * mixed-precision fma per remainder: negone is -1 kept out of the
 * compiler's sight, so that r + hi * negone stays an fma on the fp16 hi). */
__device__ inline void split_pair(float r0, float r1, float negone, uint32_t& hw, uint32_t& lw) {
  const half2v h = __builtin_convertvector((float2v){r0, r1}, half2v);
  const float l0 = __builtin_fmaf((float)h[0], negone, r0);
  const float l1 = __builtin_fmaf((float)h[1], negone, r1);
  hw = __builtin_bit_cast(uint32_t, h);
  lw = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){l0, l1}, half2v));
}

/* S in LDS (rows padded against bank conflicts) for d <= 128; 256-dim heads
 * read it through the caches */
template <int D>
struct SLds {
  static constexpr bool ON = D <= 128;
  static constexpr int P = D + 8; /* row pitch, halfs */
  static constexpr int HALFS = ON ? D * P : 8;
};

/* Exchange with the lane 16 (X = 16) or 32 (X = 32) places away, as one
 * butterfly stage: the lower lane of each pair gets own + other, the upper
 * one other - own.  The permlane swaps hand every lane both values of its
 * pair ({lower, upper}) on the VALU, with no LDS round trip. */
template <int X>
__device__ inline float xbutterfly(float v, float sg) {
  const uint32_t u = __float_as_uint(v);
  const auto p = X == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(p[0]) + sg * __uint_as_float(p[1]);
}

/* One wave's 16 keys: lane (n, kq) holds key n's fp16
 * coordinates 32 s + 8 kq + 0..7 and their 8 codes each. */
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D, int B>
struct EncSlot {
  u32x4 xw[D / 32];
  uint32_t cw[D / 32];
};

/* The 8 B-bit codes of coordinates 32 s + 8 kq + 0..7: B bytes at byte
 * 4 B s + B kq of the row, read as the aligned words that hold them (rows
 * are multiples of 8 bytes from an 8-byte aligned base, so a second word is
 * read only when the bytes straddle two, and it lies inside the row). */
template <int B>
__device__ inline uint32_t enc_codes(const uint8_t* row, int off) {
  const uint32_t* w = (const uint32_t*)(row + (off & ~3));
  const uint32_t sh = (uint32_t)(off & 3) * 8u;
  if constexpr (B == 4)
    return w[0];
  else if constexpr (B == 2)
    return w[0] >> sh;
  else
    return (off & 3) + 3 > 4 ? __builtin_amdgcn_alignbit(w[1], w[0], sh) : w[0] >> sh;
}

template <int D, int B>
__device__ inline void enc_load(EncSlot<D, B>& r, const QjlEncArgs& a, int64_t v0, int n, int kq) {
  const int64_t v = v0 + n < a.n ? v0 + n : a.n - 1; /* ragged tail: the last key again */
  const uint8_t* row = a.codes + v * (D * B / 8);
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    r.xw[s] = __builtin_nontemporal_load((const u32x4*)(a.x + v * a.stride + 32 * s + 8 * kq));
    r.cw[s] = enc_codes<B>(row, (32 * s + 8 * kq) * B / 8);
  }
}

/* S r on the matrix cores for 16 keys (r in two fp16 parts, lane (n, kq)
 * holding key n's coordinates col0 + cstep s + 0..7 in rhi[s], rlo[s]):
 * rows 16 mt .. 16 mt + 15 of S per product; lane (n, kq) gets projections
 * 16 mt + 4 kq + 0..3 of key n, and the four nibbles of a key are joined by
 * the two permlane swaps; the key's sign row goes out from lane kq == 0. */
template <int D>
__device__ inline void enc_project(const half8 (&rhi)[D / 32], const half8 (&rlo)[D / 32],
                                   const _Float16* sl, const QjlEncArgs& a, int col0, int cstep,
                                   int64_t v, bool live, int n, int kq) {
  constexpr int KS = D / 32;
  using SL = SLds<D>;
  uint32_t packed[D / 32]; /* the key's D sign bits (every lane of the key) */
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) {
    floatx4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = col0 + cstep * s;
      const half8 sa = SL::ON ? *(const half8*)(sl + (16 * mt + n) * SL::P + col)
                              : *(const half8*)(a.S + (16 * mt + n) * D + col);
      t = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa, rhi[s], t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa, rlo[s], t, 0, 0, 0);
    }
    /* bit i = (t[i] >= 0): the complement of the sign bit (no sum here
     * is -0: each starts from +0) */
    uint32_t nib = __float_as_uint(t[0]) >> 31;
#pragma unroll
    for (int i = 1; i < 4; ++i) nib |= (__float_as_uint(t[i]) >> 31) << i;
    nib ^= 0xFu;
    const auto p16 = __builtin_amdgcn_permlane16_swap(nib, nib, false, false);
    const uint32_t byte = p16[0] | (p16[1] << 4);
    const auto p32 = __builtin_amdgcn_permlane32_swap(byte, byte, false, false);
    const uint32_t bits16 = p32[0] | (p32[1] << 8);
    if (mt & 1) packed[mt / 2] |= bits16 << 16;
    else packed[mt / 2] = bits16;
  }
  if (live && kq == 0) {
    uint8_t* dst = a.signs + v * (D / 8);
    if (a.vec_signs) {
      if constexpr (D == 64) {
        *(uint2*)dst = make_uint2(packed[0], packed[1]);
      } else {
#pragma unroll
        for (int k = 0; k < D / 128; ++k)
          ((uint4*)dst)[k] = make_uint4(packed[4 * k], packed[4 * k + 1], packed[4 * k + 2],
                                        packed[4 * k + 3]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < D / 32; ++k) ((uint32_t*)dst)[k] = packed[k];
    }
  }
}

/* Sketch the 16 keys v0 .. v0 + 15 held in r. */
template <int D, int B>
__device__ inline void enc_keys(const EncSlot<D, B>& r, const QjlEncArgs& a, const _Float16* sl,
                                const float2* plev, const uint32_t (&fm)[D / 32][4], int64_t v0,
                                int lane, int n, int kq) {
  constexpr int KS = D / 32;
  const int64_t v = v0 + n;
  const bool live = v < a.n;
  /* x slice with the sign flips D (an xor of the fp16 sign bits), squares
   * for the norm */
  float y[KS][8];
  float ss = 0.0f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t hw = r.xw[s][w] ^ fm[s][w];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float f = h2f((uint16_t)(hw >> (16 * t)));
        ss += f * f;
        y[s][2 * w + t] = f;
      }
    }
  }
  ss = rows_sum(ss);
  /* Walsh-Hadamard: coordinate 32 s + 8 kq + j */
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (!(j & h)) {
          const float p = y[s][j], q = y[s][j | h];
          y[s][j] = p + q;
          y[s][j | h] = p - q;
        }
  {
    const float sg16 = (lane & 16) ? -1.0f : 1.0f, sg32 = (lane & 32) ? -1.0f : 1.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) y[s][j] = xbutterfly<32>(xbutterfly<16>(y[s][j], sg16), sg32);
  }
#pragma unroll
  for (int h = 1; h < KS; h <<= 1)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      if (!(s & h))
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = y[s][j], q = y[s | h][j];
          y[s][j] = p + q;
          y[s | h][j] = p - q;
        }
  /* residual in the rotated unit domain: y / (sqrt(d) ||x||) - c[code] */
  const float scale = ss > 0.0f ? 1.0f / (sqrtf((float)D) * sqrtf(ss)) : 0.0f;
  float g2 = 0.0f, negone = -1.0f;
  asm volatile("" : "+v"(negone));
  half8 rhi[KS], rlo[KS];
  const uint32_t cpy = (uint32_t)lane & 3u;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float2 c = plev[((r.cw[s] >> (2 * B * u)) & ((1u << (2 * B)) - 1)) * 4 + cpy];
      const float r0 = y[s][2 * u] * scale - c.x, r1 = y[s][2 * u + 1] * scale - c.y;
      g2 += r0 * r0;
      g2 += r1 * r1;
      split_pair(r0, r1, negone, hw[u], lw[u]);
    }
    rhi[s] = __builtin_bit_cast(half8, u32x4{hw[0], hw[1], hw[2], hw[3]});
    rlo[s] = __builtin_bit_cast(half8, u32x4{lw[0], lw[1], lw[2], lw[3]});
  }
  g2 = rows_sum(g2);
  if (live && kq == 0) a.gamma[v] = f2h(sqrtf(g2));
  enc_project<D>(rhi, rlo, sl, a, 8 * kq, 32, v, live, n, kq);
}

/* d <= 128: the rotation on the matrix cores as well.  Hp is the Hadamard
 * matrix (entries (-1)^popcount(a & c), exact in fp16) with its rows
 * reordered so that row 16 mt + 4 kq + i of Hp is row (d/4) kq + 4 mt + i of
 * H: then the product Hp (D x), with D x the key slices as loaded (B
 * operand, lane (n, kq) supplying coordinates 32 s + 8 kq + 0..7 of key n),
 * leaves lane (n, kq) the rotated coordinates (d/4) kq + 0 .. d/4 - 1 of
 * key n.  That slice is contiguous, so its codes are one load, and it is,
 * coordinate for coordinate, the lane's B operand slice of S r. */
template <int D>
__device__ inline int hp_row(int r) {
  const int mt = r / 16, m = r % 16;
  return (D / 4) * (m / 4) + 4 * mt + (m % 4);
}

template <int D, int B>
struct EncSlotM {
  static constexpr int CB = D * B / 32; /* code bytes of a lane's d/4 coordinates */
  u32x4 xw[D / 32];
  uint32_t cw[(CB + 3) / 4];
};

template <int D, int B>
__device__ inline void enc_load_m(EncSlotM<D, B>& r, const QjlEncArgs& a, int64_t v0, int n,
                                  int kq) {
  constexpr int CB = EncSlotM<D, B>::CB;
  const int64_t v = v0 + n < a.n ? v0 + n : a.n - 1; /* ragged tail: the last key again */
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    r.xw[s] = __builtin_nontemporal_load((const u32x4*)(a.x + v * a.stride + 32 * s + 8 * kq));
  /* rows are multiples of 8 bytes from an 8-byte aligned base */
  const uint8_t* cp = a.codes + v * (D * B / 8) + kq * CB;
  if constexpr (CB % 8 == 0) {
#pragma unroll
    for (int k = 0; k < CB / 8; ++k) {
      const u32x2 w = __builtin_nontemporal_load((const u32x2*)cp + k);
      r.cw[2 * k] = w[0];
      r.cw[2 * k + 1] = w[1];
    }
  } else if constexpr (CB % 4 == 0) {
#pragma unroll
    for (int k = 0; k < CB / 4; ++k) r.cw[k] = __builtin_nontemporal_load((const uint32_t*)cp + k);
  } else { /* d = 64, 3 bits: 6 bytes at a 2-byte boundary */
    const uint16_t* h = (const uint16_t*)cp;
    r.cw[0] = (uint32_t)__builtin_nontemporal_load(h) |
              ((uint32_t)__builtin_nontemporal_load(h + 1) << 16);
    r.cw[1] = __builtin_nontemporal_load(h + 2);
  }
}

/* The 2 B-bit field of code pair p (coordinates 2 p, 2 p + 1 of the slice). */
template <int B>
__device__ inline uint32_t pair_field(const uint32_t* cw, int p) {
  const int bit = 2 * B * p, w = bit / 32, sh = bit % 32;
  const uint32_t v =
      sh + 2 * B > 32 ? __builtin_amdgcn_alignbit(cw[w + 1], cw[w], (uint32_t)sh) : cw[w] >> sh;
  return v & ((1u << (2 * B)) - 1);
}

template <int D, int B>
__device__ inline void enc_keys_m(const EncSlotM<D, B>& r, const QjlEncArgs& a, const _Float16* sl,
                                  const u32x4* hpt, const float2* plev,
                                  const uint32_t (&fm)[D / 32][4], int64_t v0, int lane, int n,
                                  int kq) {
  constexpr int KS = D / 32, NL = D / 4;
  const int64_t v = v0 + n;
  const bool live = v < a.n;
  /* D x as fp16 operands (an xor of the sign bits), squares for the norm */
  half8 xb[KS];
  float sq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      /* (the word goes through a plain variable: a bit cast of a vector
       * element compiled to a cast of element 0) */
      const uint32_t wk = r.xw[s][k] ^ fm[s][k];
      w[k] = wk;
      /* the squares of the fp16 pair, one dot product into fp32 */
      sq[k] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, wk), __builtin_bit_cast(half2v, wk),
                                     sq[k], false);
    }
    xb[s] = __builtin_bit_cast(half8, w);
  }
  const float ss = rows_sum((sq[0] + sq[1]) + (sq[2] + sq[3]));
  /* H D x a 16-row tile at a time: lane (n, kq) gets rotated coordinates
   * l = 4 mt + 0..3 of its slice, turned at once into the residual
   * y / (sqrt(d) ||x||) - c[code] and its two fp16 parts */
  const float scale = ss > 0.0f ? 1.0f / (sqrtf((float)D) * sqrtf(ss)) : 0.0f;
  const uint32_t cpy = (uint32_t)lane & 3u;
  float g2 = 0.0f, negone = -1.0f;
  asm volatile("" : "+v"(negone));
  uint32_t rhw[KS][4], rlw[KS][4];
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) {
    floatx4 t = {0.f, 0.f, 0.f, 0.f};
    /* row R of Hp held by the lane: (-1)^popcount(R & c) for columns c =
     * 32 s + 8 kq + j splits over disjoint bits into the pattern of R & 7
     * over j, one sign for R & 8 kq (both from the table) and one for
     * R & 32 s (a sign flip of all eight entries) */
    const int R = hp_row<D>(16 * mt + n);
    const u32x4 base = hpt[(R & 7) | ((__builtin_popcount((unsigned)(R & (8 * kq))) & 1) << 3)];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t f = (__builtin_popcount((unsigned)(R & (32 * s))) & 1) ? 0x80008000u : 0u;
      const u32x4 hw = {base[0] ^ f, base[1] ^ f, base[2] ^ f, base[3] ^ f};
      t = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, hw), xb[s], t, 0, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      /* coordinates l, l + 1 of the slice, l = 4 mt + 2 h: one fp16 pair */
      const float2 c = plev[pair_field<B>(r.cw, 2 * mt + h) * 4 + cpy];
      const float r0 = t[2 * h] * scale - c.x, r1 = t[2 * h + 1] * scale - c.y;
      g2 += r0 * r0;
      g2 += r1 * r1;
      const int l = 4 * mt + 2 * h;
      split_pair(r0, r1, negone, rhw[l / 8][(l % 8) / 2], rlw[l / 8][(l % 8) / 2]);
    }
  }
  half8 rhi[KS], rlo[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    rhi[s] = __builtin_bit_cast(half8, u32x4{rhw[s][0], rhw[s][1], rhw[s][2], rhw[s][3]});
    rlo[s] = __builtin_bit_cast(half8, u32x4{rlw[s][0], rlw[s][1], rlw[s][2], rlw[s][3]});
  }
  g2 = rows_sum(g2);
  if (live && kq == 0) a.gamma[v] = f2h(sqrtf(g2));
  /* keep the S operand reads from being hoisted into the rotation (their
   * registers on top of the rotation's would halve the waves per SIMD) */
  __builtin_amdgcn_sched_barrier(0);
  enc_project<D>(rhi, rlo, sl, a, NL * kq, 8, v, live, n, kq);
}

template <int D, int B>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 3 : 1)))
qjl_encode_kernel(QjlEncArgs a) {
  using SL = SLds<D>;
  __shared__ __align__(16) _Float16 sl[SL::HALFS];
  /* the levels of each pair of codes (first code in the low bits), 4 copies
   * (entry 4 p + lane % 4) */
  __shared__ float2 plev[(1 << (2 * B)) * 4];
  /* for d <= 128, the rows of Hp (rows reordered Hadamard matrix) over 8
   * consecutive columns 8 k + j: entry p + 8 c holds the fp16 +-1 values
   * (-1)^(popcount(p & j) + c), j = 0..7 */
  __shared__ u32x4 hpt[16];
  const int lane = threadIdx.x % 64, n = lane % 16, kq = lane / 16;
  if (threadIdx.x < 16) {
    const int p = threadIdx.x & 7, c = threadIdx.x >> 3;
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = 0x3C003C00u | ((uint32_t)((__builtin_popcount((unsigned)(p & (2 * k))) + c) & 1) << 15) |
             ((uint32_t)((__builtin_popcount((unsigned)(p & (2 * k + 1))) + c) & 1) << 31);
    hpt[threadIdx.x] = w;
  }
  for (int e = threadIdx.x; e < (1 << (2 * B)) * 4; e += blockDim.x) {
    const int p = e / 4;
    plev[e] = make_float2(a.levels[p & ((1 << B) - 1)], a.levels[p >> B]);
  }
  __syncthreads();
  if constexpr (SL::ON) {
    for (int t = threadIdx.x; t < D * D / 8; t += blockDim.x) {
      const int r = t / (D / 8), c = t % (D / 8);
      *(uint4*)(sl + r * SL::P + 8 * c) = *(const uint4*)(a.S + r * D + 8 * c);
    }
    __syncthreads();
  }
  /* the lane's sign flips: coordinate 32 s + 8 kq + 2 w + t flips the fp16
   * sign bit 16 t + 15 of word w of slice s */
  uint32_t fm[D / 32][4];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    const uint32_t fb = a.sign_bits[(32 * s + 8 * kq) >> 3];
#pragma unroll
    for (int w = 0; w < 4; ++w)
      fm[s][w] = (((fb >> (2 * w)) & 1u) << 15) | (((fb >> (2 * w + 1)) & 1u) << 31);
  }
  /* each wave sketches groups of 16 keys, striding over the grid */
  const int64_t stride = (int64_t)gridDim.x * 64;
  int64_t v0 = ((int64_t)blockIdx.x * 4 + threadIdx.x / 64) * 16;
  if (v0 >= a.n) return;
  if constexpr (SL::ON) {
    /* two register slots: the next group's keys and codes load while one
     * is sketched (the LDS, not the registers, sets the waves per SIMD) */
    const int64_t cnt = (a.n - 1 - v0) / stride + 1;
    EncSlotM<D, B> ra, rb;
    enc_load_m<D, B>(ra, a, v0, n, kq);
    for (int64_t k = 0; k + 2 <= cnt; k += 2) {
      enc_load_m<D, B>(rb, a, v0 + stride, n, kq);
      enc_keys_m<D, B>(ra, a, sl, hpt, plev, fm, v0, lane, n, kq);
      v0 += stride;
      if (k + 2 < cnt) enc_load_m<D, B>(ra, a, v0 + stride, n, kq);
      enc_keys_m<D, B>(rb, a, sl, hpt, plev, fm, v0, lane, n, kq);
      v0 += stride;
    }
    if (cnt & 1) enc_keys_m<D, B>(ra, a, sl, hpt, plev, fm, v0, lane, n, kq);
  } else {
    /* one slot: with the rotation in registers a second one would cost the
     * second wave per SIMD, which hides more */
    for (; v0 < a.n; v0 += stride) {
      EncSlot<D, B> ra;
      enc_load<D, B>(ra, a, v0, n, kq);
      enc_keys<D, B>(ra, a, sl, plev, fm, v0, lane, n, kq);
    }
  }
}

struct QjlScoreArgs {
  const uint16_t* q; /* fp16 [G][d] */
  int G;
  const uint8_t* sign_bits;
  const uint16_t* S;
  const uint8_t* codes;
  const uint16_t* norms;
  const uint8_t* signs;
  const uint16_t* gamma;
  int64_t T;
  float* out; /* [G][T] */
  int vec_out; /* T % 4 == 0 and out 16-byte aligned: rows of 4 keys go out as one store */
  int vec_ng;  /* norms and gamma 8-byte aligned: 4 keys' values in one load each */
  float levels[16];
};

typedef float floatv4 __attribute__((ext_vector_type(4)));

/* Row reduction partner: the value of the lane 8 places along in the
 * 16-lane row. */
__device__ inline float ror8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}

/* A lane's share of one 16-key tile.  Lane (n, kq) takes key k0 + n's
 * coordinates kq d/4 + 0 .. d/4 - 1 (the dot products do not depend on how
 * coordinates are dealt out, as long as A and B agree), so its codes and
 * sign bits are one contiguous slice of the key's rows; plus the norms and
 * gammas of keys k0 + 4 kq + 0..3, the rows its output column covers. */
template <int D, int B>
struct KeySlice {
  static constexpr int KS = D / 32;          /* matrix-core steps per tile */
  static constexpr int CB = KS * B;          /* code bytes per lane */
  static constexpr int CW = (CB + 3) / 4;
  static constexpr int ZW = (KS + 3) / 4;    /* KS sign bytes */
  uint32_t cw[CW];
  uint32_t zw[ZW];
  uint32_t nm[2], gm[2]; /* fp16 norms / gammas of the 4 keys, two per word */
};

/* Streamed once: non-temporal loads.  Keys past the end are clamped to the
 * last one (their rows of the product are never stored). */
template <int D, int B>
__device__ inline void load_slice(KeySlice<D, B>& r, const QjlScoreArgs& a, int64_t k0, int n,
                                  int kq) {
  typedef KeySlice<D, B> KSl;
  const int64_t last = a.T - 1;
  const int64_t key = k0 + n < last ? k0 + n : last;
  /* rows are multiples of 8 bytes from an 8-byte aligned base */
  const uint8_t* cp = a.codes + key * (D * B / 8) + kq * KSl::CB;
  if constexpr (KSl::CB % 8 == 0) {
#pragma unroll
    for (int k = 0; k < KSl::CB / 8; ++k) {
      const u32x2 w = __builtin_nontemporal_load((const u32x2*)cp + k);
      r.cw[2 * k] = w[0];
      r.cw[2 * k + 1] = w[1];
    }
  } else if constexpr (KSl::CB % 4 == 0) {
#pragma unroll
    for (int k = 0; k < KSl::CB / 4; ++k)
      r.cw[k] = __builtin_nontemporal_load((const uint32_t*)cp + k);
  } else { /* d = 64, 3 bits: 6 bytes at a 2-byte boundary */
    const uint16_t* h = (const uint16_t*)cp;
    r.cw[0] = (uint32_t)__builtin_nontemporal_load(h) |
              ((uint32_t)__builtin_nontemporal_load(h + 1) << 16);
    r.cw[1] = __builtin_nontemporal_load(h + 2);
  }
  const uint8_t* zp = a.signs + key * (D / 8) + kq * KSl::KS;
  if constexpr (KSl::KS == 2)
    r.zw[0] = __builtin_nontemporal_load((const uint16_t*)zp);
  else
#pragma unroll
    for (int k = 0; k < KSl::ZW; ++k) r.zw[k] = __builtin_nontemporal_load((const uint32_t*)zp + k);
  const int64_t k4 = k0 + 4 * kq;
  if (a.vec_ng && k4 + 3 <= last) {
    /* the 4 keys' norms and gammas as one 8-byte load each */
    const u32x2 nw = __builtin_nontemporal_load((const u32x2*)(a.norms + k4));
    const u32x2 gw = __builtin_nontemporal_load((const u32x2*)(a.gamma + k4));
    r.nm[0] = nw[0], r.nm[1] = nw[1], r.gm[0] = gw[0], r.gm[1] = gw[1];
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t k = k4 + 2 * i < last ? k4 + 2 * i : last;
      const int64_t k1 = k4 + 2 * i + 1 < last ? k4 + 2 * i + 1 : last;
      r.nm[i] = (uint32_t)__builtin_nontemporal_load(a.norms + k) |
                ((uint32_t)__builtin_nontemporal_load(a.norms + k1) << 16);
      r.gm[i] = (uint32_t)__builtin_nontemporal_load(a.gamma + k) |
                ((uint32_t)__builtin_nontemporal_load(a.gamma + k1) << 16);
    }
  }
}

/* The 8 B-bit codes of matrix-core step s from a lane's slice. */
template <int D, int B>
__device__ inline uint32_t step_codes(const KeySlice<D, B>& r, int s) {
  if constexpr (B == 4) {
    return r.cw[s];
  } else if constexpr (B == 2) {
    return (r.cw[s / 2] >> (16 * (s & 1))) & 0xFFFFu;
  } else {
    const int bit = 24 * s, w = bit / 32, sh = bit % 32;
    return sh + 24 > 32 ? __builtin_amdgcn_alignbit(r.cw[w + 1], r.cw[w], (uint32_t)sh)
                        : r.cw[w] >> sh;
  }
}

/* LDS tables of the scores kernel.  plev: for each pair of B-bit codes
 * (first code in the low bits) the words {fp16 c0 | fp16 c1 << 16} and
 * {fp16 r0 | fp16 r1 << 16}, r = fp16((c - fp16 c) 2^11), in 4 copies
 * (entry 4 p + lane % 4); zpm: for each byte of sign bits the 8 fp16 values
 * +-1 (bit j set -> +1 in half j). */
template <int B>
struct ScoreLds {
  static constexpr int PAIRS = 1 << (2 * B);
  uint2 plev[PAIRS * 4];
  uint4 zpm[256];
};

/* Estimates for one tile of 16 keys at k0 from the lane's slice r.  Step s
 * covers the lane's coordinates 8 s + 0..7: the levels in two products
 * (A = {c0, c1, r0, r1, c2, c3, r2, r3} fp16 straight from two table words,
 * B = the query parts in the same order), the signs in one. */
template <int D, int B>
__device__ inline floatv4 score_tile(const KeySlice<D, B>& r, const half8 (&bv)[2 * (D / 32)],
                                     const half8 (&bs)[D / 32], const ScoreLds<B>& tb,
                                     uint32_t cpy, int n) {
  constexpr int KS = D / 32;
  floatx4 c1 = {0.f, 0.f, 0.f, 0.f}, c2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const uint32_t cw = step_codes<D, B>(r, s);
    const uint32_t zb = (r.zw[s / 4] >> (8 * (s % 4))) & 0xFFu;
    const uint4 z = tb.zpm[zb];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint2 e0 = tb.plev[((cw >> (4 * B * h)) & ((1u << (2 * B)) - 1)) * 4 + cpy];
      const uint2 e1 = tb.plev[((cw >> (4 * B * h + 2 * B)) & ((1u << (2 * B)) - 1)) * 4 + cpy];
      const uint4 w = {e0.x, e0.y, e1.x, e1.y};
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, w), bv[2 * s + h], c1,
                                                  0, 0, 0);
    }
    c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, z), bs[s], c2, 0, 0, 0);
  }
  /* lane (n, kq) holds keys k0 + 4 kq + 0..3 of column n; join the fp16
   * parts (column n + 8) into columns n < 8 */
  floatv4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float m1 = c1[i] + ror8(c1[i]), m2 = c2[i] + ror8(c2[i]);
    const uint16_t nh = (uint16_t)(r.nm[i / 2] >> (16 * (i & 1)));
    const uint16_t gh = (uint16_t)(r.gm[i / 2] >> (16 * (i & 1)));
    o[i] = h2f(nh) * (m1 + h2f(gh) * m2);
  }
  return o;
}

/* Store one tile's estimates: lane (n, kq) holds keys k0 + 4 kq + 0..3 of
 * query n. */
__device__ inline void store_tile(const QjlScoreArgs& a, floatv4 o, int64_t k0, int n, int kq) {
  if (n < a.G) {
    const int64_t kb = k0 + 4 * kq;
    float* dst = a.out + n * a.T + kb;
    /* ordinary stores: the two halves of a line meet in the cache */
    if (a.vec_out && kb + 4 <= a.T) {
      *(floatv4*)dst = o;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (kb + i < a.T) dst[i] = o[i];
    }
  }
}

template <int D, int B>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 4 : 1)))
qjl_scores_kernel(QjlScoreArgs a) {
  constexpr int KS = D / 32;
  __shared__ float rq[8][D];   /* R q */
  __shared__ float sq[8][D];   /* S R q * sqrt(pi/2) / d */
  __shared__ ScoreLds<B> tb;
  const int tid = threadIdx.x, lane = tid % 64, n = lane % 16, kq = lane / 16, wave = tid / 64;
  for (int e = tid; e < ScoreLds<B>::PAIRS * 4; e += blockDim.x) {
    const int p = e / 4;
    uint32_t hw = 0, lw = 0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float c = a.levels[(p >> (B * t)) & ((1 << B) - 1)];
      const _Float16 h = (_Float16)c;
      const _Float16 l = (_Float16)((c - (float)h) * 2048.0f);
      hw |= (uint32_t)__builtin_bit_cast(uint16_t, h) << (16 * t);
      lw |= (uint32_t)__builtin_bit_cast(uint16_t, l) << (16 * t);
    }
    tb.plev[e] = make_uint2(hw, lw);
  }
  {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (((tid >> (2 * k)) & 1) ? 0x3C00u : 0xBC00u) |
             ((((tid >> (2 * k + 1)) & 1) ? 0x3C00u : 0xBC00u) << 16);
    tb.zpm[tid] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  /* R q = H D q / sqrt(d), one thread per (query, coordinate), by a plain
   * O(d log d) pass through LDS */
  for (int t = tid; t < a.G * D; t += blockDim.x) {
    const int g = t / D, i = t % D;
    const float f = h2f(a.q[g * D + i]);
    rq[g][i] = ((a.sign_bits[i >> 3] >> (i & 7)) & 1) ? -f : f;
  }
  __syncthreads();
  for (int h = 1; h < D; h <<= 1) {
    float nv[(8 * D + 255) / 256];
    int k = 0;
    for (int t = tid; t < a.G * D; t += blockDim.x, ++k) {
      const int g = t / D, i = t % D;
      const float p = rq[g][i & ~h], q = rq[g][i | h];
      nv[k] = (i & h) ? p - q : p + q;
    }
    __syncthreads();
    k = 0;
    for (int t = tid; t < a.G * D; t += blockDim.x, ++k) rq[t / D][t % D] = nv[k];
    __syncthreads();
  }
  for (int t = tid; t < a.G * D; t += blockDim.x) rq[t / D][t % D] *= 1.0f / sqrtf((float)D);
  __syncthreads();
  /* S R q on the matrix cores: 16-row tiles of S (exact in fp16; lane
   * (m, kq) supplies row i0 + m, columns 32 s + 8 kq + 0..7) times the
   * rotated queries in two fp16 parts (lane (g, kq) supplies query g's
   * coordinates 32 s + 8 kq + 0..7), row tiles dealt out to the waves */
  for (int i0 = 16 * wave; i0 < D; i0 += 64) {
    floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint16_t* srow = a.S + (i0 + n) * D + 32 * s + 8 * kq;
      half8 av, bh, bm;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        av[j] = __builtin_bit_cast(_Float16, srow[j]);
        const float r = n < a.G ? rq[n & 7][32 * s + 8 * kq + j] : 0.0f;
        bh[j] = (_Float16)r;
        bm[j] = (_Float16)(r - (float)bh[j]);
      }
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bh, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bm, c, 0, 0, 0);
    }
    /* lane (g, kq) holds rows i0 + 4 kq + 0..3 of query g */
    if (n < a.G)
#pragma unroll
      for (int i = 0; i < 4; ++i) sq[n][i0 + 4 * kq + i] = c[i] * (kSqrtHalfPi / D);
  }
  __syncthreads();
  /* B operands, lane (n, kq), coordinates kq d/4 + 8 s + 0..7: columns 0..7
   * the fp16 parts of query n, 8..15 their fp16 remainders (levels and sign
   * products); for the level remainders fp16(R q 2^-11) in columns 0..7 */
  half8 bv[2 * KS], bs[KS];
  {
    const int g = n & 7;
    const bool hiCol = n < 8, ok = g < a.G;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = kq * (D / 4) + 8 * s + j;
        const float r = ok ? rq[g][i] : 0.0f, z = ok ? sq[g][i] : 0.0f;
        const _Float16 rh = (_Float16)r, zh = (_Float16)z;
        /* level products: coordinates j = 4 h + 2 u + t sit at half
         * 4 u + t (level part) and 4 u + 2 + t (remainder part) of bv[2 s + h] */
        const int h = j / 4, u = (j / 2) % 2, t = j % 2;
        bv[2 * s + h][4 * u + t] = hiCol ? rh : (_Float16)(r - (float)rh);
        bv[2 * s + h][4 * u + 2 + t] = hiCol ? (_Float16)(r * 0x1p-11f) : (_Float16)0.0f;
        bs[s][j] = hiCol ? zh : (_Float16)(z - (float)zh);
      }
  }
  /* pairs of adjacent 16-key tiles striding over the grid (a wave's two
   * stores per query then cover 128 contiguous output bytes), two register
   * slots: the next tile's loads are in flight while the current one is
   * scored */
  const uint32_t cpy = (uint32_t)lane & 3u;
  const int64_t ntile = (a.T + 15) / 16, npair = (ntile + 1) / 2;
  const int64_t stride = (int64_t)gridDim.x * 4, p0 = (int64_t)blockIdx.x * 4 + wave;
  if (p0 >= npair) return;
  const int64_t pcnt = (npair - 1 - p0) / stride + 1;
  const int64_t cnt = 2 * pcnt - (2 * (p0 + (pcnt - 1) * stride) + 1 >= ntile ? 1 : 0);
  /* the wave's k-th tile */
  auto tile_of = [&](int64_t k) { return 2 * (p0 + (k >> 1) * stride) + (k & 1); };
  /* three register slots: two tiles' loads in flight while one is scored
   * (tiles past the wave's last load its last tile again, unscored).  The
   * estimates of the first tile of a pair wait for the second's, so that
   * the two halves of each 128-byte output line go out back to back. */
  KeySlice<D, B> ra, rb, rc;
  auto tl = [&](int64_t k) { return tile_of(k < cnt ? k : cnt - 1) * 16; };
  floatv4 held = {0.f, 0.f, 0.f, 0.f};
  auto emit = [&](int64_t k, floatv4 o) {
    if (!(k & 1) && k + 1 < cnt) {
      held = o;
    } else {
      if (k & 1) store_tile(a, held, tl(k - 1), n, kq);
      store_tile(a, o, tl(k), n, kq);
    }
  };
  load_slice<D, B>(ra, a, tl(0), n, kq);
  load_slice<D, B>(rb, a, tl(1), n, kq);
  int64_t k = 0;
  for (; k + 3 <= cnt; k += 3) {
    load_slice<D, B>(rc, a, tl(k + 2), n, kq);
    emit(k, score_tile<D, B>(ra, bv, bs, tb, cpy, n));
    load_slice<D, B>(ra, a, tl(k + 3), n, kq);
    emit(k + 1, score_tile<D, B>(rb, bv, bs, tb, cpy, n));
    load_slice<D, B>(rb, a, tl(k + 4), n, kq);
    emit(k + 2, score_tile<D, B>(rc, bv, bs, tb, cpy, n));
  }
  if (k < cnt) emit(k, score_tile<D, B>(ra, bv, bs, tb, cpy, n));
  if (k + 1 < cnt) emit(k + 1, score_tile<D, B>(rb, bv, bs, tb, cpy, n));
}

/* Blocks of kernel K (256 threads) the device holds at once (occupancy x
 * CUs), looked up once per process; 1024 when no device answers. */
template <auto K>
int resident_blocks() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, K, 256, 0) != hipSuccess || cus <= 0 ||
        per <= 0) {
      (void)hipGetLastError();
      return 1024;
    }
    cached = cus * per;
  }
  return cached;
}

}  // namespace

tq_status tq_launch_qjl_encode(const tq_codebook_s* cb, const uint16_t* x, int64_t n,
                               int64_t stride, const uint8_t* sign_bits, const uint16_t* S,
                               const uint8_t* codes, uint8_t* signs, uint16_t* gamma,
                               hipStream_t s) {
  QjlEncArgs a;
  a.x = x;
  a.n = n;
  a.stride = stride;
  a.sign_bits = sign_bits;
  a.S = S;
  a.codes = codes;
  a.signs = signs;
  a.gamma = gamma;
  a.vec_signs = ((uintptr_t)signs & 15) == 0;
  for (int k = 0; k < 16; ++k) a.levels[k] = k < (1 << cb->bits) ? cb->centroids[k] : 0.0f;
  /* 4 waves of 16 keys a block; at most one round of resident blocks, whose
   * waves then stride (each block stages S and the reordered Hadamard
   * matrix once) */
  const int64_t need = (n + 63) / 64;
#define TQ_QE(DD, BB) \
  if (cb->d == DD && cb->bits == BB) { \
    const int64_t cap = resident_blocks<qjl_encode_kernel<DD, BB>>(); \
    hipLaunchKernelGGL((qjl_encode_kernel<DD, BB>), dim3((unsigned)(need < cap ? need : cap)), \
                       dim3(256), 0, s, a); \
  } else
  TQ_QE(64, 2) TQ_QE(64, 3) TQ_QE(64, 4) TQ_QE(128, 2) TQ_QE(128, 3) TQ_QE(128, 4)
  TQ_QE(256, 2) TQ_QE(256, 3) TQ_QE(256, 4) return TQ_ERR_UNSUPPORTED;
#undef TQ_QE
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

tq_status tq_launch_qjl_scores(const tq_codebook_s* cb, const uint16_t* q, int G,
                               const uint8_t* sign_bits, const uint16_t* S, const uint8_t* codes,
                               const uint16_t* norms, const uint8_t* signs,
                               const uint16_t* gamma, int64_t T, float* out, hipStream_t s) {
  QjlScoreArgs a;
  a.q = q;
  a.G = G;
  a.sign_bits = sign_bits;
  a.S = S;
  a.codes = codes;
  a.norms = norms;
  a.signs = signs;
  a.gamma = gamma;
  a.T = T;
  a.out = out;
  a.vec_out = T % 4 == 0 && ((uintptr_t)out & 15) == 0;
  a.vec_ng = ((uintptr_t)norms & 7) == 0 && ((uintptr_t)gamma & 7) == 0;
  for (int k = 0; k < 16; ++k) a.levels[k] = k < (1 << cb->bits) ? cb->centroids[k] : 0.0f;
  /* 4 waves of two 16-key tiles a block; at most one round of resident
   * blocks, whose waves then stride (each block projects the queries once) */
  const int64_t need = (T + 127) / 128;
#define TQ_QS(DD, BB) \
  if (cb->d == DD && cb->bits == BB) { \
    const int64_t cap = resident_blocks<qjl_scores_kernel<DD, BB>>(); \
    hipLaunchKernelGGL((qjl_scores_kernel<DD, BB>), dim3((unsigned)(need < cap ? need : cap)), \
                       dim3(256), 0, s, a); \
  } else
  TQ_QS(64, 2) TQ_QS(64, 3) TQ_QS(64, 4) TQ_QS(128, 2) TQ_QS(128, 3) TQ_QS(128, 4)
  TQ_QS(256, 2) TQ_QS(256, 3) TQ_QS(256, 4) return TQ_ERR_UNSUPPORTED;
#undef TQ_QS
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}
