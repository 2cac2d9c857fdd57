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
 * qjl_encode_kernel: a wave sketches 16 keys at a time (S staged in LDS
 * per block for d <= 128).  Lane (n, kq) holds
 * coordinates 32 s + 8 kq + 0..7 of key n, so the residual it computes is
 * exactly its slice of the B operand of S R^T on the matrix cores
 * (v_mfma_f32_16x16x32_f16, r split into two fp16 parts; S is exact in fp16).
 * The rotation is the butterfly Walsh-Hadamard transform: in-lane strides
 * 1, 2, 4 and >= 32, lane-xor 16 and 32 for strides 8 and 16.
 * qjl_scores_kernel: 16 keys per wave on the matrix cores, like the decode's
 * scores: A = the keys' fp16 levels (plus their fp16 remainders against
 * q 2^-11) and their signs as +-1, B = the group's rotated queries and their
 * projections split into two fp16 parts (columns 0..7 and 8..15).
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

/* 8 consecutive B-bit codes starting at a byte boundary (B bytes, read as
 * bytes: the rows are only byte-aligned for B = 3). */
template <int B>
__device__ inline uint32_t codes8(const uint8_t* p) {
  uint32_t w = 0;
#pragma unroll
  for (int k = 0; k < B; ++k) w |= (uint32_t)p[k] << (8 * k);
  return w;
}

/* S in LDS (rows padded against bank conflicts) for d <= 128; 256-dim heads
 * read it through the caches */
template <int D>
struct SLds {
  static constexpr bool ON = D <= 128;
  static constexpr int P = D + 8; /* row pitch, halfs */
  static constexpr int HALFS = ON ? D * P : 8;
};

template <int D, int B>
__global__ void __launch_bounds__(256) qjl_encode_kernel(QjlEncArgs a) {
  constexpr int KS = D / 32;
  using SL = SLds<D>;
  __shared__ __align__(16) _Float16 sl[SL::HALFS];
  const int lane = threadIdx.x % 64, n = lane % 16, kq = lane / 16;
  if constexpr (SL::ON) {
    for (int t = threadIdx.x; t < D * D / 8; t += blockDim.x) {
      const int r = t / (D / 8), c = t % (D / 8);
      *(uint4*)(sl + r * SL::P + 8 * c) = *(const uint4*)(a.S + r * D + 8 * c);
    }
    __syncthreads();
  }
  /* each wave sketches groups of 16 keys, striding over the grid */
  for (int64_t v0 = ((int64_t)blockIdx.x * 4 + threadIdx.x / 64) * 16; v0 < a.n;
       v0 += (int64_t)gridDim.x * 64) {
  const int64_t v = v0 + n;
  const bool live = v < a.n;
  /* x slice, sign flips D, squares for the norm */
  float y[KS][8];
  float ss = 0.0f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int i0 = 32 * s + 8 * kq;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (live) w = *(const uint4*)(a.x + v * a.stride + i0);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    const uint32_t flips = a.sign_bits[i0 >> 3];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float f = h2f((uint16_t)(ww[j / 2] >> (16 * (j & 1))));
      ss += f * f;
      y[s][j] = ((flips >> j) & 1) ? -f : f;
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
#pragma unroll
  for (int h = 16; h <= 32; h <<= 1)
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float o = __shfl_xor(y[s][j], h);
        y[s][j] = (lane & h) ? o - y[s][j] : y[s][j] + o;
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
  const uint8_t* row = a.codes + (live ? v : 0) * (D * B / 8);
  float g2 = 0.0f;
  half8 rhi[KS], rlo[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    /* the 8 codes of coordinates 32 s + 8 kq + 0..7: B bytes of the row */
    const uint32_t cw = live ? codes8<B>(row + (32 * s + 8 * kq) * B / 8) : 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float r = live ? y[s][j] * scale - a.levels[(cw >> (B * j)) & ((1u << B) - 1)] : 0.0f;
      g2 += r * r;
      const _Float16 hi = (_Float16)r;
      rhi[s][j] = hi;
      rlo[s][j] = (_Float16)(r - (float)hi);
    }
  }
  g2 = rows_sum(g2);
  if (live && kq == 0) a.gamma[v] = f2h(sqrtf(g2));
  /* S r on the matrix cores: rows 16 mt .. 16 mt + 15 of S per product;
   * lane (n, kq) gets projections 16 mt + 4 kq + 0..3 of key n */
  uint32_t packed[D / 32]; /* the key's D sign bits, for lane kq == 0 */
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) {
    floatx4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const half8 sa = SL::ON ? *(const half8*)(sl + (16 * mt + n) * SL::P + 32 * s + 8 * kq)
                              : *(const half8*)(a.S + (16 * mt + n) * D + 32 * s + 8 * kq);
      t = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa, rhi[s], t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa, rlo[s], t, 0, 0, 0);
    }
    uint32_t nib = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) nib |= (t[i] >= 0.0f ? 1u : 0u) << i;
    const uint32_t n1 = __shfl_xor(nib, 16), n2 = __shfl_xor(nib, 32), n3 = __shfl_xor(nib, 48);
    const uint32_t bits16 = nib | (n1 << 4) | (n2 << 8) | (n3 << 12);
    if (mt & 1) packed[mt / 2] |= bits16 << 16;
    else packed[mt / 2] = bits16;
  }
  if (live && kq == 0) {
    uint32_t* dst = (uint32_t*)(a.signs + v * (D / 8));
#pragma unroll
    for (int k = 0; k < D / 32; ++k) dst[k] = packed[k];
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
  float levels[16];
};

/* Row reduction partner: the value of the lane 8 places along in the
 * 16-lane row. */
__device__ inline float ror8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}

template <int D, int B>
__global__ void __launch_bounds__(256) qjl_scores_kernel(QjlScoreArgs a) {
  constexpr int KS = D / 32;
  __shared__ float rq[8][D];   /* R q */
  __shared__ float sq[8][D];   /* S R q * sqrt(pi/2) / d */
  __shared__ uint32_t lev[64]; /* level c as {fp16 c, fp16 (c - fp16 c) 2^11}, 4 copies */
  const int tid = threadIdx.x, lane = tid % 64, n = lane % 16, kq = lane / 16;
  if (tid < 64) {
    const float c = a.levels[tid / 4];
    const _Float16 h = (_Float16)c;
    const _Float16 l = (_Float16)((c - (float)h) * 2048.0f);
    lev[tid] = (uint32_t)__builtin_bit_cast(uint16_t, h) |
               ((uint32_t)__builtin_bit_cast(uint16_t, l) << 16);
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
  for (int t = tid; t < a.G * D; t += blockDim.x) {
    const int g = t / D, i = t % D;
    float acc = 0.0f;
    for (int j = 0; j < D; ++j) acc += h2f(a.S[i * D + j]) * rq[g][j];
    sq[g][i] = acc * (kSqrtHalfPi / D);
  }
  __syncthreads();
  /* B operands, lane (n, kq), coordinates 32 s + 8 kq + 0..7: columns 0..7
   * the fp16 parts of query n, 8..15 their fp16 remainders (levels and sign
   * products); for the level remainders fp16(R q 2^-11) in columns 0..7 */
  half8 bl[KS], br[KS], bs[KS];
  {
    const int g = n & 7;
    const bool hiCol = n < 8, ok = g < a.G;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 32 * s + 8 * kq + j;
        const float r = ok ? rq[g][i] : 0.0f, z = ok ? sq[g][i] : 0.0f;
        const _Float16 rh = (_Float16)r, zh = (_Float16)z;
        bl[s][j] = hiCol ? rh : (_Float16)(r - (float)rh);
        br[s][j] = hiCol ? (_Float16)(r * 0x1p-11f) : (_Float16)0.0f;
        bs[s][j] = hiCol ? zh : (_Float16)(z - (float)zh);
      }
  }
  /* 16-key tiles, one per wave at a time: lane (m = n, kq) supplies key
   * k0 + m's coordinates 32 s + 8 kq + 0..7 of the A operands (levels, level
   * remainders, signs as +-1) */
  const int wave = tid / 64;
  const uint32_t cpy = (uint32_t)lane & 3u;
  const int64_t ntile = (a.T + 15) / 16;
  for (int64_t tile = (int64_t)blockIdx.x * 4 + wave; tile < ntile; tile += (int64_t)gridDim.x * 4) {
    const int64_t k0 = tile * 16, key = k0 + n;
    const bool live = key < a.T;
    const uint8_t* row = a.codes + (live ? key : 0) * (D * B / 8);
    const uint8_t* sg = a.signs + (live ? key : 0) * (D / 8);
    floatx4 c1 = {0.f, 0.f, 0.f, 0.f}, c2 = {0.f, 0.f, 0.f, 0.f};
    /* the key's sign bits in one go (d/8 bytes, 4-byte aligned) */
    uint32_t zw[D / 32];
#pragma unroll
    for (int k = 0; k < D / 32; ++k) zw[k] = live ? ((const uint32_t*)sg)[k] : 0u;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      /* the 8 codes at byte (32 s + 8 kq) B / 8 from aligned words (rows are
       * a multiple of 4 bytes, so the word holding the last byte ends inside
       * the row) */
      uint32_t cw = 0;
      if (live) {
        const int off = (32 * s + 8 * kq) * B / 8;
        const uint32_t* w = (const uint32_t*)(row + (off & ~3));
        if constexpr (B == 3)
          cw = (off & 3) + 3 > 4 ? __builtin_amdgcn_alignbit(w[1], w[0], (uint32_t)(off & 3) * 8u)
                                 : w[0] >> ((off & 3) * 8);
        else
          cw = w[0] >> ((off & 3) * 8);
      }
      const uint32_t zb = (zw[s] >> (8 * kq)) & 0xFFu;
      uint32_t e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = lev[((cw >> (B * j)) & ((1u << B) - 1)) * 4 + cpy];
      half8 ah, al, az;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ah[j] = __builtin_bit_cast(_Float16, (uint16_t)(e[j] & 0xFFFFu));
        al[j] = __builtin_bit_cast(_Float16, (uint16_t)(e[j] >> 16));
        az[j] = ((zb >> j) & 1) ? (_Float16)1.0f : (_Float16)-1.0f;
      }
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl[s], c1, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, br[s], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(az, bs[s], c2, 0, 0, 0);
    }
    /* lane (n, kq) holds keys k0 + 4 kq + i of column n; join the fp16
     * parts (column n + 8) into columns n < 8 */
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float m1 = c1[i] + ror8(c1[i]), m2 = c2[i] + ror8(c2[i]);
      const int64_t kk = k0 + 4 * kq + i;
      if (n < a.G && kk < a.T) {
        const float n16 = h2f(a.norms[kk]), g16 = h2f(a.gamma[kk]);
        a.out[n * a.T + kk] = n16 * (m1 + g16 * m2);
      }
    }
  }
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
  for (int k = 0; k < 16; ++k) a.levels[k] = k < (1 << cb->bits) ? cb->centroids[k] : 0.0f;
  int64_t blocks = (n + 63) / 64; /* 4 waves of 16 keys; capped, the waves then stride */
  if (blocks > 2048) blocks = 2048;
#define TQ_QE(DD, BB) \
  if (cb->d == DD && cb->bits == BB) \
    hipLaunchKernelGGL((qjl_encode_kernel<DD, BB>), dim3((unsigned)blocks), dim3(256), 0, s, a); else
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
  for (int k = 0; k < 16; ++k) a.levels[k] = k < (1 << cb->bits) ? cb->centroids[k] : 0.0f;
  int64_t blocks = (T + 63) / 64; /* 4 waves of 16 keys; capped, the waves then stride */
  if (blocks > 4096) blocks = 4096;
#define TQ_QS(DD, BB) \
  if (cb->d == DD && cb->bits == BB) \
    hipLaunchKernelGGL((qjl_scores_kernel<DD, BB>), dim3((unsigned)blocks), dim3(256), 0, s, a); else
  TQ_QS(64, 2) TQ_QS(64, 3) TQ_QS(64, 4) TQ_QS(128, 2) TQ_QS(128, 3) TQ_QS(128, 4)
  TQ_QS(256, 2) TQ_QS(256, 3) TQ_QS(256, 4) return TQ_ERR_UNSUPPORTED;
#undef TQ_QS
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}
