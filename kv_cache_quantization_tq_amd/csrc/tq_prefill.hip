/*
 * gfx950 prefill (extend) attention over the compressed cache: a chunk of new
 * query tokens, already appended to the cache, attends causally to the
 * sequence's cached tokens, reading the packed codes directly.
 *
 * Math (per layer, sequence, KV head; the G query heads of the group share
 * every dequantized tile), as in the decode step, one query at a time:
 *   q'' = H D q * log2(e) / (d * sigma_K)
 *   s_j = n_j * sum_i q''_i * (sigma_K c_K[code_ji])        (base-2 logits)
 *   online softmax in base 2 over j <= the query's position;
 *   o = D H (sum_j p_j m_j sigma_V c_V[code_j]) / (sqrt(d) sigma_V l)
 * ("We Built a Python Library That Cuts LLM Memory Usage by 80%", "Test
 * Suite": softmax(Q K^T / sqrt d) V; AdapTQ page, "How it works (HAR + VQ)",
 * step 3: queries rotated once and scored against the codebook levels; the
 * many-query case is the prefill the TurboQuant+ page times, "Paridad de
 * Velocidad Alcanzada".)
 *
 * With many queries per tile the products are dense contractions, so they run
 * on the matrix cores (v_mfma_f32_16x16x32_f16), and each 32-token tile is
 * dequantized once per block into LDS for all its queries:
 *   keys:   fp16 levels and fp16 remainders (level - fp16 level) * 2^11, token
 *           rows; S^T[16 tokens x 16 queries] = Khi Qhi + Khi Qlo + Klo Qrem,
 *           Qhi + Qlo = q'' split into fp16 parts, Qrem = fp16(q'' 2^-11),
 *           which carries the level to ~2^-22 (scores reach tens of nats);
 *   values: fp16 levels, coordinate rows with the tile's tokens in the order
 *           the score output leaves them in the lanes, so P^T feeds the value
 *           product without moving: O^T[16 coords x 16 queries] +=
 *           V^T[16 x 32 tokens] P'^T, P' = p * m_j split into two fp16 parts.
 * A block has 128 (head, query) columns: 128 / Gp queries of each of the G
 * heads (Gp = G rounded up to a power of two), 32 per wave (16 with 256-dim
 * heads), so that each operand read from LDS feeds two products.  Two LDS tile buffers:
 * while tile t is multiplied, tile t + 1 is dequantized into the other one
 * and tile t + 2's codes are loaded into registers (one barrier a tile).
 */
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tq_internal.h"

/* This source builds two units: by itself, the 128-dim kernels and the
 * entry point tq_launch_prefill, which hands other head dims to
 * tq_launch_prefill_other; with TQ_PREFILL_OTHER defined
 * (tq_prefill_other.hip), the 64- and 256-dim kernels behind that function.
 * The units are compiled with different scheduling options (the build
 * script's per-source flags). */
tq_status tq_launch_prefill_other(const tq_kv_cache* c, const tq_codebook_s* cbk,
                                  const tq_codebook_s* cbv, const uint8_t* sign_bits,
                                  const uint16_t* q, int q_heads, int t_new, const int32_t* pos,
                                  int n_layers, float* out, hipStream_t stream);

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kCols = 128; /* (head, query) columns per block */

/* 16-column groups per wave: two (each key and value operand read from LDS
 * feeds two products) unless the registers of 256-dim heads forbid it */
constexpr int groups_for(int d) { return d == 256 ? 1 : 2; }
constexpr int waves_for(int d) { return kCols / (16 * groups_for(d)); }

struct PreArgs {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint8_t* k_norms;
  const uint8_t* v_norms;
  int64_t ls_kc, ls_vc, ls_kn, ls_vn;
  int batch, kv_heads, capacity, q_heads, group, qc, t_new, chunks;
  const int32_t* block_table; /* paged storage: [batch][max_pages] */
  int lg_tpp, max_pages, num_pages;
  const uint8_t* sign_bits;
  const uint16_t* q;
  const int32_t* pos;
  const uint32_t* lut_k;    /* pair table: two fp16 levels per index */
  const uint32_t* lut_k_lo; /* pair table: two fp16 remainders * 2^11 */
  const uint32_t* lut_v;
  const uint32_t* lut_k1;   /* per code: fp16 level * 2^e | fp16 remainder << 16 */
  float qscale, oscale;
  float kscale;             /* 2^-e: key norms against the per-code table */
  float* out;
};

__device__ inline float h2f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

/* max / sum over the four 16-lane rows (lanes n, n+16, n+32, n+48) */
__device__ inline float rows_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float rows_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

/* max over all 64 lanes on the VALU: within each 16-lane row by DPP (quad
 * swaps, then rotations by 4 and 8), then across the rows */
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));  /* quad_perm [1, 0, 3, 2] */
  v = fmaxf(v, dpp_f<0x4E>(v));  /* quad_perm [2, 3, 0, 1] */
  v = fmaxf(v, dpp_f<0x124>(v)); /* row_ror:4 */
  v = fmaxf(v, dpp_f<0x128>(v)); /* row_ror:8 */
  return rows_max(v);
}

__device__ inline __amdgpu_buffer_rsrc_t make_stream(const uint8_t* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

/* The 8 codes (8 * B bits, little-endian) at byte offset off of a stream: two
 * aligned words and a funnel shift (bytes past the stream read as 0). */
template <int B>
__device__ inline uint32_t load_codes8(__amdgpu_buffer_rsrc_t rs, int32_t off) {
  const uint32_t a = (uint32_t)off & ~3u;
  const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(rs, a, 0, 0);
  if constexpr (B == 3) {
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(rs, a + 4, 0, 0);
    return __builtin_amdgcn_alignbit(hi, lo, (uint32_t)(off & 3) * 8u);
  } else {
    /* 2 or 4 bytes at an even offset: inside the aligned word */
    return lo >> ((off & 3) * 8);
  }
}

/* Walsh-Hadamard transform of one LDS row of D floats by one wave (lane l
 * holds coordinates l + 64 j on return). */
template <int D>
struct Row {
  float v[D >= 64 ? D / 64 : 1];
};
template <int D>
__device__ inline Row<D> row_fwht(const float* row, int lane) {
  constexpr int J = D / 64;
  Row<D> r;
#pragma unroll
  for (int j = 0; j < J; ++j) r.v[j] = row[lane + 64 * j];
#pragma unroll
  for (int hj = 1; hj < J; hj <<= 1)
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (!(j & hj)) {
        const float x = r.v[j], y = r.v[j | hj];
        r.v[j] = x + y;
        r.v[j | hj] = x - y;
      }
#pragma unroll
  for (int h = 1; h < 64; h <<= 1)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float y = __shfl_xor(r.v[j], h);
      r.v[j] = (lane & h) ? y - r.v[j] : r.v[j] + y;
    }
  return r;
}

template <int D, int BK, int BV>
struct PreGeo {
  static constexpr int RBK = D * BK / 8;        /* key row bytes */
  static constexpr int SEG = D * BV / 16;       /* value segment bytes */
  static constexpr int TILE_V = 32 * D * BV / 8;
  static constexpr int KP = D + 8;              /* key tile pitch (halfs) */
  static constexpr int VP = 32 + 8;             /* value tile pitch (halfs) */
  static constexpr int PWK = 1 << (2 * BK), PWV = 1 << (2 * BV); /* pair table words */
  static constexpr int ITEMS = 4 * D;           /* 8-code items per tile (keys; values too) */
  static constexpr int NG = groups_for(D), WAVES = waves_for(D);
  static constexpr int PER = (ITEMS + 64 * WAVES - 1) / (64 * WAVES);
  /* LDS: [query / output rows (fp32) | two tile buffers] union, then tables */
  static constexpr int QBYTES = kCols * D * 4;
  static constexpr int TBYTES = 2 * 32 * KP * 2 + D * VP * 2 + 2 * 32 * 4; /* one tile */
  static constexpr int UBYTES = QBYTES > 2 * TBYTES ? QBYTES : 2 * TBYTES;
  static constexpr int BYTES = UBYTES + (2 * PWK + PWV) * 4;
};

/* Token order of the value tile's k index (see the header): k = 8 kq + j holds
 * token 4 kq + j (j < 4) or 16 + 4 kq + j - 4. */
__device__ inline int kpos(int t) { return t < 16 ? 8 * (t >> 2) + (t & 3) : 8 * ((t - 16) >> 2) + 4 + (t & 3); }

template <int D, int BK, int BV, bool PAGED>
__global__ void __launch_bounds__(64 * waves_for(D)) prefill16_kernel(PreArgs a) {
  using PG = PreGeo<D, BK, BV>;
  constexpr int NG = PG::NG, KS = D / 32, VM = D / 16;
  __shared__ __align__(16) char smem[PG::BYTES];
  float* qbuf = (float*)smem;                            /* [kCols][D] */
  /* tile buffer u: khi [32][KP], klo [32][KP], vt [D][VP] (halfs), nk [32],
   * nv [32] (floats) */
  auto khi_of = [&](int u) { return (_Float16*)(smem + u * PG::TBYTES); };
  auto klo_of = [&](int u) { return khi_of(u) + 32 * PG::KP; };
  auto vt_of = [&](int u) { return khi_of(u) + 64 * PG::KP; };
  auto nk_of = [&](int u) { return (float*)(vt_of(u) + D * PG::VP); };
  auto nv_of = [&](int u) { return nk_of(u) + 32; };
  uint32_t* tk = (uint32_t*)(smem + PG::UBYTES);         /* key pairs, then remainders */
  uint32_t* tv = tk + 2 * PG::PWK;

  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int n = lane % 16, kq = lane / 16;
  const int chunk = blockIdx.x % a.chunks;
  int64_t unit = blockIdx.x / a.chunks;
  const int kv = (int)(unit % a.kv_heads);
  unit /= a.kv_heads;
  const int b = (int)(unit % a.batch);
  const int layer = (int)(unit / a.batch);
  const int q0 = chunk * a.qc;
  const int qn = (a.t_new - q0) < a.qc ? (a.t_new - q0) : a.qc; /* queries of this chunk */
  /* first query position, clamped to [0, capacity] (queries at or past
   * capacity attend the whole cache) */
  int p0 = a.pos[b];
  p0 = p0 < 0 ? 0 : (p0 > a.capacity ? a.capacity : p0);

  /* tables */
  for (int i = tid; i < PG::PWK; i += blockDim.x) {
    tk[i] = a.lut_k[i];
    tk[PG::PWK + i] = a.lut_k_lo[i];
  }
  for (int i = tid; i < PG::PWV; i += blockDim.x) tv[i] = a.lut_v[i];

  /* queries: column c = head g * qc + query i; q'' = H D q, scaled */
  const uint8_t* sb = a.sign_bits + (int64_t)layer * (D / 8);
  for (int t = tid; t < kCols * D; t += blockDim.x) {
    const int c = t / D, i = t % D;
    const int g = c / a.qc, qi = c % a.qc;
    float v = 0.0f;
    if (g < a.group && qi < qn) {
      const int64_t row = (((int64_t)layer * a.batch + b) * a.q_heads + (int64_t)kv * a.group + g) *
                              a.t_new + q0 + qi;
      v = h2f(a.q[row * D + i]);
      v = ((sb[i >> 3] >> (i & 7)) & 1) ? -v : v;
    }
    qbuf[t] = v;
  }
  __syncthreads();
  /* wave w owns columns 16 NG w .. 16 NG w + 16 NG - 1 */
  const int c0 = 16 * NG * wave;
  for (int r = 0; r < 16 * NG; ++r) {
    float* row = qbuf + (c0 + r) * D;
    const Row<D> t = row_fwht<D>(row, lane);
#pragma unroll
    for (int j = 0; j < D / 64; ++j) row[lane + 64 * j] = t.v[j] * a.qscale;
  }
  __syncthreads();
  /* B operands: lane (n, kq) of group e holds coordinates 32 s + 8 kq + 0..7
   * of column c0 + 16 e + n: fp16 part, fp16 remainder, fp16(q'' 2^-11) */
  half8 qhi[NG][KS], qlo[NG][KS], qrm[NG][KS];
#pragma unroll
  for (int e = 0; e < NG; ++e) {
    const float* row = qbuf + (c0 + 16 * e + n) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = row[32 * s + 8 * kq + j];
        const _Float16 h = (_Float16)v;
        qhi[e][s][j] = h;
        qlo[e][s][j] = (_Float16)(v - (float)h);
        qrm[e][s][j] = (_Float16)(v * 0x1p-11f);
      }
  }
  /* the lane's columns: causal limits (tokens < lim are attended) */
  int lim[NG];
#pragma unroll
  for (int e = 0; e < NG; ++e) {
    const int col = c0 + 16 * e + n;
    const int cg = col / a.qc, ci = col % a.qc;
    const int64_t l = (int64_t)p0 + q0 + ci + 1;
    lim[e] = (cg < a.group && ci < qn) ? (int)(l > a.capacity ? a.capacity : l)
                                       : 1; /* padding columns attend token 0 only */
  }
  const int64_t blk_end = (int64_t)p0 + q0 + qn;
  const int blk_lim = (int)(blk_end > a.capacity ? a.capacity : blk_end);
  const int ntiles = (blk_lim + 31) / 32;
  __syncthreads(); /* qbuf is dead: the tiles take its place */

  /* streams of this (layer, sequence, head), or of the layer's page pool */
  const int64_t sh = PAGED ? 0 : (int64_t)b * a.kv_heads + kv;
  const int64_t srows = PAGED ? (int64_t)a.num_pages * a.kv_heads * (32 << a.lg_tpp) : a.capacity;
  const __amdgpu_buffer_rsrc_t rk =
      make_stream(a.k_codes + layer * a.ls_kc + sh * a.capacity * PG::RBK, srows * PG::RBK);
  const __amdgpu_buffer_rsrc_t rv = make_stream(
      a.v_codes + layer * a.ls_vc + sh * (a.capacity / 32) * PG::TILE_V, srows / 32 * PG::TILE_V);
  const __amdgpu_buffer_rsrc_t rkn = make_stream(a.k_norms + layer * a.ls_kn + sh * a.capacity * 2, srows * 2);
  const __amdgpu_buffer_rsrc_t rvn = make_stream(a.v_norms + layer * a.ls_vn + sh * a.capacity * 2, srows * 2);
  /* tile t's first row in the streams (value tiles: that / 32) */
  auto tile_rows = [&](int t) -> int32_t {
    if constexpr (PAGED) {
      const int tpp = 1 << a.lg_tpp;
      int phys = a.block_table[(int64_t)b * a.max_pages + (t >> a.lg_tpp)];
      phys = phys < 0 ? 0 : (phys >= a.num_pages ? a.num_pages - 1 : phys);
      return (phys * a.kv_heads + kv) * (tpp * 32) + (t & (tpp - 1)) * 32;
    } else {
      return t * 32;
    }
  };

  /* raw codes of one tile, per thread: PER key items and PER value items */
  uint32_t kraw[PG::PER], vraw[PG::PER], nraw = 0;
  auto fetch = [&](int t) {
    const int32_t r0 = tile_rows(t);
#pragma unroll
    for (int u = 0; u < PG::PER; ++u) {
      const int it = tid + u * 64 * PG::WAVES;
      kraw[u] = 0;
      vraw[u] = 0;
      if (it < PG::ITEMS) {
        const int tok = it / (D / 8), grp = it % (D / 8);
        kraw[u] = load_codes8<BK>(rk, (r0 + tok) * PG::RBK + grp * BK);
        const int seg = it / (D / 16), m = it % (D / 16);
        vraw[u] = load_codes8<BV>(rv, (r0 / 32) * PG::TILE_V + seg * PG::SEG + m * BV);
      }
    }
    if (tid < 32)
      nraw = __builtin_amdgcn_raw_buffer_load_b16(rkn, (uint32_t)(r0 + tid) * 2u, 0, 0);
    else if (tid < 64)
      nraw = __builtin_amdgcn_raw_buffer_load_b16(rvn, (uint32_t)(r0 + tid - 32) * 2u, 0, 0);
  };
  /* dequantize the fetched tile into LDS buffer u */
  auto spill = [&](int u) {
    _Float16* khi = khi_of(u);
    _Float16* klo = klo_of(u);
    _Float16* vt = vt_of(u);
    float* nk = nk_of(u);
    float* nv = nv_of(u);
#pragma unroll
    for (int w = 0; w < PG::PER; ++w) {
      const int it = tid + w * 64 * PG::WAVES;
      if (it < PG::ITEMS) {
        const int tok = it / (D / 8), grp = it % (D / 8);
        u32x4 h, l;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t e = (kraw[w] >> (2 * BK * p)) & (PG::PWK - 1);
          h[p] = tk[e];
          l[p] = tk[PG::PWK + e];
        }
        *(u32x4*)(khi + tok * PG::KP + 8 * grp) = h;
        *(u32x4*)(klo + tok * PG::KP + 8 * grp) = l;
        /* value segment seg = 16 q + r, field m: coordinate r (d/16) + m of
         * tokens 8 q + 0..7, pairs of consecutive tokens adjacent in kpos */
        const int seg = it / (D / 16), m = it % (D / 16);
        const int qq = seg >> 4, rr = seg & 15;
        _Float16* vrow = vt + (rr * (D / 16) + m) * PG::VP;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t e = (vraw[w] >> (2 * BV * p)) & (PG::PWV - 1);
          *(uint32_t*)(vrow + kpos(8 * qq + 2 * p)) = tv[e];
        }
      }
    }
    if (tid < 32) nk[tid] = h2f(nraw);
    else if (tid < 64) nv[tid - 32] = h2f(nraw);
  };

  floatx4 acc[NG][VM];
#pragma unroll
  for (int e = 0; e < NG; ++e)
#pragma unroll
    for (int m = 0; m < VM; ++m) acc[e][m] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run[NG], l_run[NG];
#pragma unroll
  for (int e = 0; e < NG; ++e) {
    m_run[e] = -INFINITY;
    l_run[e] = 0.0f;
  }

  /* tile t is multiplied from buffer t % 2 while tile t + 1 is dequantized
   * into the other one and tile t + 2's codes are loaded: one barrier a tile */
  fetch(0);
  spill(0);
  if (ntiles > 1) fetch(1);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int u = t & 1;
    const _Float16* khi = khi_of(u);
    const _Float16* klo = klo_of(u);
    const _Float16* vt = vt_of(u);
    const float* nk = nk_of(u);
    const float* nv = nv_of(u);
    if (t + 1 < ntiles) {
      spill(u ^ 1);
      if (t + 2 < ntiles) fetch(t + 2);
    }
    /* scores of the two 16-token halves, every key operand read once for the
     * NG column groups */
    floatx4 s[NG][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int e = 0; e < NG; ++e) s[e][h] = floatx4{0.f, 0.f, 0.f, 0.f};
      const _Float16* kr = khi + (16 * h + n) * PG::KP + 8 * kq;
      const _Float16* kl = klo + (16 * h + n) * PG::KP + 8 * kq;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const half8 ah = *(const half8*)(kr + 32 * ks);
        const half8 al = *(const half8*)(kl + 32 * ks);
#pragma unroll
        for (int e = 0; e < NG; ++e) {
          s[e][h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, qhi[e][ks], s[e][h], 0, 0, 0);
          s[e][h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, qlo[e][ks], s[e][h], 0, 0, 0);
          s[e][h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, qrm[e][ks], s[e][h], 0, 0, 0);
        }
      }
    }
    /* lane (n, kq) holds tokens 16 h + 4 kq + i of its columns */
    float nkv[8], nvv[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        nkv[4 * h + i] = nk[16 * h + 4 * kq + i];
        nvv[4 * h + i] = nv[16 * h + 4 * kq + i];
      }
    const int tok0 = 32 * t;
    const bool edge = tok0 + 32 > p0 + q0 + 1; /* some column may stop inside */
    half8 ph[NG], pl[NG];
#pragma unroll
    for (int e = 0; e < NG; ++e) {
      float sc[8];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tt = 16 * h + 4 * kq + i;
          float v = s[e][h][i] * nkv[4 * h + i];
          if (edge && tok0 + tt >= lim[e]) v = -INFINITY;
          sc[4 * h + i] = v;
        }
      float mt = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sc[i]);
      mt = rows_max(mt);
      if (__any(mt > m_run[e])) {
        const float mn = fmaxf(m_run[e], mt);
        const float al = __builtin_amdgcn_exp2f(m_run[e] - mn); /* 0 on the first tile */
        l_run[e] *= al;
#pragma unroll
        for (int m = 0; m < VM; ++m) acc[e][m] *= al;
        m_run[e] = mn;
      }
      /* P' = p m_j as fp16 parts, in the value product's k order */
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(sc[j] - m_run[e]);
        l_run[e] += p;
        /* fp16(p m) and the fp16 of the exact remainder p m - fp16(p m), one
         * mixed-precision FMA each */
        const _Float16 hh = (_Float16)__builtin_fmaf(p, nvv[j], 0.0f);
        ph[e][j] = hh;
        pl[e][j] = (_Float16)__builtin_fmaf(p, nvv[j], -(float)hh);
      }
    }
#pragma unroll
    for (int m = 0; m < VM; ++m) {
      const half8 av = *(const half8*)(vt + (16 * m + n) * PG::VP + 8 * kq);
#pragma unroll
      for (int e = 0; e < NG; ++e) {
        acc[e][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, ph[e], acc[e][m], 0, 0, 0);
        acc[e][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pl[e], acc[e][m], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  /* column sums over the four lane groups, then o'' = acc / l into LDS rows */
  float* obuf = qbuf;
#pragma unroll
  for (int e = 0; e < NG; ++e) {
    const float inv = a.oscale / rows_sum(l_run[e]);
    const int col = c0 + 16 * e + n;
#pragma unroll
    for (int m = 0; m < VM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) obuf[col * D + 16 * m + 4 * kq + i] = acc[e][m][i] * inv;
  }
  __syncthreads();
  /* o = D H o'': one wave per row of its columns */
  for (int r = 0; r < 16 * NG; ++r) {
    const int c = c0 + r;
    const int g = c / a.qc, qi = c % a.qc;
    const Row<D> t = row_fwht<D>(obuf + c * D, lane);
    if (g < a.group && qi < qn) {
      const int64_t row = (((int64_t)layer * a.batch + b) * a.q_heads + (int64_t)kv * a.group + g) *
                              a.t_new + q0 + qi;
#pragma unroll
      for (int j = 0; j < D / 64; ++j) {
        const int i = lane + 64 * j;
        const float v = t.v[j];
        a.out[row * D + i] = ((sb[i >> 3] >> (i & 7)) & 1) ? -v : v;
      }
    }
  }
}

/* ------------------------------------------------ 32 x 32 product form -- */

/* Heads of 64 and 128 coordinates: v_mfma_f32_32x32x16_f16, one wave per 32
 * (head, query) columns, so that a lane holds 16 of the 32 scores of one
 * column (the other 16 sit in lane l ^ 32).  Operand layouts (lane l, h =
 * l / 32): A[l % 32][8 h + j], B[8 h + j][l % 32], j < 8; the result C[8 (r
 * / 4) + 4 h + r % 4][l % 32], r < 16.
 *
 * Precision with fewer products than the 16-wide form:
 *   keys:   level v = hi + lo, hi = fp16(v), lo = fp16(v - hi) (levels
 *           scaled by 2^e so that lo stays far above fp16's absolute step,
 *           2^-e folded into the key norms: the query keeps its own scale,
 *           so its small coordinates do not become subnormal); query q = qh
 *           + ql in fp16 parts; S^T = Khi Qh + Klo Qh + Khi Ql (the dropped
 *           Klo Ql is ~2^-22 of the score);
 *   values: P' = p m / 2^E as fp16 part and fp16 remainder, two products
 *           with the value levels as the codebook's fp16 table (its scale
 *           minimises their rounding); E is the running maximum of the
 *           value-norm exponents, so P' <= 2 and the remainders of the
 *           weights that matter stay far above fp16's absolute step; the
 *           accumulator is rescaled when E grows, like the softmax maximum.
 * The value tile's k index follows the score layout: in each 16-token step,
 * k = 8 h + j holds token 4 h + (j % 4) + 8 (j / 4), so the P' registers feed
 * the value product as they are.
 *
 * Coordinates live in the lanes the way the value product leaves them: lane
 * (c, h) holds coordinates 32 m + 8 r + 4 h + i (r, i < 4) of column c.  The
 * query is loaded in that layout and both rotations (q'' = H D q, o = D H o'')
 * run in registers: butterflies within the lane for coordinate bits 0, 1 and
 * 3 and up, one exchange with lane l ^ 32 for bit 2.  The score product's k
 * index is the same permutation of the coordinates (step s, k = 8 h + j:
 * coordinate 32 (s / 2) + 8 (2 (s % 2) + j / 4) + 4 h + j % 4), so the key
 * rows are stored in that order.  With no fp32 query or output rows in LDS,
 * a block needs only its two tile buffers and the code tables (~51 KB at
 * d = 128); the registers (the accumulators and the query's two fp16 parts
 * alone take 128) hold the kernel at two waves per SIMD. */
constexpr int kWaves32 = 4;
constexpr float kLazy = 8.0f; /* base-2 slack of the softmax reference */

template <int D, int BK, int BV>
struct Geo32 {
  static_assert(D == 64 || D == 128, "32 x 32 form: heads of 64 or 128 coordinates");
  static constexpr int RBK = D * BK / 8;
  static constexpr int SEG = D * BV / 16;
  static constexpr int TILE_V = 32 * D * BV / 8;
  static constexpr int LK = 1 << BK, PWV = 1 << (2 * BV);
  static constexpr int ITEMS = 4 * D; /* 8-code items per tile, keys and values alike */
  static constexpr int PER = ITEMS / (64 * kWaves32);
  static constexpr int KP = D + 8; /* key row pitch (halfs): rows 16 bytes apart in the banks */
  /* one tile: khi, klo [32][KP], vt [4][D][8] (halfs: chunk k holds k-index
   * 8 k..8 k+7 of every coordinate row), nk, nv [32], E */
  static constexpr int TBYTES = 2 * 32 * KP * 2 + D * 32 * 2 + 2 * 32 * 4 + 16;
  static constexpr int BYTES = 2 * TBYTES + (LK + PWV) * 4;
};

/* Bank spread of the LDS tiles (64 banks of 4 bytes; a 16-byte read serves
 * 16 lanes per cycle, the 16 lanes of a half-wave reading rows 0..15 of one
 * 16-byte chunk): key rows are padded by one chunk, and the value tile is
 * stored chunk-major, so that those 16 reads are consecutive; the addresses
 * of every step stay constant offsets from one register. */

/* max over the lane pair (l, l ^ 32) */
__device__ inline float pair_max(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ inline float pair_sum(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

/* Unnormalised Walsh-Hadamard transform of one column held by a lane pair:
 * x[16 m + 4 r + i] is coordinate 32 m + 8 r + 4 h + i, h = lane / 32. */
template <int N>
__device__ inline void pair_fwht(float (&x)[N], int hh) {
#pragma unroll
  for (int b = 1; b < N; b <<= 1)
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (!(k & b)) {
        const float u = x[k], w = x[k | b];
        x[k] = u + w;
        x[k | b] = u - w;
      }
  /* coordinate bit 2: lane l < 32 holds the first of each pair */
  const float sg = hh ? -1.0f : 1.0f;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[k]), __float_as_uint(x[k]), false, false);
    x[k] = __builtin_fmaf(sg, __uint_as_float(p[1]), __uint_as_float(p[0]));
  }
}

template <int D, int BK, int BV, bool PAGED>
__global__ void __launch_bounds__(64 * kWaves32) prefill32_kernel(PreArgs a) {
  using PG = Geo32<D, BK, BV>;
  constexpr int KS = D / 16, VM = D / 32, NX = D / 2;
  __shared__ __align__(16) char smem[PG::BYTES];
  auto khi_of = [&](int u) { return (_Float16*)(smem + u * PG::TBYTES); };
  auto klo_of = [&](int u) { return khi_of(u) + 32 * PG::KP; };
  auto vt_of = [&](int u) { return khi_of(u) + 64 * PG::KP; };
  auto nk_of = [&](int u) { return (float*)(vt_of(u) + D * 32); };
  auto nv_of = [&](int u) { return nk_of(u) + 32; };
  auto ev_of = [&](int u) { return (int*)(nk_of(u) + 64); };
  uint32_t* tk = (uint32_t*)(smem + 2 * PG::TBYTES); /* per code: hi | lo << 16 */
  uint32_t* tv = tk + PG::LK;                        /* per pair of codes: two fp16 levels */

  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int cl = lane % 32, hh = lane / 32;
  const int chunk = blockIdx.x % a.chunks;
  int64_t unit = blockIdx.x / a.chunks;
  const int kv = (int)(unit % a.kv_heads);
  unit /= a.kv_heads;
  const int b = (int)(unit % a.batch);
  const int layer = (int)(unit / a.batch);
  const int q0 = chunk * a.qc;
  const int qn = (a.t_new - q0) < a.qc ? (a.t_new - q0) : a.qc;
  int p0 = a.pos[b];
  p0 = p0 < 0 ? 0 : (p0 > a.capacity ? a.capacity : p0);

  for (int i = tid; i < PG::LK; i += blockDim.x) tk[i] = a.lut_k1[i];
  for (int i = tid; i < PG::PWV; i += blockDim.x) tv[i] = a.lut_v[i];

  /* the lane's column c = head g * qc + query i; padding columns (no such
   * head or query) hold zeros and are not written */
  const int c0 = 32 * wave;
  const int col = c0 + cl;
  const int cg = col / a.qc, ci = col % a.qc;
  const bool real = cg < a.group && ci < qn;
  const int64_t orow =
      (((int64_t)layer * a.batch + b) * a.q_heads + (int64_t)kv * a.group + (real ? cg : 0)) * a.t_new +
      q0 + (real ? ci : 0);
  const uint8_t* sb = a.sign_bits + (int64_t)layer * (D / 8);

  /* q'' = H D q, scaled, split into the B operands: lane (cl, hh) of step s
   * holds coordinates 32 (s / 2) + 8 (2 (s % 2) + j / 4) + 4 hh + j % 4 */
  half8 qh[KS], ql[KS];
  {
    float x[NX];
    const uint16_t* qr = a.q + orow * D + 4 * hh;
#pragma unroll
    for (int m = 0; m < VM; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint2 w = make_uint2(0u, 0u);
        if (real) w = *(const uint2*)(qr + 32 * m + 8 * r);
        const uint32_t sgn = __builtin_amdgcn_readfirstlane((uint32_t)sb[4 * m + r]) >> (4 * hh);
        const uint32_t h4[4] = {w.x & 0xffffu, w.x >> 16, w.y & 0xffffu, w.y >> 16};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = h2f(h4[i]);
          x[16 * m + 4 * r + i] = ((sgn >> i) & 1) ? -v : v;
        }
      }
    pair_fwht(x, hh);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = x[16 * (s >> 1) + 8 * (s & 1) + j] * a.qscale;
        const _Float16 h = (_Float16)v;
        qh[s][j] = h;
        ql[s][j] = (_Float16)(v - (float)h);
      }
  }
  /* causal limit of the lane's column (tokens < lim are attended) */
  int lim;
  {
    const int64_t l = (int64_t)p0 + q0 + ci + 1;
    lim = real ? (int)(l > a.capacity ? a.capacity : l) : 1;
  }
  const int64_t blk_end = (int64_t)p0 + q0 + qn;
  const int blk_lim = (int)(blk_end > a.capacity ? a.capacity : blk_end);
  const int ntiles = (blk_lim + 31) / 32;
  __syncthreads(); /* the code tables are in place */

  const int64_t sh = PAGED ? 0 : (int64_t)b * a.kv_heads + kv;
  const int64_t srows = PAGED ? (int64_t)a.num_pages * a.kv_heads * (32 << a.lg_tpp) : a.capacity;
  const __amdgpu_buffer_rsrc_t rk =
      make_stream(a.k_codes + layer * a.ls_kc + sh * a.capacity * PG::RBK, srows * PG::RBK);
  const __amdgpu_buffer_rsrc_t rv = make_stream(
      a.v_codes + layer * a.ls_vc + sh * (a.capacity / 32) * PG::TILE_V, srows / 32 * PG::TILE_V);
  const __amdgpu_buffer_rsrc_t rkn = make_stream(a.k_norms + layer * a.ls_kn + sh * a.capacity * 2, srows * 2);
  const __amdgpu_buffer_rsrc_t rvn = make_stream(a.v_norms + layer * a.ls_vn + sh * a.capacity * 2, srows * 2);
  auto tile_rows = [&](int t) -> int32_t {
    if constexpr (PAGED) {
      const int tpp = 1 << a.lg_tpp;
      int phys = a.block_table[(int64_t)b * a.max_pages + (t >> a.lg_tpp)];
      phys = phys < 0 ? 0 : (phys >= a.num_pages ? a.num_pages - 1 : phys);
      return (phys * a.kv_heads + kv) * (tpp * 32) + (t & (tpp - 1)) * 32;
    } else {
      return t * 32;
    }
  };

  /* raw codes of one tile: PER key items and PER value items per thread
   * (with two value items, the pair q = 2 j, 2 j + 1 of one coordinate row,
   * so that the thread's stores fill whole 16-byte chunks); threads 0..31
   * load the key norms, 32..63 the value norms */
  constexpr bool VPAIR = PG::PER == 2;
  auto vitem = [&](int u) {
    return VPAIR ? (tid & 127) + 256 * (tid >> 7) + 128 * u : tid + u * 64 * kWaves32;
  };
  uint32_t kraw[PG::PER], vraw[PG::PER], nraw = 0;
  auto fetch = [&](int t) {
    const int32_t r0 = tile_rows(t);
#pragma unroll
    for (int u = 0; u < PG::PER; ++u) {
      const int it = tid + u * 64 * kWaves32;
      const int tok = it / (D / 8), grp = it % (D / 8);
      kraw[u] = load_codes8<BK>(rk, (r0 + tok) * PG::RBK + grp * BK);
      const int iv = vitem(u);
      const int seg = iv / (D / 16), m = iv % (D / 16);
      vraw[u] = load_codes8<BV>(rv, (r0 / 32) * PG::TILE_V + seg * PG::SEG + m * BV);
    }
    if (tid < 32)
      nraw = __builtin_amdgcn_raw_buffer_load_b16(rkn, (uint32_t)(r0 + tid) * 2u, 0, 0);
    else if (tid < 64)
      nraw = __builtin_amdgcn_raw_buffer_load_b16(rvn, (uint32_t)(r0 + tid - 32) * 2u, 0, 0);
  };
  /* running value-norm exponent (meaningful in wave 0) */
  int e_run = -25;
  auto spill = [&](int u) {
    _Float16* khi = khi_of(u);
    _Float16* klo = klo_of(u);
    _Float16* vt = vt_of(u);
#pragma unroll
    for (int w = 0; w < PG::PER; ++w) {
      const int it = tid + w * 64 * kWaves32;
      const int tok = it / (D / 8), grp = it % (D / 8);
      uint32_t e[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) e[p] = tk[(kraw[w] >> (BK * p)) & (PG::LK - 1)];
      uint32_t hv[4], lv[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        hv[p] = __builtin_amdgcn_perm(e[2 * p + 1], e[2 * p], 0x05040100u);
        lv[p] = __builtin_amdgcn_perm(e[2 * p + 1], e[2 * p], 0x07060302u);
      }
      /* coordinates 8 grp + 0..3 and + 4..7 (m = grp / 4, r = grp % 4) go to
       * row positions 32 m + 16 (r / 2) + 4 (r % 2) and 8 further on */
      const int pos = 32 * (grp >> 2) + 16 * ((grp >> 1) & 1) + 4 * (grp & 1);
      _Float16* kh = khi + tok * PG::KP + pos;
      _Float16* kl = klo + tok * PG::KP + pos;
      *(uint2*)kh = make_uint2(hv[0], hv[1]);
      *(uint2*)(kh + 8) = make_uint2(hv[2], hv[3]);
      *(uint2*)kl = make_uint2(lv[0], lv[1]);
      *(uint2*)(kl + 8) = make_uint2(lv[2], lv[3]);
    }
    /* value segment seg = 16 q + r, field m: coordinate r (d/16) + m of
     * tokens 8 q + 0..7; tokens 8 q + 0..3 and 8 q + 4..7 are runs of 4 in
     * the row's k order (chunks 2 (q / 2) and 2 (q / 2) + 1, at 4 (q % 2)) */
    uint32_t pv[PG::PER][4];
#pragma unroll
    for (int w = 0; w < PG::PER; ++w)
#pragma unroll
      for (int p = 0; p < 4; ++p) pv[w][p] = tv[(vraw[w] >> (2 * BV * p)) & (PG::PWV - 1)];
    if constexpr (VPAIR) {
      const int iv = vitem(0);
      const int seg = iv / (D / 16), m = iv % (D / 16);
      const int vrow = (seg & 15) * (D / 16) + m;
      _Float16* vr = vt + (2 * (seg >> 5) * D + vrow) * 8;
      *(u32x4*)vr = u32x4{pv[0][0], pv[0][1], pv[1][0], pv[1][1]};
      *(u32x4*)(vr + 8 * D) = u32x4{pv[0][2], pv[0][3], pv[1][2], pv[1][3]};
    } else {
#pragma unroll
      for (int w = 0; w < PG::PER; ++w) {
        const int iv = vitem(w);
        const int seg = iv / (D / 16), m = iv % (D / 16);
        const int qq = seg >> 4, rr = seg & 15;
        const int vrow = rr * (D / 16) + m;
        _Float16* vr = vt + (2 * (qq >> 1) * D + vrow) * 8 + 4 * (qq & 1);
        *(uint2*)vr = make_uint2(pv[w][0], pv[w][1]);
        *(uint2*)(vr + 8 * D) = make_uint2(pv[w][2], pv[w][3]);
      }
    }
    /* norms; the value norms scaled by 2^-E, E the running maximum of the
     * tiles' largest value-norm exponents */
    if (wave == 0) {
      const float nf = h2f(nraw);
      const float mx = wave_max(tid >= 32 ? nf : 0.0f);
      const int et = ((int)(__float_as_uint(mx) >> 23) & 255) - 127;
      e_run = et > e_run ? et : e_run;
      if (tid < 32) nk_of(u)[tid] = nf * a.kscale;
      else nv_of(u)[tid - 32] = __builtin_ldexpf(nf, -e_run);
      if (tid == 32) *ev_of(u) = e_run;
    }
  };

  floatx16 acc[VM];
#pragma unroll
  for (int m = 0; m < VM; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  int e_cur = -25;

  /* tile t is multiplied from buffer t % 2 while tile t + 1 is dequantized
   * into the other one and tile t + 2's codes are loaded (past the last
   * tile, the last tile again): one barrier a tile */
  fetch(0);
  spill(0);
  fetch(ntiles > 1 ? 1 : 0);
  __syncthreads();
  /* tiles below t_edge end at or before every real column's first query
   * (padding columns attend token 0 only, but their outputs are not
   * written, so they need no mask there either) */
  const int t_edge = (p0 + q0 + 1) / 32 < ntiles ? (p0 + q0 + 1) / 32 : ntiles;
  auto step = [&](const int t, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const int u = t & 1;
    const _Float16* khi = khi_of(u);
    const _Float16* klo = klo_of(u);
    const _Float16* vt = vt_of(u);
    const float* nk = nk_of(u);
    const float* nv = nv_of(u);
    const int et = *ev_of(u);
    floatx16 S;
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = 0.0f;
    const _Float16* kr = khi + cl * PG::KP + 8 * hh;
    const _Float16* kl = klo + cl * PG::KP + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const half8 ah = *(const half8*)(kr + 16 * ks);
      const half8 al = *(const half8*)(kl + 16 * ks);
      S = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, qh[ks], S, 0, 0, 0);
      S = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, qh[ks], S, 0, 0, 0);
      S = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, ql[ks], S, 0, 0, 0);
    }
    spill(u ^ 1);
    fetch(t + 2 < ntiles ? t + 2 : ntiles - 1);
    /* S[r]: token 8 (r / 4) + 4 hh + r % 4 of the lane's column */
    float mt = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 a4 = *(const float4*)(nk + 8 * q + 4 * hh);
      const float n4[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = S[4 * q + i] * n4[i];
        if (EDGE && 32 * t + 8 * q + 4 * hh + i >= lim) v = -INFINITY;
        S[4 * q + i] = v;
        mt = fmaxf(mt, v);
      }
    }
    mt = pair_max(mt);
    /* One rescale for both running scales, and only when needed: the
     * softmax reference m_run moves only when a column's maximum passes it
     * by more than kLazy (so p = 2^(s - m_run) <= 2^kLazy: the products
     * are the same up to the common factor, which l_run carries too), and
     * E moves when a tile brings a larger value-norm exponent (uniform). */
    const bool grow = mt > m_run + kLazy;
    if (__any(grow) || et > e_cur) {
      const float mn = grow ? mt : m_run;
      float al = __builtin_amdgcn_exp2f(m_run - mn); /* 0 on the first tile */
      l_run *= al;
      if (et > e_cur) al = __builtin_ldexpf(al, e_cur - et);
#pragma unroll
      for (int m = 0; m < VM; ++m) acc[m] *= al;
      m_run = mn;
      e_cur = et > e_cur ? et : e_cur;
    }
    half8 ph[2], pl[2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 b4 = *(const float4*)(nv + 8 * q + 4 * hh);
      const float n4[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * q + i;
        const float p = __builtin_amdgcn_exp2f(S[r] - m_run);
        l_run += p;
        /* fp16(p m) and the fp16 of the exact remainder, one fma each */
        const _Float16 h = (_Float16)__builtin_fmaf(p, n4[i], 0.0f);
        ph[r >> 3][r & 7] = h;
        pl[r >> 3][r & 7] = (_Float16)__builtin_fmaf(p, n4[i], -(float)h);
      }
    }
#pragma unroll
    for (int m = 0; m < VM; ++m) {
      const _Float16* vr = vt + (hh * D + 32 * m + cl) * 8;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const half8 av = *(const half8*)(vr + 16 * k * D);
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, ph[k], acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pl[k], acc[m], 0, 0, 0);
      }
    }
    __syncthreads();
  };
  int t = 0;
  for (; t < t_edge; ++t) step(t, std::false_type{});
  for (; t < ntiles; ++t) step(t, std::true_type{});

  /* o = D H (acc 2^E / l), the lane's coordinates written as runs of 4 */
  {
    const float inv = __builtin_ldexpf(a.oscale, e_cur) / pair_sum(l_run);
    float x[NX];
#pragma unroll
    for (int m = 0; m < VM; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[16 * m + r] = acc[m][r] * inv;
    pair_fwht(x, hh);
    if (real) {
      float* orp = a.out + orow * D + 4 * hh;
#pragma unroll
      for (int m = 0; m < VM; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t sgn = __builtin_amdgcn_readfirstlane((uint32_t)sb[4 * m + r]) >> (4 * hh);
          float o4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = x[16 * m + 4 * r + i];
            o4[i] = ((sgn >> i) & 1) ? -v : v;
          }
          *(float4*)(orp + 32 * m + 8 * r) = make_float4(o4[0], o4[1], o4[2], o4[3]);
        }
    }
  }
}

template <int D, int BK, int BV>
tq_status launch_prefill_t(const PreArgs& a, int64_t blocks, hipStream_t s) {
  const dim3 grid((unsigned)blocks);
  if constexpr (D == 256) {
    if (a.block_table)
      hipLaunchKernelGGL((prefill16_kernel<D, BK, BV, true>), grid, dim3(64 * waves_for(D)), 0, s, a);
    else
      hipLaunchKernelGGL((prefill16_kernel<D, BK, BV, false>), grid, dim3(64 * waves_for(D)), 0, s, a);
  } else {
    if (a.block_table)
      hipLaunchKernelGGL((prefill32_kernel<D, BK, BV, true>), grid, dim3(64 * kWaves32), 0, s, a);
    else
      hipLaunchKernelGGL((prefill32_kernel<D, BK, BV, false>), grid, dim3(64 * kWaves32), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

}  // namespace

#ifndef TQ_PREFILL_OTHER
tq_status tq_launch_prefill(const tq_kv_cache* c, const tq_codebook_s* cbk,
                            const tq_codebook_s* cbv, const uint8_t* sign_bits,
                            const uint16_t* q, int q_heads, int t_new, const int32_t* pos,
                            int n_layers, float* out, hipStream_t s) {
#else
tq_status tq_launch_prefill_other(const tq_kv_cache* c, const tq_codebook_s* cbk,
                                  const tq_codebook_s* cbv, const uint8_t* sign_bits,
                                  const uint16_t* q, int q_heads, int t_new, const int32_t* pos,
                                  int n_layers, float* out, hipStream_t s) {
#endif
  PreArgs a;
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
  int gp = 1;
  while (gp < a.group) gp *= 2;
  a.qc = kCols / gp;
  a.t_new = t_new;
  a.chunks = (t_new + a.qc - 1) / a.qc;
  a.block_table = c->block_table;
  a.lg_tpp = 0;
  if (c->block_table)
    while ((32 << a.lg_tpp) < c->page_tokens) ++a.lg_tpp;
  a.max_pages = c->block_table ? c->max_pages : 0;
  a.num_pages = c->block_table ? c->num_pages : 0;
  a.sign_bits = sign_bits;
  a.q = q;
  a.pos = pos;
  a.lut_k = cbk->dec_lut;
  a.lut_k_lo = cbk->dec_lut_lo;
  a.lut_v = cbv->dec_lut;
  a.lut_k1 = cbk->pre_klut;
  const double d = c->head_dim;
  a.qscale = (float)(1.4426950408889634 / (d * cbk->sigma));
  a.kscale = (float)ldexp(1.0, -cbk->pre_exp);
  a.oscale = (float)(1.0 / (sqrt(d) * cbv->sigma));
  a.out = out;
  const int64_t blocks = (int64_t)n_layers * c->batch * c->kv_heads * a.chunks;
  if (blocks == 0) return TQ_OK;
#define TQ_PRE(DD, KK, VV) \
  if (c->head_dim == DD && c->bits_k == KK && c->bits_v == VV) return launch_prefill_t<DD, KK, VV>(a, blocks, s);
#define TQ_PRE_D(DD) \
  TQ_PRE(DD, 2, 2) TQ_PRE(DD, 2, 3) TQ_PRE(DD, 2, 4) TQ_PRE(DD, 3, 2) TQ_PRE(DD, 3, 3) \
  TQ_PRE(DD, 3, 4) TQ_PRE(DD, 4, 2) TQ_PRE(DD, 4, 3) TQ_PRE(DD, 4, 4)
#ifndef TQ_PREFILL_OTHER
  TQ_PRE_D(128)
#undef TQ_PRE_D
#undef TQ_PRE
  return tq_launch_prefill_other(c, cbk, cbv, sign_bits, q, q_heads, t_new, pos, n_layers, out, s);
#else
  TQ_PRE_D(64) TQ_PRE_D(256)
#undef TQ_PRE_D
#undef TQ_PRE
  return TQ_ERR_UNSUPPORTED;
#endif
}
