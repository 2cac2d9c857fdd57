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
 * Splits of one (layer, seq, kv head) write (m, l, acc) records; the last
 * split to arrive (an atomic counter per unit, reset by that split) merges
 * them and writes the output, so a call is a single kernel.
 * The levels are stored as fp16(c * sigma) with sigma chosen per codebook to
 * minimise their fp16 rounding; sigma is divided out of the query and output.
 *
 * Lane roles in a wave (lane = 16 q4 + n):
 *   K operand: tile token 8 (n / 4) + n % 4 (first product) or that + 4
 *              (second), coordinates [q4 d/4, (q4+1) d/4) of its row, one
 *              contiguous d*bits/32-byte load;
 *   score out: tile tokens 8 q4 .. 8 q4 + 7 (four per product), column n;
 *   V operand: segment lane of the 32-token value tile (see tq.h);
 *   value out: coordinates [q4 d/4, (q4+1) d/4) of head n.
 */
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

/* Waves per workgroup.  One block fills a CU (its lookup tables take most of
 * the LDS), so this is the CU's occupancy: 12 waves (3 per SIMD) where the
 * registers allow it (<= 170 VGPRs), else 8. */
constexpr int waves_for(int d, int bk, int bv) {
  return (d == 256 || (d == 128 && bk == 4 && bv == 4)) ? 8 : 12;
}
/* Decoder lookup tables in LDS.  Every table row is 256 bytes and holds
 * copies of one entry, one copy per lane (64 copies of a 4-byte entry, or 32
 * copies of an 8-byte entry, lane l reading copy l % 32: a 64-bit read serves
 * at most 32 lanes per LDS cycle), so the lanes of a lookup hit distinct
 * banks whatever the codes.  The row address is one byte permute: the index
 * byte goes to bits 8..15, the lane's copy offset to bits 0..7.
 *   Word tables (4-byte entries): the fp16 levels of two codes, indexed by a
 *     byte (bits 4), 6 bits (bits 3) or a nibble (bits 2).
 *   Split key tables (bits 3 and 4, 8-byte entries): {fp16 pair, fp16 pair
 *     of (level - fp16 level) * 2^11}, indexed by a byte: for bits 3 its low
 *     6 bits (two codes; the rows repeat every 64), so that a pair of codes
 *     anywhere in the packed row is one funnel shift and one byte permute away.  Key scores reach tens of nats at
 *     long context, where the ~1e-4 relative fp16 rounding of a level would
 *     move the softmax visibly; the remainder, multiplied by q * 2^-11 in the
 *     same matrix product, makes the level exact to ~2^-22.
 *   Quad value tables (bits 2, 8-byte entries): the four fp16 levels of a
 *     byte of four codes. */
template <int B>
struct KTab {
  static constexpr bool SPLIT = B >= 3;
  static constexpr int ENTRIES = B >= 3 ? 256 : 16; /* rows */
  static constexpr int SRC = B == 4 ? 256 : (B == 3 ? 64 : 16); /* distinct entries */
  static constexpr int BYTES = ENTRIES * 256;
};
template <int B>
struct VTab {
  static constexpr bool QUAD = B == 2;
  /* 3 bits: the 64 pair entries in 256 rows repeating every 64, so that the
   * index is the low 6 bits of a byte */
  static constexpr int ENTRIES = 256;
  static constexpr int SRC = B == 3 ? 64 : 256;
  static constexpr int BYTES = ENTRIES * 256;
};

/* Fill a word table: 64 copies of src[e] per row, e the row index modulo
 * SRC.  All of a thread's source words are loaded before any is stored, so
 * the block waits for one round of (L2-resident) loads rather than one per
 * iteration. */
template <int ENTRIES, int WAVES, int SRC = ENTRIES>
__device__ inline void fill_words(uint32_t* dst, const uint32_t* src) {
  constexpr int N = ENTRIES * 64, T = 64 * WAVES, IT = (N + T - 1) / T;
  uint32_t v[IT];
#pragma unroll
  for (int k = 0; k < IT; ++k) {
    const int i = threadIdx.x + k * T;
    v[k] = i < N ? src[(i >> 6) % SRC] : 0u;
  }
#pragma unroll
  for (int k = 0; k < IT; ++k) {
    const int i = threadIdx.x + k * T;
    if (i < N) dst[i] = v[k];
  }
}

/* Fill an 8-byte-entry table: 32 copies of {a[e * stride], b[e * stride]}
 * per row, e the row index modulo SRC (loads batched as above). */
template <int ENTRIES, int WAVES, int SRC = ENTRIES>
__device__ inline void fill_pairs(uint32_t* dst, const uint32_t* a, const uint32_t* b,
                                  int stride) {
  constexpr int N = ENTRIES * 32, T = 64 * WAVES, IT = (N + T - 1) / T;
  uint2 v[IT];
#pragma unroll
  for (int k = 0; k < IT; ++k) {
    const int i = threadIdx.x + k * T;
    const int e = (i >> 5) % SRC;
    v[k] = i < N ? make_uint2(a[e * stride], b[e * stride]) : make_uint2(0u, 0u);
  }
  uint2* d2 = (uint2*)dst;
#pragma unroll
  for (int k = 0; k < IT; ++k) {
    const int i = threadIdx.x + k * T;
    if (i < N) d2[i] = v[k];
  }
}

/* LDS word at byte address a of table t (a = (entry << 8) | lane offset). */
__device__ inline uint32_t lut_at(const uint32_t* t, uint32_t a) {
  return *(const uint32_t*)((const char*)t + a);
}
__device__ inline uint2 lut_at2(const uint32_t* t, uint32_t a) {
  return *(const uint2*)((const char*)t + a);
}

/* v_perm_b32 selector putting byte k of the first operand at bits 8..15 and
 * bytes 0 and 2 of the second (the lane offset, and the table base / 64 KB)
 * at bits 0..7 and 16..23. */
__device__ inline constexpr uint32_t sel_byte(int k) { return 0x0C020000u | ((4u + k) << 8); }

/* Dequantize an 8*B-bit field (8 codes) into 8 fp16 (4 words).  lo: the
 * lane's offset word (lane * 4). */
template <int B>
__device__ inline u32x4 deq8(const uint32_t* lut, uint32_t f, uint32_t lo) {
  u32x4 o;
  if constexpr (B == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = lut_at(lut, __builtin_amdgcn_perm(f, lo, sel_byte(k)));
  } else if constexpr (B == 3) {
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = lut_at(lut, (((f >> (6 * k)) & 0x3Fu) << 8) | lo);
  } else {
    /* nibbles 0, 2 in bytes 0, 1 of g; nibbles 1, 3 in bytes 0, 1 of h */
    const uint32_t g = f & 0x0F0Fu, h = (f >> 4) & 0x0F0Fu;
    o[0] = lut_at(lut, __builtin_amdgcn_perm(g, lo, sel_byte(0)));
    o[1] = lut_at(lut, __builtin_amdgcn_perm(h, lo, sel_byte(0)));
    o[2] = lut_at(lut, __builtin_amdgcn_perm(g, lo, sel_byte(1)));
    o[3] = lut_at(lut, __builtin_amdgcn_perm(h, lo, sel_byte(1)));
  }
  return o;
}

/* Split key lookups of all pairs of 3-bit codes in a lane's packed row piece
 * w (F fields of 8 codes): e[s][j] = entry of codes 8 s + 2 j, 8 s + 2 j + 1.
 * The pair at bit p = 24 s + 6 j is the low 6 bits of byte 0 of the string
 * shifted right by p, and the pair of field s + 1 is byte 3 of the same shift. */
template <int NW, int F>
__device__ inline void deq_split3(const uint32_t* lut, const uint32_t (&w)[NW], uint32_t lo8,
                                  uint2 (&e)[F][4]) {
  static_assert(F % 2 == 0, "fields come in pairs");
#pragma unroll
  for (int g = 0; g < F / 2; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = 48 * g + 6 * j, i = p / 32, sh = p % 32;
      const uint32_t hi = i + 1 < NW ? w[i + 1] : 0u;
      const uint32_t x = sh == 0 ? w[i] : __builtin_amdgcn_alignbit(hi, w[i], sh);
      e[2 * g][j] = lut_at2(lut, __builtin_amdgcn_perm(x, lo8, sel_byte(0)));
      e[2 * g + 1][j] = lut_at2(lut, __builtin_amdgcn_perm(x, lo8, sel_byte(3)));
    }
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

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

/* Loads of the packed cache go through buffer resources: a wave-uniform
 * stream base and size in scalar registers, a constant per-lane offset and a
 * scalar per-tile offset, so no vector address arithmetic is needed per
 * tile.  They are non-temporal (streaming): the cache is read once per step. */
constexpr int kNT = 2; /* cache-policy bits of a streaming load */

__device__ inline __amdgpu_buffer_rsrc_t make_stream(const uint8_t* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

/* Load N bytes (N % 4 == 0 or N == 6) at voff + soff of a stream, aligned to
 * A bytes. */
template <int N, int A>
__device__ inline void load_words(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int32_t soff,
                                  uint32_t (&w)[(N + 3) / 4]) {
  if constexpr (A >= 16 && N % 16 == 0) {
#pragma unroll
    for (int k = 0; k < N / 16; ++k) {
      const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16 * k, soff, kNT);
      w[4 * k] = t.x; w[4 * k + 1] = t.y; w[4 * k + 2] = t.z; w[4 * k + 3] = t.w;
    }
  } else if constexpr (A >= 8 && N % 8 == 0) {
#pragma unroll
    for (int k = 0; k < N / 8; ++k) {
      const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(rs, voff + 8 * k, soff, kNT);
      w[2 * k] = t.x; w[2 * k + 1] = t.y;
    }
  } else if constexpr (A >= 4 && N % 12 == 0) {
#pragma unroll
    for (int k = 0; k < N / 12; ++k) {
      const u32x3 t = __builtin_amdgcn_raw_buffer_load_b96(rs, voff + 12 * k, soff, kNT);
      w[3 * k] = t.x; w[3 * k + 1] = t.y; w[3 * k + 2] = t.z;
    }
  } else if constexpr (A >= 4 && N % 4 == 0) {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) w[k] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 4 * k, soff, kNT);
  } else {
    static_assert(N == 6, "unsupported load");
    const uint32_t h0 = __builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, kNT);
    const uint32_t h1 = __builtin_amdgcn_raw_buffer_load_b16(rs, voff + 2, soff, kNT);
    const uint32_t h2 = __builtin_amdgcn_raw_buffer_load_b16(rs, voff + 4, soff, kNT);
    w[0] = h0 | (h1 << 16);
    w[1] = h2;
  }
}

template <class T>
__device__ inline T load_norms(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int32_t soff);
template <>
__device__ inline uint32_t load_norms<uint32_t>(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, kNT);
}
template <>
__device__ inline uint2 load_norms<uint2>(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int32_t soff) {
  const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, kNT);
  return make_uint2(t.x, t.y);
}


/* v + v of the lane 8 places along in the same row (a single v_add_f32_dpp) */
__device__ inline float ror8_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true));
}

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

__device__ inline float h2f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

template <int D, int BK, int BV>
struct DecGeo {
  static constexpr int DIM = D, BITS_K = BK, BITS_V = BV;
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
  static constexpr int DEPTH = D == 256 ? 2 : 3; /* tiles in flight per wave (registers) */
};

struct DecArgs {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint8_t* k_norms;
  const uint8_t* v_norms;
  int64_t ls_kc, ls_vc, ls_kn, ls_vn;
  int batch, kv_heads, capacity, q_heads, group, n_layers;
  int max_len, splits, tiles_per_split;
  int upb;         /* units per block (> 1 only with one split and no Sparse V) */
  int64_t units;   /* (layer, sequence, KV head) units of the call */
  const int32_t* block_table; /* paged storage: [batch][max_pages] */
  int lg_tpp, max_pages, num_pages; /* log2(tiles per page), table row, pool pages */
  float sparse_eps;      /* Sparse V threshold (sparse kernels only) */
  float sparse_lg_eps;   /* log2 of it */
  uint32_t* skip_counts; /* optional [n_layers][batch][kv_heads] skipped-tile counts */
  uint32_t* skip_tiles;  /* optional [n_layers][batch][kv_heads][skip_words] bitmaps */
  int skip_words;        /* words per unit of skip_tiles: one bit per tile */
  const uint8_t* sign_bits;
  const uint16_t* q;
  const int32_t* seq_lens;
  const uint32_t* lut_k;
  const uint32_t* lut_k_lo;
  const uint32_t* lut_v;
  const uint32_t* lut_v_quad;
  float qscale;    /* log2(e) / (d * sigma_K) */
  float oscale;    /* 1 / (sqrt(d) * sigma_V) */
  float* out;
  void* ws;        /* [units] int32 arrival counters (zero between calls), then records */
  int64_t ctr_bytes;
};

/* Rows of rotated queries (and merged sums) a block keeps: the heads of all
 * its units (units per block x group size <= 16). */
constexpr int kQRows = 16;

/* LDS of one decode block. */
template <int D, int BK, int BV>
constexpr size_t decode_lds_bytes() {
  return (size_t)((KTab<BK>::BYTES + VTab<BV>::BYTES) > waves_for(D, BK, BV) * (8 * (D + 4) + 16) * 4
                      ? (KTab<BK>::BYTES + VTab<BV>::BYTES)
                      : waves_for(D, BK, BV) * (8 * (D + 4) + 16) * 4) +
         kQRows * D * 4;
}

/* Walsh-Hadamard transform of one row of D floats by one wave: lane l holds
 * coordinates l + 64 j; butterflies of stride >= 64 stay in the lane, the
 * others pair lanes l and l ^ h.  Returns the lane's transformed values. */
template <int D>
struct RowRegs {
  float v[D >= 64 ? D / 64 : 1];
};
template <int D>
__device__ inline RowRegs<D> wave_fwht(const float* row, int lane) {
  constexpr int J = D >= 64 ? D / 64 : 1;
  RowRegs<D> r;
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
  for (int h = 1; h < 64 && h < D; h <<= 1)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float y = __shfl_xor(r.v[j], h);
      r.v[j] = (lane & h) ? y - r.v[j] : r.v[j] + y;
    }
  return r;
}

/* One 32-token tile's loads for one lane.  The norms are only those of the
 * tokens whose softmax this lane computes (see tile_step): four consecutive
 * tokens (CF 2) or two (CF 4). */
template <int CF>
struct NormWords;
template <>
struct NormWords<2> {
  typedef uint2 T;
};
template <>
struct NormWords<4> {
  typedef uint32_t T;
};

template <class DG, int CF>
struct TileRegs {
  uint32_t kw0[DG::KW], kw1[DG::KW], vw[DG::VW];
  typename NormWords<CF>::T kn, vn;
  int32_t vt, nt; /* the tile's value-tile and norm offsets, when its values load later */
};

/* The four streams of one (layer, sequence, KV head) and a lane's offsets. */
struct TileAddr {
  __amdgpu_buffer_rsrc_t k;   /* key rows */
  __amdgpu_buffer_rsrc_t v;   /* value tiles */
  __amdgpu_buffer_rsrc_t kn;  /* key norms */
  __amdgpu_buffer_rsrc_t vn;  /* value norms */
  uint32_t koff, voff, noff;
};

/* Byte offsets of one tile in the four streams (first key row, value tile,
 * first norm). */
struct TileOff {
  int32_t k, v, n;
};

template <class DG, int CF, bool WITH_V = true>
__device__ inline void load_tile(TileRegs<DG, CF>& r, const TileAddr& ad, TileOff o) {
  typedef typename NormWords<CF>::T NT;
  load_words<DG::KB, DG::KA>(ad.k, ad.koff, o.k, r.kw0);
  load_words<DG::KB, DG::KA>(ad.k, ad.koff, o.k + 4 * DG::RB, r.kw1);
  if constexpr (WITH_V) load_words<DG::SEG, DG::VA>(ad.v, ad.voff, o.v, r.vw);
  r.vt = o.v;
  r.nt = o.n;
  r.kn = load_norms<NT>(ad.kn, ad.noff, o.n);
  if constexpr (WITH_V) r.vn = load_norms<NT>(ad.vn, ad.noff, o.n);
}

/* A lane offset past every stream's end: buffer loads from it return zeros
 * without touching memory. */
constexpr uint32_t kNoLoad = 0x80000000u;

/* Read-only kernel inputs read through the constant address space, so that
 * uniform reads become scalar loads. */
template <class T>
__device__ inline T ld_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

/* Tile token (0..31) of slot u (0..7) of a lane in row q4 of the products. */
__device__ inline int tok_of(int q4, int u) { return 8 * q4 + u; }

/* DPP move within 16-lane rows (lanes whose source lies outside the row
 * read 0). */
template <int CTRL>
__device__ inline float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ inline uint32_t dpp_mov_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
constexpr int kShl4 = 0x104, kShl8 = 0x108, kShl12 = 0x10C;
constexpr int kShr4 = 0x114, kShr8 = 0x118;
constexpr int kRor4 = 0x124, kRor8 = 0x128;

__device__ inline float max_ror4(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRor4, 0xF, 0xF, false)));
}
__device__ inline float max_ror8(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRor8, 0xF, 0xF, false)));
}
__device__ inline float add_ror4(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRor4, 0xF, 0xF, false));
}

/* x * h + c, h an fp16 value given by its bits (one mixed-precision FMA). */
__device__ inline float fma_h(float x, uint32_t h, float c) {
  return __builtin_fmaf(x, (float)__builtin_bit_cast(_Float16, (uint16_t)h), c);
}


/* Score one tile and update the online softmax: p[v] receives the weights
 * (relative to the updated running max) of the lane's 8 / CF (token, head)
 * slots, l_run their sum.  PARTIAL: some of its tokens lie at or past len
 * and are masked out.  When the max moves, the running sums are rescaled by
 * alpha: acc here (DEFER false), or by the caller (DEFER true: alpha is
 * returned and the result says whether it moved), for a caller that still
 * has an earlier tile's values to add at the old reference. */
template <class DG, int BK, bool PARTIAL, int CF, bool DEFER>
__device__ inline bool score_part(const TileRegs<DG, CF>& r,
                                  const half8 (&bq)[KTab<BK>::SPLIT ? 2 * DG::KS : DG::KS],
                                  const uint32_t* lk, uint32_t lok, floatx4 (&acc)[DG::VM],
                                  float& m_run, float& l_run, bool& first, int tok0, int len,
                                  int q4, int n, float (&p)[8 / CF], float& alpha,
                                  float* smax = nullptr) {
  floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (KTab<BK>::SPLIT) {
    /* split tables (3 and 4 bits): all lookups of the tile's keys first, so
     * that many are in flight, then the products; an operand is {fp16 pair,
     * remainder pair} of two codes twice */
    uint2 e0[DG::KS][4], e1[DG::KS][4];
    if constexpr (BK == 3) {
      deq_split3<DG::KW, DG::KS>(lk, r.kw0, lok, e0);
      deq_split3<DG::KW, DG::KS>(lk, r.kw1, lok, e1);
    } else {
#pragma unroll
      for (int s = 0; s < DG::KS; ++s)
#pragma unroll
        for (int k = 0; k < 4; ++k) e0[s][k] = lut_at2(lk, __builtin_amdgcn_perm(r.kw0[s], lok, sel_byte(k)));
#pragma unroll
      for (int s = 0; s < DG::KS; ++s)
#pragma unroll
        for (int k = 0; k < 4; ++k) e1[s][k] = lut_at2(lk, __builtin_amdgcn_perm(r.kw1[s], lok, sel_byte(k)));
    }
#pragma unroll
    for (int s = 0; s < DG::KS; ++s) {
      const u32x4 a0 = {e0[s][0].x, e0[s][0].y, e0[s][1].x, e0[s][1].y};
      const u32x4 a1 = {e0[s][2].x, e0[s][2].y, e0[s][3].x, e0[s][3].y};
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a0), bq[2 * s], s0, 0, 0, 0);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a1), bq[2 * s + 1], s0, 0, 0, 0);
      const u32x4 b0 = {e1[s][0].x, e1[s][0].y, e1[s][1].x, e1[s][1].y};
      const u32x4 b1 = {e1[s][2].x, e1[s][2].y, e1[s][3].x, e1[s][3].y};
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, b0), bq[2 * s], s1, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, b1), bq[2 * s + 1], s1, 0, 0, 0);
    }
  } else {
    /* 2-bit keys: word tables (fp16 pairs, no remainder) */
#pragma unroll
    for (int s = 0; s < DG::KS; ++s) {
      const u32x4 a0 = deq8<BK>(lk, field<BK>(r.kw0, s), lok);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a0), bq[s], s0, 0, 0, 0);
      const u32x4 a1 = deq8<BK>(lk, field<BK>(r.kw1, s), lok);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a1), bq[s], s1, 0, 0, 0);
    }
  }
  /* Softmax on compacted values.  After the products lane (q4, n) holds, for
   * slots u = 0..7 (tile token tok_of(q4, u)), column n's partial score:
   * columns 0..7 the fp16(q'') part of head n, 8..15 the remainder part of
   * head n - 8.  Joined (hi + lo) and spread over the row's lanes so that
   * each lane owns V = 8 / CF distinct (token, head) scores:
   *   CF 2: lane n takes slots 4 b + v (b = n >> 3) of head n & 7;
   *   CF 4 (group <= 4): lane n takes slots 2 a + v (a = n >> 2) of head
   *   n & 3. */
  constexpr int V = 8 / CF;
  float sc[V];
  int slot0;
  const bool upper = n >= 8; /* lane-constant selectors */
  if constexpr (CF == 2) {
    slot0 = upper ? 4 : 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      /* every lane runs both cross-lane moves (a lane that skipped one would
       * leave its partner reading a disabled lane), then selects */
      const float a0 = ror8_add(s0[v]), a1 = ror8_add(s1[v]);
      sc[v] = upper ? a1 : a0;
    }
  } else {
    slot0 = 2 * (n >> 2);
    const bool odd = (n & 4) != 0;
    float j[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      j[i] = ror8_add(s0[i]);
      j[4 + i] = ror8_add(s1[i]);
    }
    /* lanes 8..11 repeat heads 0..3, so slots 4, 5 are local there; groups
     * 4..7 and 12..15 take slots 2, 3 and 6, 7 from four lanes down */
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const float x = upper ? j[4 + v] : j[v];
      const float t = upper ? j[6 + v] : j[2 + v];
      const float y = dpp_mov<kShr4>(t);
      sc[v] = odd ? y : x;
    }
  }
  /* scores relative to the running max: w = s - m_run in one fma */
  uint32_t knh[V];
  if constexpr (CF == 2) {
    knh[0] = r.kn.x & 0xFFFFu; knh[1] = r.kn.x >> 16; knh[2] = r.kn.y & 0xFFFFu; knh[3] = r.kn.y >> 16;
  } else {
    knh[0] = r.kn & 0xFFFFu; knh[1] = r.kn >> 16;
  }
  bool moved = false;
  float mt = -INFINITY;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const float w = fma_h(sc[v], knh[v], -m_run);
    if (PARTIAL) {
      sc[v] = tok0 + tok_of(q4, slot0 + v) < len ? w : -INFINITY;
    } else {
      sc[v] = w;
    }
    mt = fmaxf(mt, sc[v]);
  }
  /* a new maximum (or the wave's first tile, which sets it): move the
   * reference and rescale the running sums; rare after the first tiles.
   * Any lane's score above its head's reference decides it; only then is
   * the head's maximum reduced, over the lanes that share the head and
   * over the rows. */
  if (__builtin_expect(__any(mt > 0.0f) || first, 0)) {
    if constexpr (CF == 4) mt = max_ror4(mt);
    mt = rows_max(max_ror8(mt));
    const float dm = first ? mt : fmaxf(mt, 0.0f);
    const float al = first ? 0.0f : __builtin_amdgcn_exp2f(-dm);
    l_run *= al;
    if constexpr (DEFER) {
      alpha = al;
      moved = true;
    } else {
#pragma unroll
      for (int m = 0; m < DG::VM; ++m) acc[m] *= al;
    }
    m_run += dm;
#pragma unroll
    for (int v = 0; v < V; ++v) sc[v] -= dm;
    first = false;
  }
#pragma unroll
  for (int v = 0; v < V; v += 2) {
    p[v] = __builtin_amdgcn_exp2f(sc[v]);
    p[v + 1] = __builtin_amdgcn_exp2f(sc[v + 1]);
    l_run += p[v] + p[v + 1];
  }
  if constexpr (DEFER) {
    /* the largest of the lane's scores relative to the running max */
    float m = sc[0];
#pragma unroll
    for (int v = 1; v < V; ++v) m = fmaxf(m, sc[v]);
    *smax = m;
  }
  return moved;
}

/* Accumulate one tile's values with its weights p (from score_part), the
 * value norms vn and the value words vw of the tile. */
template <class DG, int BV, int CF>
__device__ inline void value_part(const float (&p)[8 / CF], typename NormWords<CF>::T vn,
                                  const uint32_t (&vw)[DG::VW], const uint32_t* lv, uint32_t lo,
                                  uint32_t lo8, floatx4 (&acc)[DG::VM], int n) {
  constexpr int V = 8 / CF;
  const bool upper = n >= 8; /* lane-constant selectors */
  uint32_t vnh[V];
  if constexpr (CF == 2) {
    vnh[0] = vn.x & 0xFFFFu; vnh[1] = vn.x >> 16; vnh[2] = vn.y & 0xFFFFu; vnh[3] = vn.y >> 16;
  } else {
    vnh[0] = vn & 0xFFFFu; vnh[1] = vn >> 16;
  }
  /* P' = p m split into fp16(p m) (columns 0..7) and the fp16 remainder
   * (columns 8..15), as fp16 pairs of consecutive slots */
  uint32_t hp[V / 2], lp[V / 2];
#pragma unroll
  for (int v = 0; v < V; v += 2) {
    const float p0 = p[v], p1 = p[v + 1];
    /* fp16(p m) and the fp16 of the exact remainder p m - fp16(p m), each
     * one mixed-precision FMA */
    const float vn0 = (float)__builtin_bit_cast(_Float16, (uint16_t)vnh[v]);
    const float vn1 = (float)__builtin_bit_cast(_Float16, (uint16_t)vnh[v + 1]);
    const _Float16 h0 = (_Float16)__builtin_fmaf(p0, vn0, 0.0f);
    const _Float16 h1 = (_Float16)__builtin_fmaf(p1, vn1, 0.0f);
    const _Float16 r0 = (_Float16)__builtin_fmaf(p0, vn0, -(float)h0);
    const _Float16 r1 = (_Float16)__builtin_fmaf(p1, vn1, -(float)h1);
    hp[v / 2] = __builtin_bit_cast(uint32_t, half2v{h0, h1});
    lp[v / 2] = __builtin_bit_cast(uint32_t, half2v{r0, r1});
  }
  /* back to the operand layout: lane (q4, n) needs slots 0..7 of column n */
  /* (all cross-lane moves run on every lane before the selects) */
  u32x4 pw;
  if constexpr (CF == 2) {
    /* slots 0..3 live in the lower half, 4..7 in the upper one */
    const uint32_t l0 = dpp_mov_u<kRor8>(lp[0]), l1 = dpp_mov_u<kRor8>(lp[1]);
    const uint32_t h0 = dpp_mov_u<kRor8>(hp[0]), h1 = dpp_mov_u<kRor8>(hp[1]);
    pw[0] = upper ? l0 : hp[0];
    pw[1] = upper ? l1 : hp[1];
    pw[2] = upper ? lp[0] : h0;
    pw[3] = upper ? lp[1] : h1;
  } else {
    /* slot pair w of head g lives in lane 4 w + g; columns 0..3 read the
     * fp16 parts, 8..11 the remainders (4..7 and 12..15 are unused) */
    const uint32_t l8 = dpp_mov_u<kShr8>(lp[0]), l4 = dpp_mov_u<kShr4>(lp[0]);
    const uint32_t lu = dpp_mov_u<kShl4>(lp[0]);
    const uint32_t h4 = dpp_mov_u<kShl4>(hp[0]), h8 = dpp_mov_u<kShl8>(hp[0]);
    const uint32_t h12 = dpp_mov_u<kShl12>(hp[0]);
    pw[0] = upper ? l8 : hp[0];
    pw[1] = upper ? l4 : h4;
    pw[2] = upper ? lp[0] : h8;
    pw[3] = upper ? lu : h12;
  }
  const half8 pb = __builtin_bit_cast(half8, pw);
  if constexpr (VTab<BV>::QUAD) {
    /* a value word holds two 16-bit fields; each byte of one is four tokens'
     * codes, looked up as four fp16 levels at once */
#pragma unroll
    for (int m = 0; m < DG::VM; ++m) {
      const uint2 w0 = lut_at2(lv, __builtin_amdgcn_perm(vw[m / 2], lo8, sel_byte(2 * (m & 1))));
      const uint2 w1 = lut_at2(lv, __builtin_amdgcn_perm(vw[m / 2], lo8, sel_byte(2 * (m & 1) + 1)));
      const u32x4 av = {w0.x, w0.y, w1.x, w1.y};
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av), pb, acc[m], 0, 0, 0);
    }
  } else if constexpr (BV == 3) {
    /* fields m, m + 1 (m even) are the 48 bits from bit 24 m: shifted right
     * by 24 m + 6 k, the string holds pair k of field m in the low 6 bits of
     * byte 0 and pair k of field m + 1 in those of byte 3 (the table's rows
     * repeat every 64), so one funnel shift serves two lookups */
#pragma unroll
    for (int g = 0; g < DG::VM / 2; ++g) {
      u32x4 a0, a1;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int p = 48 * g + 6 * k, i = p / 32, sh = p % 32;
        const uint32_t hi = i + 1 < DG::VW ? vw[i + 1] : 0u;
        const uint32_t x = sh == 0 ? vw[i] : __builtin_amdgcn_alignbit(hi, vw[i], (uint32_t)sh);
        a0[k] = lut_at(lv, __builtin_amdgcn_perm(x, lo, sel_byte(0)));
        a1[k] = lut_at(lv, __builtin_amdgcn_perm(x, lo, sel_byte(3)));
      }
      acc[2 * g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a0), pb,
                                                          acc[2 * g], 0, 0, 0);
      acc[2 * g + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a1), pb,
                                                              acc[2 * g + 1], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int m = 0; m < DG::VM; ++m) {
      const u32x4 av = deq8<BV>(lv, field<BV>(vw, m), lo);
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av), pb, acc[m], 0, 0, 0);
    }
  }
}

/* Score, softmax-update and accumulate one tile whose values came with it. */
template <class DG, int BK, int BV, bool PARTIAL, int CF>
__device__ inline void tile_step(const TileRegs<DG, CF>& r,
                                 const half8 (&bq)[KTab<BK>::SPLIT ? 2 * DG::KS : DG::KS],
                                 const uint32_t* lk, const uint32_t* lv, uint32_t lo,
                                 uint32_t lo8, uint32_t lok, floatx4 (&acc)[DG::VM],
                                 float& m_run, float& l_run, bool& first, int tok0, int len,
                                 int q4, int n) {
  float p[8 / CF], alpha;
  score_part<DG, BK, PARTIAL, CF, false>(r, bq, lk, lok, acc, m_run, l_run, first, tok0, len, q4,
                                         n, p, alpha);
  value_part<DG, BV, CF>(p, r.vn, r.vw, lv, lo, lo8, acc, n);
}

/* The full tiles of a wave with the Sparse V gate ("TurboQuant+ ...",
 * "Sparse V": value work of positions with negligible attention weight is
 * skipped).  A tile's values are loaded and accumulated unless, for every
 * query head of the group and every token of the tile, the weight relative
 * to the block's largest running max of that head is below eps.  That
 * reference never exceeds the final max, so a skipped token's final weight
 * is below eps too; the softmax denominator keeps every token.
 *
 * To skip the value bytes, a tile's values are requested only after its
 * scores: the wave scores one tile ahead.  Per step, with tile t scored and
 * its value load in flight: score tile t + W (its keys and norms came
 * through the ring), request its values (or a no-memory load past the
 * stream's end when skipped, so that the wait counts stay static), refill
 * the freed ring slot, then accumulate tile t's values, and only then apply
 * the rescale that the scoring of t + W may have asked for (t's weights are
 * still at the old reference).  On entry ra holds tile (and rb tile + W
 * with a depth-3 ring); the rest of the ring is loaded here.
 *
 * A skipped tile's value load reads zeros (codes and norms), so its weights
 * P' = p m are zero and its value products add nothing.  SKIPWORK false runs
 * them anyway, with no branch around the accumulators (such a branch makes
 * every kept tile copy them); SKIPWORK true branches around them, which pays
 * off only when most tiles are skipped. */
template <class DG, int BK, int BV, int CF, bool SKIPWORK, class PF>
__device__ inline void sparse_tiles(const DecArgs& a, const TileAddr& ad, TileRegs<DG, CF>& ra,
                                    TileRegs<DG, CF>& rb, TileRegs<DG, CF>& rc, PF& pf,
                                    const half8 (&bq)[KTab<BK>::SPLIT ? 2 * DG::KS : DG::KS],
                                    const uint32_t* lk, const uint32_t* lv, uint32_t lo,
                                    uint32_t lo8, uint32_t lok, floatx4 (&acc)[DG::VM],
                                    float& m_run, float& l_run, bool& first, int& tile,
                                    int full_end, int len, int q4, int n, int lane, float* mref,
                                    int layer, int b, int kv) {
  typedef typename NormWords<CF>::T NT;
  constexpr int V = 8 / CF, W = waves_for(DG::DIM, BK, BV), NH = CF == 4 ? 4 : 8;
  const int head = n & (NH - 1);
  const bool voter = head < a.group; /* padding columns do not vote */
  const float lg_eps = a.sparse_lg_eps;
  /* the block's reference grows through plain stores of running maxima (a
   * lost race leaves a smaller one, which is still a valid reference) */
  auto publish = [&]() {
    if (lane < NH && lane < a.group &&
        m_run > __hip_atomic_load(&mref[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))
      __hip_atomic_store(&mref[lane], m_run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  /* does any (token, head) weight of the tile reach eps against the larger
   * of the block's reference and the wave's running max?  smax is the
   * lane's largest score relative to m_run (log2) */
  auto keep_of = [&](float smax) -> bool {
    const float ref =
        __hip_atomic_load(&mref[head], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return __any(voter && smax - fmaxf(ref - m_run, 0.0f) >= lg_eps);
  };
  /* a tile's value codes and norms go to its own ring slot, whose key
   * refills leave them alone, so no register copy ever waits on an
   * in-flight load */
  auto load_v = [&](TileRegs<DG, CF>& r, bool keep) {
    load_words<DG::SEG, DG::VA>(ad.v, keep ? ad.voff : kNoLoad, r.vt, r.vw);
    r.vn = load_norms<NT>(ad.vn, keep ? ad.noff : kNoLoad, r.nt);
  };
  uint32_t nskip = 0;
  if constexpr (DG::DEPTH == 3)
    pf(rc, tile + 2 * W);
  else
    pf(rb, tile + W);
  /* the first tile: scored here (it sets the running max) */
  float pc[V], alpha = 1.0f, sm;
  if (score_part<DG, BK, false, CF, true>(ra, bq, lk, lok, acc, m_run, l_run, first, tile * 32,
                                          len, q4, n, pc, alpha, &sm))
    publish();
  bool keepc = keep_of(sm);
  load_v(ra, keepc);
  pf(ra, tile + DG::DEPTH * W);
  /* the value half of a step: tile's values (in slot cur) at weights pc */
  uint32_t* const skip_map =
      a.skip_tiles ? a.skip_tiles + (((int64_t)layer * a.batch + b) * a.kv_heads + kv) * a.skip_words
                   : nullptr;
  auto values = [&](TileRegs<DG, CF>& cur) {
    if (!SKIPWORK || keepc) value_part<DG, BV, CF>(pc, cur.vn, cur.vw, lv, lo, lo8, acc, n);
    if (!keepc) {
      ++nskip;
      if (skip_map && lane == 0) atomicOr(skip_map + (tile >> 5), 1u << (tile & 31));
    }
  };
  /* one step: cur holds the values of tile, nxt the keys of tile + W (which
   * exists) */
  auto step = [&](TileRegs<DG, CF>& cur, TileRegs<DG, CF>& nxt) {
    float pn[V], al = 1.0f, smn;
    const bool moved = score_part<DG, BK, false, CF, true>(nxt, bq, lk, lok, acc, m_run, l_run,
                                                           first, (tile + W) * 32, len, q4, n,
                                                           pn, al, &smn);
    if (moved) publish();
    const bool keepn = keep_of(smn);
    load_v(nxt, keepn);
    pf(nxt, tile + W + DG::DEPTH * W);
    values(cur);
    if (moved) {
#pragma unroll
      for (int m = 0; m < DG::VM; ++m) acc[m] *= al;
    }
    tile += W;
#pragma unroll
    for (int v = 0; v < V; ++v) pc[v] = pn[v];
    keepc = keepn;
  };
  /* the wave's full tiles are tile, tile + W, ..., cnt of them; whole ring
   * turns first (no exits inside, so the wait counts stay those of the
   * steady state), then the rest, then the last tile's values */
  const int cnt = (full_end - 1 - tile) / W + 1;
  int k = 1;
  if constexpr (DG::DEPTH == 3) {
    for (; k + 3 <= cnt; k += 3) {
      step(ra, rb);
      step(rb, rc);
      step(rc, ra);
    }
    if (k < cnt) {
      step(ra, rb);
      if (k + 1 < cnt) {
        step(rb, rc);
        values(rc);
      } else {
        values(rb);
      }
    } else {
      values(ra);
    }
  } else {
    for (; k + 2 <= cnt; k += 2) {
      step(ra, rb);
      step(rb, ra);
    }
    if (k < cnt) {
      step(ra, rb);
      values(rb);
    } else {
      values(ra);
    }
  }
  tile += W;
  if (a.skip_counts && lane == 0 && nskip)
    atomicAdd(a.skip_counts + ((int64_t)layer * a.batch + b) * a.kv_heads + kv, nskip);
}

/* SPARSE: 0 dense; 1 the Sparse V gate, skipped tiles still running their
 * value products; 2 the gate, skipped tiles leaving them out */
template <int D, int BK, int BV, int CF, bool PAGED, int SPARSE, bool MULTI>
__global__ void __launch_bounds__(64 * waves_for(D, BK, BV))
decode_kernel(DecArgs a) {
  using DG = DecGeo<D, BK, BV>;
  constexpr int kWaves = waves_for(D, BK, BV);
  /* static LDS (addresses known at compile time, so table bases fold into
   * the ds_read offset field): [V table | K table] during the token loop,
   * reused as the wave-merge buffer afterwards; then the rotated queries */
  __shared__ __align__(16) char smem[decode_lds_bytes<D, BK, BV>()];
  uint32_t* lut_v = (uint32_t*)smem;
  uint32_t* lut_k = (uint32_t*)(smem + VTab<BV>::BYTES);
  /* Key lookups address the key table from the LDS base: its part below
   * 64 KB folds into the ds_read offset field, the 64 KB pages ride in the
   * lane-offset operand of the address permute (no extra add per lookup). */
  constexpr uint32_t KPAGE = VTab<BV>::BYTES & ~0xFFFFu;
  const uint32_t* lut_k_rd = (const uint32_t*)(smem + (VTab<BV>::BYTES - KPAGE));
  float* qbuf = (float*)(smem + decode_lds_bytes<D, BK, BV>() - kQRows * D * 4);
  float* mbuf = (float*)smem; /* aliases the tables after the token loop */
  const int G = a.group;
  /* the wave index is uniform within a wave: say so, so that tile indices
   * and load bases live in scalar registers */
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  const int q4 = lane / 16, n = lane % 16;
  /* A block takes one split of one (layer, sequence, KV head) unit, or (with
   * one split) upb whole units, each streamed by kWaves / upb of its waves,
   * all sharing the block's lookup tables.  ug: this wave's unit in the
   * block, wu: its index among that unit's waves. */
  const int upb = MULTI ? a.upb : 1, wpu = MULTI ? kWaves / upb : kWaves;
  const int ug = wave / wpu, wu = wave - ug * wpu;
  const int split = upb == 1 ? (int)(blockIdx.x % a.splits) : 0;
  const int64_t unit_id = upb == 1 ? (int64_t)(blockIdx.x / a.splits) : (int64_t)blockIdx.x * upb + ug;
  const bool unit_ok = unit_id < a.units; /* the last block's spare waves stream nothing */
  int64_t unit = unit_ok ? unit_id : a.units - 1;
  const int kv = (int)(unit % a.kv_heads);
  unit /= a.kv_heads;
  const int b = (int)(unit % a.batch);
  const int layer = (int)(unit / a.batch);

  int len = unit_ok ? a.seq_lens[b] : 0;
  len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
  const int ntiles = (len + 31) / 32;
  const int t_begin = split * a.tiles_per_split;
  int t_end = t_begin + a.tiles_per_split;
  if (t_end > ntiles) t_end = ntiles;

  /* streams: the (sequence, head) rows of the layer (contiguous), or the
   * layer's whole page pool (paged, tile offsets then go through the block
   * table) */
  const int64_t sh = PAGED ? 0 : (int64_t)b * a.kv_heads + kv;
  const int64_t srows = PAGED ? (int64_t)a.num_pages * a.kv_heads * (32 << a.lg_tpp) : a.capacity;
  TileAddr ad;
  ad.k = make_stream(a.k_codes + layer * a.ls_kc + sh * a.capacity * DG::RB, srows * DG::RB);
  ad.v = make_stream(a.v_codes + layer * a.ls_vc + sh * (a.capacity / 32) * DG::TILE,
                     srows / 32 * DG::TILE);
  ad.kn = make_stream(a.k_norms + layer * a.ls_kn + sh * a.capacity * 2, srows * 2);
  ad.vn = make_stream(a.v_norms + layer * a.ls_vn + sh * a.capacity * 2, srows * 2);
  /* score rows: row 4 i + j of the first product is tile token 8 i + j, of
   * the second 8 i + 4 + j (so that slot u of row group q4 is token 8 q4 + u) */
  ad.koff = (uint32_t)((8 * (n >> 2) + (n & 3)) * DG::RB + q4 * DG::KB);
  ad.voff = (uint32_t)(lane * DG::SEG);
  /* norms of the tokens this lane's softmax covers (see tile_step) */
  ad.noff = (uint32_t)(2 * tok_of(q4, CF == 2 ? 4 * (n >> 3) : 2 * (n >> 2)));
  const uint32_t lo = (uint32_t)lane << 2;           /* value tables, 4-byte entries */
  const uint32_t lo8 = (uint32_t)(lane & 31) << 3;   /* value tables, 8-byte entries */
  const uint32_t lok = (KTab<BK>::SPLIT ? lo8 : lo) | KPAGE; /* key table */

  /* the first tiles' loads go out before the tables are built, so their
   * latency overlaps the prologue (issued on every path, clamped to a tile
   * that exists, so that the loop's waits stay exact) */
  const int full_end = (len / 32) < t_end ? (len / 32) : t_end;
  int tile = t_begin + wu;
  const int W = MULTI ? wpu : kWaves;  /* tile stride between a wave's tiles */
  const int last = full_end > 0 ? full_end - 1 : 0;
  /* tile t's offsets: tile t of the stream, or tile t % tpp of the pool page
   * the block table gives for page t / tpp (clamped into the pool) */
  auto toff = [&](int t) -> TileOff {
    if constexpr (PAGED) {
      const int tpp = 1 << a.lg_tpp, pg = t >> a.lg_tpp, w = t & (tpp - 1);
      int phys = ld_const(a.block_table + (int64_t)b * a.max_pages + pg);
      phys = phys < 0 ? 0 : (phys >= a.num_pages ? a.num_pages - 1 : phys);
      const int pb = phys * a.kv_heads + kv;
      return TileOff{pb * (tpp * 32 * DG::RB) + w * (32 * DG::RB), pb * (tpp * DG::TILE) + w * DG::TILE,
                     pb * (tpp * 64) + w * 64};
    } else {
      return TileOff{t * (32 * DG::RB), t * DG::TILE, t * 64};
    }
  };
  /* with Sparse V the tile's values load only once its scores say they are
   * needed (see below) */
  auto pf = [&](TileRegs<DG, CF>& r, int t) {
    load_tile<DG, CF, !SPARSE>(r, ad, toff(t < last ? t : last));
  };
  TileRegs<DG, CF> ra, rb, rc;
  pf(ra, tile);
  if constexpr (DG::DEPTH == 3) pf(rb, tile + W);

  if constexpr (KTab<BK>::SPLIT)
    fill_pairs<KTab<BK>::ENTRIES, kWaves, KTab<BK>::SRC>(lut_k, a.lut_k, a.lut_k_lo, 1);
  else
    fill_words<KTab<BK>::ENTRIES, kWaves>(lut_k, a.lut_k);
  if constexpr (VTab<BV>::QUAD)
    fill_pairs<VTab<BV>::ENTRIES, kWaves>(lut_v, a.lut_v_quad, a.lut_v_quad + 1, 2);
  else
    fill_words<VTab<BV>::ENTRIES, kWaves, VTab<BV>::SRC>(lut_v, a.lut_v);
  /* rotated queries: qbuf[u G + g][i] = (D q_g)_i of the block's unit u,
   * then FWHT, then scale */
  const uint8_t* sb = a.sign_bits + (int64_t)layer * (D / 8);
  auto unit_of = [&](int u, int& ul, int& ub, int& ukv) -> bool {
    int64_t id = upb == 1 ? (int64_t)(blockIdx.x / a.splits) : (int64_t)blockIdx.x * upb + u;
    const bool ok = id < a.units;
    if (!ok) id = a.units - 1;
    ukv = (int)(id % a.kv_heads);
    id /= a.kv_heads;
    ub = (int)(id % a.batch);
    ul = (int)(id / a.batch);
    return ok;
  };
  for (int t = threadIdx.x; t < upb * G * D; t += blockDim.x) {
    const int r = t / D, i = t % D, u = r / G, g = r % G;
    int ul, ub, ukv;
    float v = 0.0f;
    if (unit_of(u, ul, ub, ukv)) {
      v = h2f(a.q[((((int64_t)ul * a.batch + ub) * a.q_heads + (int64_t)ukv * G + g) * D) + i]);
      if ((a.sign_bits[(int64_t)ul * (D / 8) + (i >> 3)] >> (i & 7)) & 1) v = -v;
    }
    qbuf[t] = v;
  }
  /* Sparse V: a running max per head shared by the block's waves, so that
   * each gates against the largest one seen */
  __shared__ float mref[8];
  if constexpr (SPARSE)
    if (threadIdx.x < 8) mref[threadIdx.x] = -INFINITY;
  __syncthreads();
  /* one wave per head transforms its row in registers */
  for (int r = wave; r < upb * G; r += kWaves) {
    const RowRegs<D> t = wave_fwht<D>(qbuf + r * D, lane);
#pragma unroll
    for (int j = 0; j < (D >= 64 ? D / 64 : 1); ++j) qbuf[r * D + lane + 64 * j] = t.v[j];
  }
  __syncthreads();

  /* B operands of the score products: fp16(q'') in columns 0..7 (one per
   * head), the fp16 remainder q'' - fp16(q'') in columns 8..15.  With split
   * key tables an operand covers 4 coordinates c0..c3 of the lane's 8 as
   * rows [c0 c1 c0' c1' c2 c3 c2' c3'], where the primed rows meet the level
   * remainders and hold fp16(q'' * 2^-11) in columns 0..7, zero elsewhere. */
  constexpr int NB = KTab<BK>::SPLIT ? 2 * DG::KS : DG::KS;
  half8 bq[NB];
  {
    const int g = n & 7;
    const float* qg = qbuf + (ug * G + g) * D + q4 * DG::KQ;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        int j;
        bool rem = false;
        if constexpr (KTab<BK>::SPLIT) {
          j = 4 * t + 2 * (r / 4) + (r & 1);
          rem = (r & 2) != 0;
        } else {
          j = 8 * t + r;
        }
        const float v = g < G ? qg[j] * a.qscale : 0.0f;
        const _Float16 hi = (_Float16)v;
        _Float16 e;
        if (rem)
          e = n < 8 ? (_Float16)(v * 0x1p-11f) : (_Float16)0.0f;
        else
          e = n < 8 ? hi : (_Float16)(v - (float)hi);
        bq[t][r] = e;
      }
    }
  }

  floatx4 acc[DG::VM];
#pragma unroll
  for (int m = 0; m < DG::VM; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
  /* running max (base 2) of this wave's scores, set by its first tile */
  float m_run = 0.0f, l_run = 0.0f;
  bool first = true;

  /* full tiles, software-pipelined: the loads of the next tiles are in
   * flight while this one is scored and accumulated (a ring of register
   * sets, so no copies between tiles).  Prefetches are issued on every path
   * (past the end they re-read the wave's last tile) so the number of loads
   * in flight is the same everywhere and each wait covers only the tile
   * about to be used. */
  if constexpr (SPARSE) {
    if (tile < full_end)
      sparse_tiles<DG, BK, BV, CF, SPARSE == 2>(a, ad, ra, rb, rc, pf, bq, lut_k_rd, lut_v, lo,
                                                lo8, lok, acc, m_run, l_run, first, tile,
                                                full_end, len, q4, n, lane, mref, layer, b, kv);
  } else if (tile < full_end) {
    auto step = [&](const TileRegs<DG, CF>& r) {
      tile_step<DG, BK, BV, false, CF>(r, bq, lut_k_rd, lut_v, lo, lo8, lok, acc, m_run, l_run,
                                       first, tile * 32, len, q4, n);
    };
    if constexpr (DG::DEPTH == 3) {
      for (;;) {
        pf(rc, tile + 2 * W);
        step(ra);
        if ((tile += W) >= full_end) break;
        pf(ra, tile + 2 * W);
        step(rb);
        if ((tile += W) >= full_end) break;
        pf(rb, tile + 2 * W);
        step(rc);
        if ((tile += W) >= full_end) break;
      }
    } else {
      for (;;) {
        pf(rb, tile + W);
        step(ra);
        if ((tile += W) >= full_end) break;
        pf(ra, tile + W);
        step(rb);
        if ((tile += W) >= full_end) break;
      }
    }
  }
  /* the ragged last tile, if this wave owns it */
  if (tile < t_end) {
    TileRegs<DG, CF> rp;
    load_tile<DG, CF>(rp, ad, toff(tile));
    tile_step<DG, BK, BV, true, CF>(rp, bq, lut_k_rd, lut_v, lo, lo8, lok, acc, m_run, l_run,
                                    first, tile * 32, len, q4, n);
  }
  if (first) m_run = -1e30f; /* no tiles: contributes nothing to the merge */
  /* the lanes of a head hold disjoint tokens' sums */
  l_run = rows_sum(l_run);
  if constexpr (CF == 4) l_run = add_ror4(l_run);
  l_run += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(l_run), kRor8, 0xF, 0xF, false));
  /* value sums: column g (< 8) += column g + 8 (the fp16 remainders of p m) */
#pragma unroll
  for (int m = 0; m < DG::VM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[m][i] = ror8_add(acc[m][i]);

  /* merge the waves: mbuf[w] = {m[8], l[8], acc[8][D + 4]} (rows padded so
   * that the lanes' writes spread over the banks) */
  constexpr int MR = D + 4, MW = 8 * MR + 16;
  __syncthreads(); /* tables are dead from here on */
  float* mw = mbuf + wave * MW;
  if (n < 8) {
    if (q4 == 0) {
      mw[n] = m_run;
      mw[8 + n] = l_run;
    }
#pragma unroll
    for (int m = 0; m < DG::VM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) mw[16 + n * MR + (4 * q4 + i) * DG::VM + m] = acc[m][i];
  }
  __syncthreads();
  /* merged record per head of each unit in qbuf (reused): qbuf[u G + g][i];
   * wsc[w][g] = the weight of wave w's sums, exp2(m_w - M) (a wave belongs
   * to one unit, waves u wpu .. u wpu + wpu - 1) */
  float* res = qbuf;
  __shared__ float mg[kQRows], lg[kQRows], wsc[kWaves][8];
  if (threadIdx.x < upb * G) {
    const int u = threadIdx.x / G, g = threadIdx.x % G;
    float M = -1e30f;
    for (int w = u * wpu; w < (u + 1) * wpu; ++w) M = fmaxf(M, mbuf[w * MW + g]);
    float L = 0.0f;
    for (int w = u * wpu; w < (u + 1) * wpu; ++w) {
      const float* r = mbuf + w * MW;
      const float e = __builtin_amdgcn_exp2f(r[g] - M);
      wsc[w][g] = e;
      L += e * r[8 + g];
    }
    mg[threadIdx.x] = M;
    lg[threadIdx.x] = L;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < upb * G * D; t += blockDim.x) {
    const int r = t / D, i = t % D, u = r / G, g = r % G;
    float s = 0.0f;
    for (int w = u * wpu; w < (u + 1) * wpu; ++w) s += wsc[w][g] * mbuf[w * MW + 16 + g * MR + i];
    res[t] = s;
  }
  __syncthreads();
  const int64_t head0 = ((int64_t)layer * a.batch + b) * a.q_heads + (int64_t)kv * G;
  if (a.splits == 1) {
    /* one wave per head of each unit: inverse rotation, 1/l and the scales,
     * straight out */
    for (int r = wave; r < upb * G; r += kWaves) {
      int ul, ub, ukv;
      if (!unit_of(r / G, ul, ub, ukv)) continue;
      const int64_t h0 = ((int64_t)ul * a.batch + ub) * a.q_heads + (int64_t)ukv * G + r % G;
      const uint8_t* usb = a.sign_bits + (int64_t)ul * (D / 8);
      const RowRegs<D> t = wave_fwht<D>(res + r * D, lane);
      const float L = lg[r];
      const float f = L > 0.0f ? a.oscale / L : 0.0f;
#pragma unroll
      for (int j = 0; j < (D >= 64 ? D / 64 : 1); ++j) {
        const int i = lane + 64 * j;
        if (i < D) {
          const float v = t.v[j] * f;
          a.out[h0 * D + i] = ((usb[i >> 3] >> (i & 7)) & 1) ? -v : v;
        }
      }
    }
  } else {
    /* partial record per (head, split): {m, l, acc[D]}, after the counters.
     * Records and counters are exchanged between blocks (possibly on other
     * XCDs) with device-scope relaxed atomic stores and loads, which go to
     * the coherent level directly; a wait for this block's stores orders them
     * before its counter increment.  (Device-scope fences would write back
     * and invalidate the whole L2 instead, stalling every block's streams.) */
    const int64_t uid = blockIdx.x / a.splits;
    float* recs = (float*)((char*)a.ws + a.ctr_bytes);
    for (int t = threadIdx.x; t < G * (D + 2); t += blockDim.x) {
      const int g = t / (D + 2), k = t % (D + 2);
      float* rec = recs + ((head0 + g) * a.splits + split) * (D + 2);
      const float v = k == 0 ? mg[g] : (k == 1 ? lg[g] : res[g * D + (k - 2)]);
      __hip_atomic_store(rec + k, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0); /* this wave's records are written */
    __syncthreads();
    /* the last split of the unit to finish merges all of them */
    __shared__ int last;
    if (threadIdx.x == 0) {
      int* ctr = (int*)a.ws + uid;
      const int ticket = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = ticket == a.splits - 1;
      /* every split has arrived: ready for the next call */
      if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return;
    auto rd = [](const float* p) {
      return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    if (threadIdx.x < G) {
      const int g = threadIdx.x;
      const float* r = recs + (head0 + g) * a.splits * (D + 2);
      float M = -1e30f;
      for (int sp = 0; sp < a.splits; ++sp) M = fmaxf(M, rd(r + sp * (D + 2)));
      float L = 0.0f;
      for (int sp = 0; sp < a.splits; ++sp)
        L += __builtin_amdgcn_exp2f(rd(r + sp * (D + 2)) - M) * rd(r + sp * (D + 2) + 1);
      mg[g] = M;
      lg[g] = L;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < G * D; t += blockDim.x) {
      const int g = t / D, i = t % D;
      const float* r = recs + (head0 + g) * a.splits * (D + 2);
      float s = 0.0f;
      for (int sp = 0; sp < a.splits; ++sp)
        s += __builtin_amdgcn_exp2f(rd(r + sp * (D + 2)) - mg[g]) * rd(r + sp * (D + 2) + 2 + i);
      res[t] = s;
    }
    __syncthreads();
    if (wave < G) {
      /* head `wave`: inverse rotation, 1/l and the scales, straight out */
      const RowRegs<D> t = wave_fwht<D>(res + wave * D, lane);
      const float L = lg[wave];
      const float f = L > 0.0f ? a.oscale / L : 0.0f;
#pragma unroll
      for (int j = 0; j < (D >= 64 ? D / 64 : 1); ++j) {
        const int i = lane + 64 * j;
        if (i < D) {
          const float v = t.v[j] * f;
          a.out[(head0 + wave) * D + i] = ((sb[i >> 3] >> (i & 7)) & 1) ? -v : v;
        }
      }
    }
  }
}

/* Groups of up to 4 query heads compact their softmax 4 ways, up to 8 2 ways;
 * several units per block only in the dense, contiguous form. */
template <int D, int BK, int BV>
tq_status launch_decode_t(const DecArgs& a, hipStream_t s) {
  const int64_t blocks = a.upb > 1 ? (a.units + a.upb - 1) / a.upb : a.units * a.splits;
  const dim3 grid((unsigned)blocks), block(64 * waves_for(D, BK, BV));
#define TQ_LAUNCH(CF, PG, SP, MU) \
  hipLaunchKernelGGL((decode_kernel<D, BK, BV, CF, PG, SP, MU>), grid, block, 0, s, a)
  /* Sparse V: from eps 1e-3 on, most tiles of a long context are skipped,
   * and leaving out their value products is worth the branch (contiguous
   * storage only; paged storage always runs them) */
  const bool sp = a.sparse_eps > 0.0f, mu = a.upb > 1, skipwork = a.sparse_eps >= 1e-3f;
  if (a.block_table) {
    if (a.group <= 4) {
      if (sp) TQ_LAUNCH(4, true, 1, false); else TQ_LAUNCH(4, true, 0, false);
    } else {
      if (sp) TQ_LAUNCH(2, true, 1, false); else TQ_LAUNCH(2, true, 0, false);
    }
  } else {
    if (a.group <= 4) {
      if (sp && skipwork) TQ_LAUNCH(4, false, 2, false);
      else if (sp) TQ_LAUNCH(4, false, 1, false);
      else if (mu) TQ_LAUNCH(4, false, 0, true);
      else TQ_LAUNCH(4, false, 0, false);
    } else {
      if (sp && skipwork) TQ_LAUNCH(2, false, 2, false);
      else if (sp) TQ_LAUNCH(2, false, 1, false);
      else if (mu) TQ_LAUNCH(2, false, 0, true);
      else TQ_LAUNCH(2, false, 0, false);
    }
  }
#undef TQ_LAUNCH
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

}  // namespace

/* Blocks of this instantiation the device runs at once (occupancy x CUs);
 * looked up once per process, with a fallback when no device answers. */
template <int D, int BK, int BV>
int concurrent_blocks_t() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_kernel<D, BK, BV, 2, false, 0, false>, 64 * waves_for(D, BK, BV),
                                                     0) != hipSuccess ||
        cus <= 0 || per <= 0) {
      (void)hipGetLastError();
      return 256 * 2;
    }
    cached = cus * per;
  }
  return cached;
}

static int concurrent_blocks(int d, int bk, int bv) {
#define TQ_OCC(DD, KK, VV) \
  if (d == DD && bk == KK && bv == VV) return concurrent_blocks_t<DD, KK, VV>();
#define TQ_OCC_D(DD) \
  TQ_OCC(DD, 2, 2) TQ_OCC(DD, 2, 3) TQ_OCC(DD, 2, 4) TQ_OCC(DD, 3, 2) TQ_OCC(DD, 3, 3) \
  TQ_OCC(DD, 3, 4) TQ_OCC(DD, 4, 2) TQ_OCC(DD, 4, 3) TQ_OCC(DD, 4, 4)
  TQ_OCC_D(64) TQ_OCC_D(128) TQ_OCC_D(256)
#undef TQ_OCC_D
#undef TQ_OCC
  return 512;
}

/* Split count: the smallest that keeps the last round of blocks at least 90%
 * full (blocks / (rounds * concurrent)), else the best one found, with every
 * wave keeping at least two tiles. */
tq_decode_plan tq_plan_decode(const tq_kv_cache* c, int q_heads, int max_len, int n_layers) {
  tq_decode_plan p;
  const int64_t units = (int64_t)n_layers * c->batch * c->kv_heads;
  const int tiles = (max_len + 31) / 32;
  const int64_t conc = concurrent_blocks(c->head_dim, c->bits_k, c->bits_v);
  const int waves = waves_for(c->head_dim, c->bits_k, c->bits_v);
  int max_splits = tiles / (2 * waves);
  if (max_splits > 64) max_splits = 64;
  if (max_splits < 1) max_splits = 1;
  int splits = 1;
  double best = -1.0;
  for (int sp = 1; sp <= max_splits; ++sp) {
    const int64_t blocks = units * sp;
    const int64_t rounds = (blocks + conc - 1) / conc;
    const double eff = (double)blocks / (double)(rounds * conc);
    if (eff > best + 1e-9) { best = eff; splits = sp; }
    if (eff >= 0.9) break;
  }
  p.splits = splits;
  p.tiles_per_split = tiles > 0 ? (tiles + splits - 1) / splits : 0;
  /* With one split, up to 4 units share a block (its waves split between
   * them, one table fill for all) when the rounds of blocks stay >= 90%
   * full: many-round workloads pay the block's fixed cost (launch, first
   * loads, table fill, merge) once per upb units. */
  p.upb = 1;
  if (splits == 1) {
    const int G = q_heads / c->kv_heads;
    for (int u = 4; u >= 2; --u) {
      if (waves % u != 0 || u * G > kQRows) continue;
      const int64_t blocks = (units + u - 1) / u;
      const int64_t rounds = (blocks + conc - 1) / conc;
      if ((double)blocks / (double)(rounds * conc) >= 0.9) {
        p.upb = u;
        break;
      }
    }
  }
  p.ctr_bytes = ((size_t)units * sizeof(int) + 255) & ~(size_t)255;
  p.ws_bytes = splits > 1 ? p.ctr_bytes + (size_t)n_layers * c->batch * q_heads * splits *
                                              (c->head_dim + 2) * sizeof(float)
                          : 0;
  return p;
}

tq_status tq_launch_decode(const tq_kv_cache* c, const tq_codebook_s* cbk,
                           const tq_codebook_s* cbv, const uint8_t* sign_bits,
                           const uint16_t* q, int q_heads, const int32_t* seq_lens,
                           int max_len, int n_layers, float* out, void* ws,
                           const tq_decode_plan& plan, float sparse_eps, uint32_t* skip_counts,
                           uint32_t* skip_tiles, hipStream_t s) {
  DecArgs a;
  a.sparse_eps = sparse_eps;
  a.sparse_lg_eps = sparse_eps > 0.0f ? (float)log2((double)sparse_eps) : -INFINITY;
  a.skip_counts = skip_counts;
  a.skip_tiles = skip_tiles;
  a.skip_words = tq_skip_words(max_len);
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
  /* Sparse V and paged storage keep one unit per block */
  a.upb = (sparse_eps > 0.0f || c->block_table) ? 1 : plan.upb;
  a.units = (int64_t)n_layers * c->batch * c->kv_heads;
  a.sign_bits = sign_bits;
  a.q = q;
  a.seq_lens = seq_lens;
  a.lut_k = cbk->dec_lut;
  a.lut_k_lo = cbk->dec_lut_lo;
  a.lut_v_quad = cbv->dec_quad;
  a.lut_v = cbv->dec_lut;
  const double d = c->head_dim;
  a.qscale = (float)(1.4426950408889634 / (d * cbk->sigma));
  a.oscale = (float)(1.0 / (sqrt(d) * cbv->sigma));
  a.out = out;
  a.ws = ws;
  a.ctr_bytes = (int64_t)plan.ctr_bytes;
  a.block_table = c->block_table;
  a.lg_tpp = 0;
  if (c->block_table)
    while ((32 << a.lg_tpp) < c->page_tokens) ++a.lg_tpp;
  a.max_pages = c->block_table ? c->max_pages : 0;
  a.num_pages = c->block_table ? c->num_pages : 0;
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
