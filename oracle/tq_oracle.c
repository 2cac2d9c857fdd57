/*
 * CPU oracle for the TurboQuant-style KV-cache codec and the decode attention
 * that reads it.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the library never links it.  It shares
 * no code, header, table or constant with the GPU path.
 *
 * Plain loops, fp64 throughout, no blocking, no fast transforms:
 *   - explicit Sylvester Hadamard matrix and explicit rotation R = H D / sqrt(d)
 *     (AdapTQ page, "How it works (HAR + VQ)", step 1: y = (1/sqrt d) H D x);
 *   - Lloyd iterations on the Gaussian density, integrals by composite Simpson
 *     quadrature ("We Built a Python Library That Cuts LLM Memory Usage by 80%",
 *     "The Paper": coordinates after rotation follow N(0, 1/d), optimal
 *     Lloyd-Max quantizer precomputed for that Gaussian);
 *   - exact fp16 norm by 128-bit integer arithmetic (same page, "The Paper":
 *     the norm is stored separately in FP16);
 *   - scalar argmin quantization of each rotated coordinate;
 *   - dequantization back to the original domain and naive softmax attention
 *     (same page, "Test Suite": softmax(Q K^T / sqrt d) V).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- fp16 -- */

/* Exact value of an fp16 bit pattern (inf/NaN map to themselves). */
double orc_half_to_double(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)f, -24);
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = ldexp((double)(1024 + f), e - 25);
  return s ? -v : v;
}

/* Integer m with |x| = m * 2^-24 for a finite fp16 pattern. */
static uint64_t half_quanta(uint16_t h) {
  int e = (h >> 10) & 31, f = h & 1023;
  if (e == 0) return (uint64_t)f;
  return (uint64_t)(1024 + f) << (e - 1);
}

/* ------------------------------------------------------------ rotation -- */

/* Sylvester construction by doubling: H_1 = [1],
 * H_2m = [[H_m, H_m], [H_m, -H_m]].  H is d x d, row-major, d a power of 2. */
void orc_hadamard(int d, double* H) {
  H[0] = 1.0;
  for (int m = 1; m < d; m *= 2)
    for (int i = 0; i < m; ++i)
      for (int j = 0; j < m; ++j) {
        double h = H[i * d + j];
        H[i * d + (j + m)] = h;
        H[(i + m) * d + j] = h;
        H[(i + m) * d + (j + m)] = -h;
      }
}

/* R = H D / sqrt(d) with D = diag(s), s_j = -1 iff bit j of sign_bits is set
 * (bit j lives in byte j/8 at position j%8). */
void orc_rotation(int d, const uint8_t* sign_bits, double* R) {
  double* H = (double*)malloc(sizeof(double) * (size_t)d * d);
  orc_hadamard(d, H);
  double inv = 1.0 / sqrt((double)d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      double s = ((sign_bits[j >> 3] >> (j & 7)) & 1) ? -1.0 : 1.0;
      R[i * d + j] = H[i * d + j] * s * inv;
    }
  free(H);
}

/* ------------------------------------------------------------ codebook -- */

static double phi(double z) { return exp(-0.5 * z * z) * 0.3989422804014327; }

/* Composite Simpson over [a, b] with n (even) intervals of phi(z) and z phi(z). */
static void simpson_cell(double a, double b, int n, double* mass, double* moment) {
  double h = (b - a) / n, m0 = 0.0, m1 = 0.0;
  for (int k = 0; k <= n; ++k) {
    double z = a + h * k;
    double w = (k == 0 || k == n) ? 1.0 : ((k & 1) ? 4.0 : 2.0);
    double p = phi(z);
    m0 += w * p;
    m1 += w * z * p;
  }
  *mass = m0 * h / 3.0;
  *moment = m1 * h / 3.0;
}

/* Lloyd-Max quantizer for N(0,1) with L = 2^bits levels.
 * c[L]: levels, t[L-1]: decision thresholds (midpoints), *mse: distortion.
 * Start from L levels spread uniformly over [-3, 3]; alternate the midpoint
 * rule and the conditional-mean rule (mass and first moment of each cell by
 * Simpson on [-12, 12]) until no level moves by 1e-14; then make the set
 * exactly antisymmetric.  Returns the number of iterations. */
int orc_lloyd_max(int bits, double* c, double* t, double* mse) {
  const int L = 1 << bits, N = 20000;
  const double lo = -12.0, hi = 12.0;
  for (int k = 0; k < L; ++k) c[k] = -3.0 + 6.0 * (k + 0.5) / L;
  int it = 0;
  for (; it < 200000; ++it) {
    for (int k = 1; k < L; ++k) t[k - 1] = 0.5 * (c[k - 1] + c[k]);
    double delta = 0.0;
    for (int k = 0; k < L; ++k) {
      double a = (k == 0) ? lo : t[k - 1], b = (k == L - 1) ? hi : t[k];
      double m0, m1;
      simpson_cell(a, b, N, &m0, &m1);
      double nc = m1 / m0;
      if (fabs(nc - c[k]) > delta) delta = fabs(nc - c[k]);
      c[k] = nc;
    }
    if (delta < 1e-14) break;
  }
  for (int k = 0; k < L / 2; ++k) {
    double m = 0.5 * (c[L - 1 - k] - c[k]);
    c[k] = -m;
    c[L - 1 - k] = m;
  }
  for (int k = 1; k < L; ++k) t[k - 1] = 0.5 * (c[k - 1] + c[k]);
  /* distortion: sum over cells of the integral of (z - c_k)^2 phi(z) */
  double D = 0.0;
  for (int k = 0; k < L; ++k) {
    double a = (k == 0) ? lo : t[k - 1], b = (k == L - 1) ? hi : t[k];
    double h = (b - a) / N, acc = 0.0;
    for (int j = 0; j <= N; ++j) {
      double z = a + h * j, w = (j == 0 || j == N) ? 1.0 : ((j & 1) ? 4.0 : 2.0);
      acc += w * (z - c[k]) * (z - c[k]) * phi(z);
    }
    D += acc * h / 3.0;
  }
  *mse = D;
  return it;
}

/* ---------------------------------------------------------------- norm -- */

/* fp16 nearest (ties to even) to the exact Euclidean norm of d fp16 values.
 * x_i = m_i 2^-24 with integer m_i, so S = sum m_i^2 is exact in 128 bits and
 * the norm is sqrt(S) 2^-24.  A candidate from fp64 is corrected by exact
 * comparisons of 4 S with (A + B)^2, where A < B are neighbouring fp16 values
 * in units of 2^-24 and (A + B) / 2 is the rounding midpoint.
 * *exact_norm receives sqrt(S) 2^-24 in fp64.  Inf/NaN inputs give NaN. */
uint16_t orc_norm16(const uint16_t* x, int d, double* exact_norm) {
  unsigned __int128 S = 0;
  for (int i = 0; i < d; ++i) {
    if (((x[i] >> 10) & 31) == 31) { *exact_norm = NAN; return 0x7E00; }
    unsigned __int128 m = half_quanta(x[i]);
    S += m * m;
  }
  double n = sqrt((double)S) * ldexp(1.0, -24);
  *exact_norm = n;
  /* Non-negative fp16 patterns are ordered like their values: walk the
   * pattern index p (0 .. 0x7C00 = inf) until the midpoint tests hold. */
  uint16_t p;
  {
    double v = n;
    /* start near the answer: truncate the fp64 value to an fp16 pattern */
    if (v >= 65504.0) p = 0x7BFF;
    else {
      int e;
      double m = frexp(v, &e); /* v = m 2^e, m in [0.5, 1) */
      if (v == 0.0) p = 0;
      else if (e - 1 < -14) p = (uint16_t)(v * 16777216.0);
      else p = (uint16_t)(((e - 1 + 15) << 10) | ((int)((m * 2.0 - 1.0) * 1024.0) & 1023));
    }
  }
  /* value of pattern p in units of 2^-24 (p = 0x7C00 stands for 65536) */
  #define QV(pp) ((pp) >= 0x7C00 ? (unsigned __int128)65536 << 24 : (unsigned __int128)half_quanta(pp))
  unsigned __int128 S4 = S * 4;
  for (;;) {
    if (p < 0x7C00) { /* compare with the upper midpoint */
      unsigned __int128 up = QV(p) + QV(p + 1);
      unsigned __int128 up2 = up * up;
      if (S4 > up2 || (S4 == up2 && (p & 1))) { ++p; continue; }
    }
    if (p > 0) { /* compare with the lower midpoint */
      unsigned __int128 dn = QV(p - 1) + QV(p);
      unsigned __int128 dn2 = dn * dn;
      if (S4 < dn2 || (S4 == dn2 && (p & 1))) { --p; continue; }
    }
    break;
  }
  #undef QV
  return p; /* 0x7C00 = +inf when the norm rounds past 65504 */
}

/* -------------------------------------------------------------- encode -- */

/* For each of n fp16 vectors x[n][d]:
 *   norms[v]   = fp16 nearest to ||x|| (orc_norm16);
 *   y          = R x / ||x|| with the exact norm (y = 0 for the zero vector);
 *   codes[v*d+i] = argmin_k |y_i - c[k]|, the smaller k on a tie;
 *   band[v*d+i]  = min_k |y_i - t[k]|, distance to the nearest threshold;
 *   alt[v*d+i]   = the code on the other side of that nearest threshold
 *                  (t[k] separates levels k and k + 1; the first of equally
 *                  near thresholds counts).  Within a tiny distance of a
 *                  threshold either neighbouring code is a correct encoding.
 * c[2^bits], t[2^bits - 1] are the dimension-scaled codebook (levels and
 * thresholds divided by sqrt(d)); R is orc_rotation's matrix.  band and alt
 * may be NULL. */
void orc_encode(const uint16_t* x, int64_t n, int d, int bits, const double* R,
                const double* c, const double* t, uint8_t* codes, uint16_t* norms,
                double* band, uint8_t* alt) {
  const int L = 1 << bits;
  double* xv = (double*)malloc(sizeof(double) * d);
  for (int64_t v = 0; v < n; ++v) {
    const uint16_t* xr = x + v * d;
    double nrm;
    norms[v] = orc_norm16(xr, d, &nrm);
    for (int j = 0; j < d; ++j) xv[j] = orc_half_to_double(xr[j]);
    for (int i = 0; i < d; ++i) {
      double y = 0.0;
      if (nrm > 0.0) {
        for (int j = 0; j < d; ++j) y += R[i * d + j] * xv[j];
        y /= nrm;
      }
      int best = 0;
      double bd = fabs(y - c[0]);
      for (int k = 1; k < L; ++k) {
        double dk = fabs(y - c[k]);
        if (dk < bd) { bd = dk; best = k; }
      }
      double md = INFINITY;
      int kt = 0;
      for (int k = 0; k < L - 1; ++k) {
        double dk = fabs(y - t[k]);
        if (dk < md) { md = dk; kt = k; }
      }
      codes[v * d + i] = (uint8_t)best;
      if (band) band[v * d + i] = md;
      if (alt) alt[v * d + i] = (uint8_t)(best == kt ? kt + 1 : kt);
    }
  }
  free(xv);
}

/* ------------------------------------------------------------- packing -- */

/* Row layout: a vector's d codes of `bits` bits form one little-endian bit
 * string of d*bits/8 bytes; code i occupies bits [bits*i, bits*i + bits),
 * bit j of the string is bit (j % 8) of byte j / 8. */
void orc_pack_rows(const uint8_t* codes, int64_t n, int d, int bits, uint8_t* out) {
  const int rb = d * bits / 8;
  memset(out, 0, (size_t)(n * rb));
  for (int64_t v = 0; v < n; ++v)
    for (int i = 0; i < d; ++i)
      for (int k = 0; k < bits; ++k) {
        int64_t bit = (int64_t)bits * i + k;
        if ((codes[v * d + i] >> k) & 1) out[v * rb + bit / 8] |= (uint8_t)(1u << (bit % 8));
      }
}

void orc_unpack_rows(const uint8_t* packed, int64_t n, int d, int bits, uint8_t* codes) {
  const int rb = d * bits / 8;
  for (int64_t v = 0; v < n; ++v)
    for (int i = 0; i < d; ++i) {
      int c = 0;
      for (int k = 0; k < bits; ++k) {
        int64_t bit = (int64_t)bits * i + k;
        c |= ((packed[v * rb + bit / 8] >> (bit % 8)) & 1) << k;
      }
      codes[v * d + i] = (uint8_t)c;
    }
}

/* Value-tile layout: the codes of 32 consecutive tokens form one tile of
 * 32*d*bits/8 bytes, cut into 64 segments of d*bits/16 bytes.  Segment
 * l = 16 q + r (q in 0..3, r in 0..15) is a little-endian bit string holding,
 * for m in 0..d/16-1 and u in 0..7, at bit offset (8 m + u) * bits, the code of
 * coordinate r * (d/16) + m of tile token tok(q, u) = 8 q + u.  codes[32][d]
 * are the tile's tokens in order. */
static int tile_token(int q, int u) { return 8 * q + u; }

void orc_pack_vtile(const uint8_t* codes, int d, int bits, uint8_t* tile) {
  const int seg = d * bits / 16, M = d / 16;
  memset(tile, 0, (size_t)(32 * d * bits / 8));
  for (int q = 0; q < 4; ++q)
    for (int r = 0; r < 16; ++r)
      for (int m = 0; m < M; ++m)
        for (int u = 0; u < 8; ++u) {
          int code = codes[tile_token(q, u) * d + r * M + m];
          for (int k = 0; k < bits; ++k) {
            int bit = (8 * m + u) * bits + k;
            if ((code >> k) & 1) tile[(16 * q + r) * seg + bit / 8] |= (uint8_t)(1u << (bit % 8));
          }
        }
}

void orc_unpack_vtile(const uint8_t* tile, int d, int bits, uint8_t* codes) {
  const int seg = d * bits / 16, M = d / 16;
  for (int q = 0; q < 4; ++q)
    for (int r = 0; r < 16; ++r)
      for (int m = 0; m < M; ++m)
        for (int u = 0; u < 8; ++u) {
          int code = 0;
          for (int k = 0; k < bits; ++k) {
            int bit = (8 * m + u) * bits + k;
            code |= ((tile[(16 * q + r) * seg + bit / 8] >> (bit % 8)) & 1) << k;
          }
          codes[tile_token(q, u) * d + r * M + m] = (uint8_t)code;
        }
}

/* ------------------------------------------------------------- dequant -- */

/* x_hat = n16 * R^T c[codes]: the stored fp16 norm times the rotated-back
 * levels, no renormalisation.  out[n][d]. */
void orc_dequant(const uint8_t* codes, const uint16_t* norms, int64_t n, int d,
                 const double* R, const double* c, double* out) {
  for (int64_t v = 0; v < n; ++v) {
    double nv = orc_half_to_double(norms[v]);
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int i = 0; i < d; ++i) s += R[i * d + j] * c[codes[v * d + i]];
      out[v * d + j] = nv * s;
    }
  }
}

/* ----------------------------------------------------------- attention -- */

/* For each of G queries q[G][d]: s_j = q . K[j] / sqrt(d) over the T keys,
 * p = softmax(s) (maximum subtracted), out[g] = sum_j p_j V[j].
 * T = 0 gives zeros. */
void orc_attention(const double* q, int G, const double* K, const double* V, int64_t T,
                   int d, double* out) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  double scale = 1.0 / sqrt((double)d);
  for (int g = 0; g < G; ++g) {
    for (int i = 0; i < d; ++i) out[g * d + i] = 0.0;
    if (T == 0) continue;
    double mx = -INFINITY;
    for (int64_t j = 0; j < T; ++j) {
      double a = 0.0;
      for (int i = 0; i < d; ++i) a += q[g * d + i] * K[j * d + i];
      s[j] = a * scale;
      if (s[j] > mx) mx = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < T; ++j) {
      s[j] = exp(s[j] - mx);
      l += s[j];
    }
    for (int64_t j = 0; j < T; ++j)
      for (int i = 0; i < d; ++i) out[g * d + i] += s[j] * V[j * d + i];
    for (int i = 0; i < d; ++i) out[g * d + i] /= l;
  }
  free(s);
}

/* Sparse V ("TurboQuant+ ...", section "Sparse V": value positions whose
 * attention weight is negligible are left out).  The page gives no
 * threshold; the reading here: position j is left out of the value sum when
 * its weight relative to the largest one, exp(s_j - max_k s_k), is below eps.
 * The softmax denominator keeps every position (all scores are computed; only
 * the value side is skipped).  eps <= 0 keeps everything (plain attention).
 *   out[g]   = sum_{j kept} p_j V[j] / l,   l = sum_j p_j,  p_j = exp(s_j - max)
 *   bound[g] = sum_{j left out} p_j |V[j]| / l   (coordinate-wise)
 * A computation that leaves out any subset of the left-out positions (and
 * nothing else) differs from out and from plain attention by at most bound,
 * coordinate by coordinate.  weights (optional, [G][T]) receives
 * exp(s_j - max). */
void orc_attention_sparse(const double* q, int G, const double* K, const double* V, int64_t T,
                          int d, double eps, double* out, double* bound, double* weights) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  double scale = 1.0 / sqrt((double)d);
  for (int g = 0; g < G; ++g) {
    for (int i = 0; i < d; ++i) out[g * d + i] = bound[g * d + i] = 0.0;
    if (T == 0) continue;
    double mx = -INFINITY;
    for (int64_t j = 0; j < T; ++j) {
      double a = 0.0;
      for (int i = 0; i < d; ++i) a += q[g * d + i] * K[j * d + i];
      s[j] = a * scale;
      if (s[j] > mx) mx = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < T; ++j) {
      s[j] = exp(s[j] - mx);
      l += s[j];
      if (weights) weights[(int64_t)g * T + j] = s[j];
    }
    for (int64_t j = 0; j < T; ++j) {
      if (s[j] >= eps)
        for (int i = 0; i < d; ++i) out[g * d + i] += s[j] * V[j * d + i];
      else
        for (int i = 0; i < d; ++i) bound[g * d + i] += s[j] * fabs(V[j * d + i]);
    }
    for (int i = 0; i < d; ++i) {
      out[g * d + i] /= l;
      bound[g * d + i] /= l;
    }
  }
  free(s);
}

/* Attention with an explicit set of positions left out of the value sum
 * (the Sparse V reading above, for a left-out set chosen by someone else):
 *   out[g] = sum_{j : keep[j]} p_j V[j] / sum_j p_j,  p_j = exp(s_j - max s)
 * for all G queries; the denominator keeps every position.  keep[T] holds 0
 * or 1 per position.  weights (optional, [G][T]) receives exp(s_j - max s),
 * so a caller can check that every left-out position was negligible. */
void orc_attention_keep(const double* q, int G, const double* K, const double* V, int64_t T,
                        int d, const uint8_t* keep, double* out, double* weights) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  double scale = 1.0 / sqrt((double)d);
  for (int g = 0; g < G; ++g) {
    for (int i = 0; i < d; ++i) out[g * d + i] = 0.0;
    if (T == 0) continue;
    double mx = -INFINITY;
    for (int64_t j = 0; j < T; ++j) {
      double a = 0.0;
      for (int i = 0; i < d; ++i) a += q[g * d + i] * K[j * d + i];
      s[j] = a * scale;
      if (s[j] > mx) mx = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < T; ++j) {
      s[j] = exp(s[j] - mx);
      l += s[j];
      if (weights) weights[(int64_t)g * T + j] = s[j];
    }
    for (int64_t j = 0; j < T; ++j)
      if (keep[j])
        for (int i = 0; i < d; ++i) out[g * d + i] += s[j] * V[j * d + i];
    for (int i = 0; i < d; ++i) out[g * d + i] /= l;
  }
  free(s);
}

/* ------------------------------------------------------------------ QJL -- */

/* Stage 2 of the method ("We Built a Python Library That Cuts LLM Memory
 * Usage by 80%", "Why not both stages?": a second stage of one bit per
 * coordinate for the residual, making inner-product estimates unbiased,
 * which that library skips).  The page gives no
 * more; the reading here is the quantized Johnson-Lindenstrauss sketch of the
 * stage-1 residual of a key, in the rotated unit domain:
 *   r = R x / ||x|| - c[codes],   gamma = ||r||,
 *   z_i = sign((S r)_i), i < m    (bit i set iff (S r)_i >= 0),
 * S an m x d matrix of i.i.d. N(0,1) draws given by the caller, and an inner
 * product with a query q estimated as
 *   <q, x> ~= n16 * ( <R q, c[codes]> + sqrt(pi/2) / m * gamma * <S R q, z> ),
 * whose second term is unbiased for n16 <R q, r> over the draw of S, because
 * E[sign(s.r) (s.u)] = sqrt(2/pi) <u, r> / ||r|| for s ~ N(0, I). */

/* Signs of S r (m x d, row-major) as m bits LSB-first, and gamma = ||r||;
 * proj (optional, m values) receives S r. */
void orc_qjl_project(const double* r, int d, const double* S, int m, uint8_t* bits,
                     double* gamma, double* proj) {
  double g = 0.0;
  for (int j = 0; j < d; ++j) g += r[j] * r[j];
  *gamma = sqrt(g);
  memset(bits, 0, (size_t)(m + 7) / 8);
  for (int i = 0; i < m; ++i) {
    double t = 0.0;
    for (int j = 0; j < d; ++j) t += S[i * d + j] * r[j];
    if (proj) proj[i] = t;
    if (t >= 0.0) bits[i / 8] |= (uint8_t)(1u << (i % 8));
  }
}

/* Stage 1 and 2 of n fp16 vectors x[n][d]: codes (unpacked, as orc_encode),
 * norms, the sign bits [n][m/8], gamma [n] and the projections [n][m]. */
void orc_qjl_encode(const uint16_t* x, int64_t n, int d, int bits, const double* R,
                    const double* c, const double* t, const double* S, int m, uint8_t* codes,
                    uint16_t* norms, uint8_t* signs, double* gamma, double* proj) {
  orc_encode(x, n, d, bits, R, c, t, codes, norms, NULL, NULL);
  double* xv = (double*)malloc(sizeof(double) * d);
  double* r = (double*)malloc(sizeof(double) * d);
  for (int64_t v = 0; v < n; ++v) {
    double nrm;
    orc_norm16(x + v * d, d, &nrm);
    for (int j = 0; j < d; ++j) xv[j] = orc_half_to_double(x[v * d + j]);
    for (int i = 0; i < d; ++i) {
      double y = 0.0;
      if (nrm > 0.0) {
        for (int j = 0; j < d; ++j) y += R[i * d + j] * xv[j];
        y /= nrm;
      }
      r[i] = y - c[codes[v * d + i]];
    }
    orc_qjl_project(r, d, S, m, signs + v * ((m + 7) / 8), gamma + v, proj ? proj + v * m : NULL);
  }
  free(xv);
  free(r);
}

/* The estimate of <q, x> for one query q[d] (original domain) and one encoded
 * key: codes[d] (unpacked), its fp16 norm n16 and fp16 gamma16 (as values),
 * its m sign bits; R, c, S as above. */
double orc_qjl_estimate(const double* q, int d, const double* R, const double* c,
                        const uint8_t* codes, double n16, double gamma16, const uint8_t* signs,
                        const double* S, int m) {
  double* rq = (double*)malloc(sizeof(double) * d);
  for (int i = 0; i < d; ++i) {
    double a = 0.0;
    for (int j = 0; j < d; ++j) a += R[i * d + j] * q[j];
    rq[i] = a;
  }
  double mse = 0.0;
  for (int i = 0; i < d; ++i) mse += rq[i] * c[codes[i]];
  double corr = 0.0;
  for (int k = 0; k < m; ++k) {
    double sq = 0.0;
    for (int j = 0; j < d; ++j) sq += S[k * d + j] * rq[j];
    corr += ((signs[k / 8] >> (k % 8)) & 1) ? sq : -sq;
  }
  free(rq);
  return n16 * (mse + sqrt(acos(-1.0) / 2.0) / m * gamma16 * corr);
}
