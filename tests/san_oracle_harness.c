/*
 * Drives every function of the CPU oracle (oracle/tq_oracle.c) over the
 * shapes and edge cases the tests use, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  Exits non-zero on a
 * failed sanity check; the sanitizers abort on any memory or UB error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_half_to_double(uint16_t h);
void orc_hadamard(int d, double* H);
void orc_rotation(int d, const uint8_t* sign_bits, double* R);
int orc_lloyd_max(int bits, double* c, double* t, double* mse);
uint16_t orc_norm16(const uint16_t* x, int d, double* exact_norm);
void orc_encode(const uint16_t* x, int64_t n, int d, int bits, const double* R, const double* c,
                const double* t, uint8_t* codes, uint16_t* norms, double* band, uint8_t* alt);
void orc_pack_rows(const uint8_t* codes, int64_t n, int d, int bits, uint8_t* out);
void orc_unpack_rows(const uint8_t* packed, int64_t n, int d, int bits, uint8_t* codes);
void orc_pack_vtile(const uint8_t* codes, int d, int bits, uint8_t* tile);
void orc_unpack_vtile(const uint8_t* tile, int d, int bits, uint8_t* codes);
void orc_dequant(const uint8_t* codes, const uint16_t* norms, int64_t n, int d, const double* R,
                 const double* c, double* out);
void orc_attention(const double* q, int G, const double* K, const double* V, int64_t T, int d,
                   double* out);
void orc_attention_sparse(const double* q, int G, const double* K, const double* V, int64_t T,
                          int d, double eps, double* out, double* bound, double* weights);
void orc_attention_keep(const double* q, int G, const double* K, const double* V, int64_t T,
                        int d, const uint8_t* keep, double* out, double* weights);
void orc_qjl_project(const double* r, int d, const double* S, int m, uint8_t* bits, double* gamma,
                     double* proj);
void orc_qjl_encode(const uint16_t* x, int64_t n, int d, int bits, const double* R,
                    const double* c, const double* t, const double* S, int m, uint8_t* codes,
                    uint16_t* norms, uint8_t* signs, double* gamma, double* proj);
double orc_qjl_estimate(const double* q, int d, const double* R, const double* c,
                        const uint8_t* codes, double n16, double gamma16, const uint8_t* signs,
                        const double* S, int m);

static uint64_t rs = 88172645463325252ull;
static uint64_t rnd(void) {
  rs ^= rs << 13;
  rs ^= rs >> 7;
  rs ^= rs << 17;
  return rs;
}
static double gauss(void) {
  double u = (rnd() >> 11) * 0x1p-53 + 1e-300, v = (rnd() >> 11) * 0x1p-53;
  return sqrt(-2 * log(u)) * cos(6.283185307179586 * v);
}
/* fp16 bits of a moderate double (truncation is enough for test inputs) */
static uint16_t to_half(double v) {
  uint16_t s = v < 0 ? 0x8000 : 0;
  double a = fabs(v);
  if (a < 0x1p-14) return s | (uint16_t)(a * 0x1p24);
  int e;
  double m = frexp(a, &e);
  if (e + 14 > 30) return s | 0x7BFF;
  return s | (uint16_t)(((e + 14) << 10) | ((int)((m * 2 - 1) * 1024) & 1023));
}

#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                      \
    }                                                                \
  } while (0)

static int run_dim(int d) {
  const int n = 37, T = 45, G = 3;
  uint8_t sb[32];
  for (int i = 0; i < d / 8; ++i) sb[i] = (uint8_t)rnd();
  double* H = malloc(sizeof(double) * d * d);
  double* R = malloc(sizeof(double) * d * d);
  orc_hadamard(d, H);
  orc_rotation(d, sb, R);
  for (int i = 0; i < d; ++i) {
    double s = 0;
    for (int j = 0; j < d; ++j) s += H[i * d + j] * H[i * d + j];
    CHECK(s == d);
  }
  uint16_t* x = malloc(sizeof(uint16_t) * n * d);
  for (int v = 0; v < n; ++v)
    for (int i = 0; i < d; ++i) x[v * d + i] = to_half(gauss() * (v == 3 ? 0.0 : 1.0 + v));
  x[5 * d + 1] = 0x7BFF; /* 65504 */
  x[6 * d + 2] = 0x0001; /* smallest subnormal */
  double* S = malloc(sizeof(double) * d * d);
  for (int i = 0; i < d * d; ++i) S[i] = gauss();
  for (int bits = 1; bits <= 4; ++bits) {
    const int L = 1 << bits;
    double c[16], t[16], mse;
    orc_lloyd_max(bits, c, t, &mse);
    CHECK(mse > 0 && mse < 1);
    for (int k = 0; k < L; ++k) c[k] /= sqrt((double)d);
    for (int k = 0; k + 1 < L; ++k) t[k] /= sqrt((double)d);
    uint8_t* codes = malloc((size_t)n * d);
    uint8_t* alt = malloc((size_t)n * d);
    uint16_t norms[64];
    double* band = malloc(sizeof(double) * n * d);
    orc_encode(x, n, d, bits, R, c, t, codes, norms, band, alt);
    orc_encode(x, n, d, bits, R, c, t, codes, norms, NULL, NULL);
    orc_encode(x, 0, d, bits, R, c, t, codes, norms, band, alt);
    for (int i = 0; i < n * d; ++i) {
      CHECK(codes[i] < L);
      if (bits > 1) CHECK(abs((int)alt[i] - (int)codes[i]) == 1);
    }
    if (bits >= 2) {
      const int rb = d * bits / 8;
      uint8_t* packed = malloc((size_t)n * rb);
      uint8_t* back = malloc((size_t)n * d);
      orc_pack_rows(codes, n, d, bits, packed);
      orc_unpack_rows(packed, n, d, bits, back);
      CHECK(memcmp(back, codes, (size_t)n * d) == 0);
      uint8_t* tile = malloc((size_t)32 * rb);
      orc_pack_vtile(codes, d, bits, tile); /* the first 32 vectors */
      orc_unpack_vtile(tile, d, bits, back);
      CHECK(memcmp(back, codes, (size_t)32 * d) == 0);
      double* xh = malloc(sizeof(double) * n * d);
      orc_dequant(codes, norms, n, d, R, c, xh);
      double* q = malloc(sizeof(double) * G * d);
      for (int i = 0; i < G * d; ++i) q[i] = gauss();
      double* out = malloc(sizeof(double) * G * d);
      double* out2 = malloc(sizeof(double) * G * d);
      double* bound = malloc(sizeof(double) * G * d);
      double* w = malloc(sizeof(double) * G * T);
      uint8_t keep[64];
      for (int j = 0; j < T; ++j) keep[j] = (uint8_t)(rnd() & 1);
      orc_attention(q, G, xh, xh, n < T ? n : T, d, out);
      orc_attention(q, G, xh, xh, 0, d, out);
      orc_attention_sparse(q, G, xh, xh, n, d, 1e-3, out, bound, NULL);
      orc_attention_sparse(q, G, xh, xh, 0, d, 1e-3, out, bound, w);
      orc_attention_keep(q, G, xh, xh, n, d, keep, out2, NULL);
      orc_attention_keep(q, G, xh, xh, 0, d, keep, out2, w);
      uint8_t* signs = malloc((size_t)n * (d / 8));
      double* gamma = malloc(sizeof(double) * n);
      double* proj = malloc(sizeof(double) * n * d);
      orc_qjl_encode(x, n, d, bits, R, c, t, S, d, codes, norms, signs, gamma, proj);
      orc_qjl_encode(x, n, d, bits, R, c, t, S, d, codes, norms, signs, gamma, NULL);
      double r[256], g;
      uint8_t pb[32];
      for (int i = 0; i < d; ++i) r[i] = gauss();
      orc_qjl_project(r, d, S, d, pb, &g, NULL);
      CHECK(g > 0);
      double e = orc_qjl_estimate(q, d, R, c, codes, 1.0, 0.5, signs, S, d);
      CHECK(isfinite(e));
      free(packed), free(back), free(tile), free(xh), free(q), free(out), free(out2);
      free(bound), free(w), free(signs), free(gamma), free(proj);
    }
    free(codes), free(alt), free(band);
  }
  free(H), free(R), free(x), free(S);
  return 0;
}

int main(void) {
  for (int h = 0; h < 65536; h += 7) (void)orc_half_to_double((uint16_t)h);
  uint16_t sp[4] = {0x7C00, 0, 0, 0}; /* inf input: NaN norm */
  double en;
  CHECK(orc_norm16(sp, 4, &en) == 0x7E00 && isnan(en));
  uint16_t big[256];
  for (int i = 0; i < 256; ++i) big[i] = 0x7BFF;
  CHECK(orc_norm16(big, 256, &en) == 0x7C00); /* rounds past 65504 */
  uint16_t zero[64] = {0};
  CHECK(orc_norm16(zero, 64, &en) == 0 && en == 0.0);
  for (int d = 64; d <= 256; d *= 2)
    if (run_dim(d)) return 1;
  printf("oracle harness ok\n");
  return 0;
}
