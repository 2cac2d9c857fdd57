/*
 * Seeded synthetic inputs for the KV-cache codec: one definition, compiled
 * twice (gcc for the host side, hipcc for the device side) so that both sides
 * produce bit-identical fp16 inputs from the same counters.
 *
 * This header holds no step of the codec itself (no rotation, codebook,
 * quantizer or attention); it only draws numbers.
 *
 * Generator: splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), used counter-style: the c-th output of the
 * stream with state s is mix(s + (c + 1) * 0x9E3779B97F4A7C15).
 *
 * Normal deviates: Box-Muller, z = sqrt(-2 ln u1) * cos(2 pi u2), with ln, cos
 * and exp written here from their series using only +, -, *, / and sqrt
 * (correctly rounded on both sides) and no contraction into FMA, so the fp64
 * results do not depend on a math library.  The final value is rounded to
 * fp16 with round-to-nearest-even by integer bit manipulation.
 *
 * The including file defines SYNTH_FN (the function qualifiers) and must
 * compile with floating-point contraction off.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ull

/* Stream tags. */
#define SYNTH_TAG_K 1u
#define SYNTH_TAG_V 2u
#define SYNTH_TAG_Q 3u
#define SYNTH_TAG_SCALE_K 4u
#define SYNTH_TAG_SCALE_V 5u
#define SYNTH_TAG_OUTLIER_K 6u
#define SYNTH_TAG_OUTLIER_V 7u
#define SYNTH_TAG_SIGN 8u
#define SYNTH_TAG_ISO 9u

SYNTH_FN uint64_t synth_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* c-th output of the splitmix64 stream whose state starts at s. */
SYNTH_FN uint64_t synth_at(uint64_t s, uint64_t c) {
  return synth_mix(s + (c + 1ull) * SYNTH_GOLDEN);
}

/* Key of a sub-stream: chained draws, one per coordinate of the key. */
SYNTH_FN uint64_t synth_key(uint64_t master, uint64_t tag, uint64_t a, uint64_t b,
                            uint64_t c) {
  uint64_t s = synth_at(master, tag);
  s = synth_at(s, a);
  s = synth_at(s, b);
  return synth_at(s, c);
}

/* Uniform in the open interval (0, 1): 53 random bits, centred in the cell. */
SYNTH_FN double synth_u01(uint64_t bits) {
  return ((double)(bits >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* Split a positive finite double into m in [sqrt(1/2), sqrt(2)) and e with
 * v = m * 2^e, by exponent-field arithmetic (exact). */
SYNTH_FN double synth_frexp(double v, int* e) {
  union { double d; uint64_t u; } w;
  w.d = v;
  int ex = (int)((w.u >> 52) & 0x7FF);
  int scale = 0;
  if (ex == 0) { /* subnormal: scale up by 2^64 first */
    w.d = v * 18446744073709551616.0;
    ex = (int)((w.u >> 52) & 0x7FF);
    scale = -64;
  }
  int k = ex - 1023;
  w.u = (w.u & 0x800FFFFFFFFFFFFFull) | (1023ull << 52); /* m in [1, 2) */
  if (w.d > 1.4142135623730951) {
    w.u = (w.u & 0x800FFFFFFFFFFFFFull) | (1022ull << 52); /* m in [0.5, 1) */
    k += 1;
  }
  *e = k + scale;
  return w.d;
}

/* Natural log of v > 0: v = m 2^e, ln m = 2 atanh(s), s = (m-1)/(m+1),
 * |s| <= 0.1716, series to s^27 (next term < 1e-21). */
SYNTH_FN double synth_log(double v) {
  int e;
  double m = synth_frexp(v, &e);
  double s = (m - 1.0) / (m + 1.0);
  double s2 = s * s;
  double p = 1.0 / 27.0;
  p = p * s2 + 1.0 / 25.0;
  p = p * s2 + 1.0 / 23.0;
  p = p * s2 + 1.0 / 21.0;
  p = p * s2 + 1.0 / 19.0;
  p = p * s2 + 1.0 / 17.0;
  p = p * s2 + 1.0 / 15.0;
  p = p * s2 + 1.0 / 13.0;
  p = p * s2 + 1.0 / 11.0;
  p = p * s2 + 1.0 / 9.0;
  p = p * s2 + 1.0 / 7.0;
  p = p * s2 + 1.0 / 5.0;
  p = p * s2 + 1.0 / 3.0;
  p = p * s2 + 1.0;
  double ln2_hi = 6.93147180369123816490e-01; /* ln 2 split so e*ln2_hi is exact */
  double ln2_lo = 1.90821492927058770002e-10;
  return (double)e * ln2_hi + ((double)e * ln2_lo + 2.0 * s * p);
}

/* cos(2 pi w) for any finite w: reduce to a in [0, 1/4] by periodicity and
 * symmetry, then the Taylor series of cos to x^26 at x = 2 pi a <= pi/2. */
SYNTH_FN double synth_cos2pi(double w) {
  double f = w - (double)(int64_t)w; /* fractional part, w >= 0 here */
  if (f < 0.0) f += 1.0;
  if (f > 0.5) f = 1.0 - f;          /* cos is even and 1-periodic in w */
  double sign = 1.0;
  if (f > 0.25) { f = 0.5 - f; sign = -1.0; }
  double x = 6.283185307179586 * f;
  double x2 = x * x;
  /* p = sum_k>=1 (-1)^(k-1) x^(2k-2) / (2k)!, k = 13 .. 1 */
  double p = 2.4795962632247976e-27;   /* 1/26! */
  p = p * x2 - 1.6117375710961184e-24; /* 1/24! */
  p = p * x2 + 8.896791392450574e-22;  /* 1/22! */
  p = p * x2 - 4.110317623312165e-19;  /* 1/20! */
  p = p * x2 + 1.5619206968586225e-16; /* 1/18! */
  p = p * x2 - 4.779477332387385e-14;  /* 1/16! */
  p = p * x2 + 1.1470745597729725e-11; /* 1/14! */
  p = p * x2 - 2.08767569878681e-09;   /* 1/12! */
  p = p * x2 + 2.755731922398589e-07;  /* 1/10! */
  p = p * x2 - 2.48015873015873e-05;   /* 1/8! */
  p = p * x2 + 1.388888888888889e-03;  /* 1/6! */
  p = p * x2 - 4.1666666666666664e-02; /* 1/4! */
  p = p * x2 + 0.5;                    /* 1/2! */
  return sign * (1.0 - x2 * p);
}

/* exp(v) for |v| < 700: v = k ln2 + r, |r| <= ln2/2, Taylor to r^20. */
SYNTH_FN double synth_exp(double v) {
  double kf = v * 1.4426950408889634;
  int k = (int)(kf < 0.0 ? kf - 0.5 : kf + 0.5);
  double ln2_hi = 6.93147180369123816490e-01;
  double ln2_lo = 1.90821492927058770002e-10;
  double r = (v - (double)k * ln2_hi) - (double)k * ln2_lo;
  double p = 1.0 / 2432902008176640000.0; /* 1/20! */
  double fact = 2432902008176640000.0;
  for (int j = 19; j >= 1; --j) {
    fact = fact / (double)(j + 1);        /* fact = j! exactly for j <= 20 */
    p = p * r + 1.0 / fact;
  }
  p = p * r + 1.0;
  union { double d; uint64_t u; } s;
  s.u = (uint64_t)(k + 1023) << 52;       /* 2^k, normal range only */
  return p * s.d;
}

/* Standard normal deviate number c of a stream. */
SYNTH_FN double synth_normal(uint64_t stream, uint64_t c) {
  double u1 = synth_u01(synth_at(stream, 2ull * c));
  double u2 = synth_u01(synth_at(stream, 2ull * c + 1ull));
  double r = -2.0 * synth_log(u1);
  return (r > 0.0 ? __builtin_sqrt(r) : 0.0) * synth_cos2pi(u2);
}

/* Round a double to the nearest fp16 (ties to even), returning its bits.
 * Overflow gives +-inf; NaN gives a quiet NaN. */
SYNTH_FN uint16_t synth_f16_rne(double v) {
  union { double d; uint64_t u; } w;
  w.d = v;
  uint16_t sign = (uint16_t)((w.u >> 48) & 0x8000u);
  int ex = (int)((w.u >> 52) & 0x7FF);
  uint64_t man = w.u & 0x000FFFFFFFFFFFFFull;
  if (ex == 0x7FF) return (uint16_t)(sign | (man ? 0x7E00u : 0x7C00u));
  if (ex == 0) return sign; /* fp64 subnormals are far below fp16's range */
  int e = ex - 1023;        /* v = 1.man * 2^e */
  uint64_t sig = man | (1ull << 52);      /* 53-bit significand */
  /* fp16 value = q * 2^(E-10) with q the 11-bit significand; for subnormal
   * fp16 the quantum is 2^-24. Compute the shift that brings sig to quanta. */
  int quantum_exp = (e >= -14) ? (e - 10) : -24;
  int shift = 52 - (e - quantum_exp);      /* sig * 2^(e-52) / 2^quantum_exp */
  if (shift > 63) return sign;             /* rounds to zero */
  uint64_t q, rem, half;
  if (shift <= 0) { q = sig << (-shift); rem = 0; half = 1; }
  else {
    q = sig >> shift;
    rem = sig & ((1ull << shift) - 1ull);
    half = 1ull << (shift - 1);
  }
  if (shift > 0 && (rem > half || (rem == half && (q & 1ull)))) q += 1ull;
  /* q counts quanta of 2^quantum_exp; rebuild the fp16 bits */
  if (quantum_exp == -24) {
    /* binades at or below 2^-14: the fp16 bit pattern of q * 2^-24 is q
     * itself for q <= 2048 (including the carry into 2^-13) */
    return (uint16_t)(sign | (uint16_t)q);
  }
  int E = e;
  if (q >= 2048u) { q >>= 1; E += 1; }     /* carried into the next binade */
  if (E > 15) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024u));
}

/* The four outlier channels of one (layer, kv head, K or V) stream: the first
 * four distinct values of draw % d. */
SYNTH_FN void synth_outliers(uint64_t master, uint32_t tag, uint64_t layer,
                             uint64_t head, int d, int* ch) {
  uint64_t s = synth_key(master, tag, layer, head, 0);
  int n = 0;
  for (uint64_t c = 0; n < 4; ++c) {
    int v = (int)(synth_at(s, c) % (uint64_t)d);
    int dup = 0;
    for (int j = 0; j < n; ++j) dup |= (ch[j] == v);
    if (!dup) ch[n++] = v;
  }
}

/* One fp16 K or V coordinate: z * (10 if outlier channel) * exp(0.5 z').
 * stream = synth_key(master, TAG_K/V, layer, seq, head); scale_stream the
 * matching TAG_SCALE_K/V key; t = token, i = coordinate. */
SYNTH_FN uint16_t synth_kv_value(uint64_t stream, uint64_t scale_stream,
                                 const int* outl, int d, uint64_t t, int i) {
  double z = synth_normal(stream, t * (uint64_t)d + (uint64_t)i);
  int o = (outl[0] == i) | (outl[1] == i) | (outl[2] == i) | (outl[3] == i);
  if (o) z = z * 10.0;
  double s = synth_exp(0.5 * synth_normal(scale_stream, t));
  return synth_f16_rne(z * s);
}

#endif
