/*
 * Host side of the seeded input generator (see synth_core.h for the
 * definition).  Built with gcc -ffp-contract=off; exported with C linkage.
 */
#define SYNTH_FN static inline
#include "synth_core.h"

/* fp16 K (kind 0) or V (kind 1) vectors of one (layer, seq, kv head) stream,
 * tokens t0 .. t0+nt-1, written as out[t][d]. */
void synth_kv_host(uint64_t master, int kind, int layer, int seq, int head, int d,
                   int64_t t0, int64_t nt, uint16_t* out) {
  uint32_t tag = kind ? SYNTH_TAG_V : SYNTH_TAG_K;
  uint32_t stag = kind ? SYNTH_TAG_SCALE_V : SYNTH_TAG_SCALE_K;
  uint32_t otag = kind ? SYNTH_TAG_OUTLIER_V : SYNTH_TAG_OUTLIER_K;
  uint64_t s = synth_key(master, tag, (uint64_t)layer, (uint64_t)seq, (uint64_t)head);
  uint64_t ss = synth_key(master, stag, (uint64_t)layer, (uint64_t)seq, (uint64_t)head);
  int outl[4];
  synth_outliers(master, otag, (uint64_t)layer, (uint64_t)head, d, outl);
  for (int64_t t = 0; t < nt; ++t)
    for (int i = 0; i < d; ++i)
      out[t * d + i] = synth_kv_value(s, ss, outl, d, (uint64_t)(t0 + t), i);
}

/* fp16 N(0,1) query of (step, layer, seq, query head). */
void synth_q_host(uint64_t master, int step, int layer, int seq, int qhead, int d,
                  uint16_t* out) {
  uint64_t s = synth_key(master, SYNTH_TAG_Q, (uint64_t)step,
                         ((uint64_t)layer << 32) | (uint64_t)seq, (uint64_t)qhead);
  for (int i = 0; i < d; ++i) out[i] = synth_f16_rne(synth_normal(s, (uint64_t)i));
}

/* The d sign bits of one layer, packed LSB-first into d/8 bytes. */
void synth_sign_bits_host(uint64_t master, int layer, int d, uint8_t* out) {
  uint64_t s = synth_key(master, SYNTH_TAG_SIGN, (uint64_t)layer, 0, 0);
  for (int i = 0; i < d / 8; ++i) out[i] = 0;
  for (int i = 0; i < d; ++i)
    if (synth_at(s, (uint64_t)i) >> 63) out[i >> 3] |= (uint8_t)(1u << (i & 7));
}

void synth_outliers_host(uint64_t master, int kind, int layer, int head, int d, int* ch) {
  synth_outliers(master, kind ? SYNTH_TAG_OUTLIER_V : SYNTH_TAG_OUTLIER_K,
                 (uint64_t)layer, (uint64_t)head, d, ch);
}

/* Isotropic fp16 N(0,1) vectors (no outliers, no scale): n rows of d. */
void synth_iso_host(uint64_t master, uint64_t stream_id, int64_t n, int d, uint16_t* out) {
  uint64_t s = synth_key(master, SYNTH_TAG_ISO, stream_id, 0, 0);
  for (int64_t k = 0; k < n * d; ++k) out[k] = synth_f16_rne(synth_normal(s, (uint64_t)k));
}

/* Raw fp64 normal deviates of a stream (for statistical checks). */
void synth_normals_host(uint64_t stream, uint64_t c0, int64_t n, double* out) {
  for (int64_t k = 0; k < n; ++k) out[k] = synth_normal(stream, c0 + (uint64_t)k);
}

uint64_t synth_key_host(uint64_t master, uint64_t tag, uint64_t a, uint64_t b, uint64_t c) {
  return synth_key(master, tag, a, b, c);
}

uint16_t synth_f16_rne_host(double v) { return synth_f16_rne(v); }
double synth_log_host(double v) { return synth_log(v); }
double synth_exp_host(double v) { return synth_exp(v); }
double synth_cos2pi_host(double v) { return synth_cos2pi(v); }
