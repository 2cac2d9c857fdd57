/*
 * Device side of the seeded input generator (see synth_core.h): fills fp16
 * K/V and query tensors in GPU memory, bit-identical to synth_host.c.
 * Built with hipcc -ffp-contract=off.
 */
#include <hip/hip_runtime.h>
#pragma clang fp contract(off)
#define SYNTH_FN static __device__ inline
#include "synth_core.h"

#define SYNTH_TOK 64

/* grid: (ceil(nt / SYNTH_TOK), heads, seqs); block 256.
 * out[seq*s_seq + head*s_head + t*s_tok + i], t relative to t0. */
__global__ void __launch_bounds__(256)
synth_kv_kernel(uint64_t master, int kind, int layer, int d, int64_t t0, int64_t nt,
                uint16_t* __restrict__ out, int64_t s_seq, int64_t s_head, int64_t s_tok) {
  __shared__ int outl[4];
  __shared__ double scale[SYNTH_TOK];
  const int head = blockIdx.y, seq = blockIdx.z;
  const uint32_t tag = kind ? SYNTH_TAG_V : SYNTH_TAG_K;
  const uint32_t stag = kind ? SYNTH_TAG_SCALE_V : SYNTH_TAG_SCALE_K;
  const uint32_t otag = kind ? SYNTH_TAG_OUTLIER_V : SYNTH_TAG_OUTLIER_K;
  const uint64_t s = synth_key(master, tag, (uint64_t)layer, (uint64_t)seq, (uint64_t)head);
  const uint64_t ss = synth_key(master, stag, (uint64_t)layer, (uint64_t)seq, (uint64_t)head);
  const int64_t tb = (int64_t)blockIdx.x * SYNTH_TOK;
  if (threadIdx.x == 0) {
    int ch[4];
    synth_outliers(master, otag, (uint64_t)layer, (uint64_t)head, d, ch);
    for (int j = 0; j < 4; ++j) outl[j] = ch[j];
  }
  if (threadIdx.x < SYNTH_TOK) {
    int64_t t = tb + threadIdx.x;
    scale[threadIdx.x] = (t < nt) ? synth_exp(0.5 * synth_normal(ss, (uint64_t)(t0 + t))) : 0.0;
  }
  __syncthreads();
  int ol[4] = {outl[0], outl[1], outl[2], outl[3]};
  int64_t ntok = nt - tb < SYNTH_TOK ? nt - tb : SYNTH_TOK;
  for (int64_t e = threadIdx.x; e < ntok * d; e += blockDim.x) {
    int64_t tt = e / d;
    int i = (int)(e - tt * d);
    int64_t t = tb + tt;
    double z = synth_normal(s, (uint64_t)(t0 + t) * (uint64_t)d + (uint64_t)i);
    int o = (ol[0] == i) | (ol[1] == i) | (ol[2] == i) | (ol[3] == i);
    if (o) z = z * 10.0;
    out[seq * s_seq + head * s_head + t * s_tok + i] = synth_f16_rne(z * scale[tt]);
  }
}

/* grid: (heads, seqs); block = d threads. q[seq*s_seq + head*d + i]. */
__global__ void synth_q_kernel(uint64_t master, int step, int layer, int d,
                               uint16_t* __restrict__ out, int64_t s_seq) {
  const int head = blockIdx.x, seq = blockIdx.y;
  uint64_t s = synth_key(master, SYNTH_TAG_Q, (uint64_t)step,
                         ((uint64_t)layer << 32) | (uint64_t)seq, (uint64_t)head);
  int i = threadIdx.x;
  if (i < d) out[seq * s_seq + (int64_t)head * d + i] = synth_f16_rne(synth_normal(s, (uint64_t)i));
}

extern "C" int synth_kv_dev(uint64_t master, int kind, int layer, int seqs, int heads, int d,
                            int64_t t0, int64_t nt, uint16_t* out, int64_t s_seq,
                            int64_t s_head, int64_t s_tok, void* stream) {
  if (nt <= 0) return 0;
  dim3 grid((unsigned)((nt + SYNTH_TOK - 1) / SYNTH_TOK), (unsigned)heads, (unsigned)seqs);
  hipLaunchKernelGGL(synth_kv_kernel, grid, dim3(256), 0, (hipStream_t)stream, master, kind,
                     layer, d, t0, nt, out, s_seq, s_head, s_tok);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int synth_q_dev(uint64_t master, int step, int layer, int seqs, int heads, int d,
                           uint16_t* out, int64_t s_seq, void* stream) {
  hipLaunchKernelGGL(synth_q_kernel, dim3((unsigned)heads, (unsigned)seqs), dim3((unsigned)d), 0,
                     (hipStream_t)stream, master, step, layer, d, out, s_seq);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
