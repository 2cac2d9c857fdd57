/*
 * Drives the host side of the C ABI (kv_cache_quantization_tq_amd/csrc/
 * tq_host.cpp) without a GPU, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py): status strings, the
 * host Lloyd-Max, the codebook build up to its device upload (which fails
 * cleanly without a device), cache sizing, and every entry point's argument
 * validation.  The kernel launchers and the decode planner live in the HIP
 * sources; here they are stand-ins that count calls, so the harness can check
 * that rejected calls never launch and accepted ones do.
 */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "tq.h"
#include "tq_internal.h"

static int launches = 0;

tq_status tq_launch_encode_rows(const tq_codebook_s*, const uint16_t*, int64_t, int64_t,
                                const uint8_t*, uint8_t*, uint16_t*, hipStream_t) {
  ++launches;
  return TQ_OK;
}
tq_status tq_launch_append(const tq_kv_cache*, const tq_codebook_s*, const tq_codebook_s*,
                           const uint8_t*, const uint16_t*, const uint16_t*, int, const int32_t*,
                           int, hipStream_t) {
  ++launches;
  return TQ_OK;
}
tq_status tq_launch_prefill(const tq_kv_cache*, const tq_codebook_s*, const tq_codebook_s*,
                            const uint8_t*, const uint16_t*, int, int, const int32_t*, int, float*,
                            hipStream_t) {
  ++launches;
  return TQ_OK;
}
tq_status tq_launch_qjl_encode(const tq_codebook_s*, const uint16_t*, int64_t, int64_t,
                               const uint8_t*, const uint16_t*, const uint8_t*, uint8_t*,
                               uint16_t*, hipStream_t) {
  ++launches;
  return TQ_OK;
}
tq_status tq_launch_qjl_scores(const tq_codebook_s*, const uint16_t*, int, const uint8_t*,
                               const uint16_t*, const uint8_t*, const uint16_t*, const uint8_t*,
                               const uint16_t*, int64_t, float*, hipStream_t) {
  ++launches;
  return TQ_OK;
}
tq_decode_plan tq_plan_decode(const tq_kv_cache* c, int q_heads, int max_len, int n_layers) {
  tq_decode_plan p;
  p.splits = max_len > 4096 ? 4 : 1;
  p.upb = 1;
  p.tiles_per_split = (max_len + 31) / 32;
  p.ctr_bytes = 256;
  p.ws_bytes = p.splits > 1 ? 256 + (size_t)n_layers * c->batch * q_heads * p.splits *
                                        (c->head_dim + 2) * 4
                            : 0;
  return p;
}
tq_status tq_launch_decode(const tq_kv_cache*, const tq_codebook_s*, const tq_codebook_s*,
                           const uint8_t*, const uint16_t*, int, const int32_t*, int, int, float*,
                           void*, const tq_decode_plan&, float, uint32_t*, uint32_t*,
                           hipStream_t) {
  ++launches;
  return TQ_OK;
}

static int scratch_lookups = 0;
tq_status tq_noalloc_scratch(void** out, hipStream_t) {
  ++scratch_lookups;
  *out = (void*)(uintptr_t)0x200000;
  return TQ_OK;
}

#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                      \
    }                                                                \
  } while (0)

/* an address of the given alignment that is never dereferenced */
static void* fake(uintptr_t a) { return (void*)(uintptr_t)(0x100000 + a); }

static tq_kv_cache cache(int d, int bk, int bv, int cap) {
  tq_kv_cache c;
  memset(&c, 0, sizeof c);
  c.k_codes = (uint8_t*)fake(0);
  c.v_codes = (uint8_t*)fake(256);
  c.k_norms = (uint16_t*)fake(512);
  c.v_norms = (uint16_t*)fake(768);
  c.batch = 2;
  c.kv_heads = 4;
  c.head_dim = d;
  c.bits_k = bk;
  c.bits_v = bv;
  c.capacity = cap;
  return c;
}

int main() {
  for (int s = 0; s <= 6; ++s) CHECK(tq_status_str((tq_status)s) != nullptr);
  float cen[16], bnd[15];
  for (int d = 32; d <= 512; d *= 2)
    for (int b = 1; b <= 5; ++b) {
      const tq_status st = tq_codebook_compute(d, b, cen, bnd);
      const bool ok = (d == 64 || d == 128 || d == 256) && b >= 2 && b <= 4;
      CHECK(st == (ok ? TQ_OK : TQ_ERR_UNSUPPORTED));
      if (ok)
        for (int k = 0; k + 1 < (1 << b); ++k) CHECK(cen[k] < bnd[k] && bnd[k] < cen[k + 1]);
    }
  CHECK(tq_codebook_compute(128, 4, nullptr, bnd) == TQ_ERR_ARG);
  /* the codebook build runs its tables on the host, then fails to upload
   * without a device (or succeeds where one is present) */
  for (int d = 64; d <= 256; d *= 2)
    for (int b = 2; b <= 4; ++b) {
      tq_codebook h = nullptr;
      const tq_status st = tq_codebook_init(d, b, &h);
      CHECK(st == TQ_OK || st == TQ_ERR_DEVICE);
      if (st == TQ_OK) tq_codebook_free(h);
      else CHECK(h == nullptr);
    }
  CHECK(tq_codebook_init(96, 4, nullptr) == TQ_ERR_ARG);
  tq_codebook_free(nullptr);
  CHECK(tq_codebook_head_dim(nullptr) == 0 && tq_codebook_bits(nullptr) == 0);

  /* handles built by hand (no device tables; the launchers are stand-ins) */
  static tq_codebook_s ck, cv;
  memset(&ck, 0, sizeof ck);
  memset(&cv, 0, sizeof cv);
  ck.d = cv.d = 128;
  ck.bits = 4;
  cv.bits = 2;
  CHECK(tq_codebook_read(&ck, cen, bnd) == TQ_OK);

  /* encode */
  int before = launches;
  CHECK(tq_encode(&ck, (uint16_t*)fake(16), 10, 128, (uint8_t*)fake(4), (uint8_t*)fake(8),
                  (uint16_t*)fake(2), nullptr) == TQ_OK);
  CHECK(launches == before + 1);
  CHECK(tq_encode(&ck, (uint16_t*)fake(16), 10, 100, (uint8_t*)fake(4), (uint8_t*)fake(8),
                  (uint16_t*)fake(2), nullptr) == TQ_ERR_ARG);
  CHECK(tq_encode(&ck, (uint16_t*)fake(8), 10, 128, (uint8_t*)fake(4), (uint8_t*)fake(8),
                  (uint16_t*)fake(2), nullptr) == TQ_ERR_ARG);
  CHECK(tq_encode(&ck, nullptr, 0, 128, nullptr, nullptr, nullptr, nullptr) == TQ_OK);
  CHECK(launches == before + 1);

  /* cache sizing */
  tq_kv_cache c = cache(128, 4, 2, 1024);
  int64_t a, b2, n1, n2;
  CHECK(tq_cache_layer_bytes(&c, &a, &b2, &n1, &n2) == TQ_OK);
  CHECK(a == 2 * 4 * 1024 * 64 && b2 == 2 * 4 * 1024 * 32 && n1 == 2 * 4 * 1024 * 2);
  tq_kv_cache bad = c;
  bad.capacity = 1000;
  CHECK(tq_cache_layer_bytes(&bad, &a, &b2, &n1, &n2) == TQ_ERR_ARG);
  bad = c;
  bad.capacity = 1 << 25;
  CHECK(tq_cache_layer_bytes(&bad, &a, &b2, &n1, &n2) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_cache_layer_bytes(nullptr, &a, &b2, &n1, &n2) == TQ_ERR_ARG);

  /* append */
  before = launches;
  const uint8_t* sb = (const uint8_t*)fake(4);
  const uint16_t* kn = (const uint16_t*)fake(16);
  const int32_t* pos = (const int32_t*)fake(4);
  CHECK(tq_append(&c, &ck, &cv, sb, kn, kn, 5, pos, 0, 2, nullptr) == TQ_OK);
  CHECK(tq_append(&c, &ck, &cv, sb, kn, kn, 5, pos, -1, 2, nullptr) == TQ_OK);
  CHECK(launches == before + 2);
  CHECK(tq_append(&c, &ck, &cv, sb, kn, kn, 5, pos, 1020, 2, nullptr) == TQ_ERR_CAPACITY);
  CHECK(tq_append(&c, &ck, &cv, sb, kn, kn, 5, pos, 2147483647, 2, nullptr) == TQ_ERR_CAPACITY);
  CHECK(tq_append(&c, &ck, &cv, sb, kn, kn, 5, pos, -2, 2, nullptr) == TQ_ERR_ARG);
  CHECK(tq_append(&c, &cv, &ck, sb, kn, kn, 5, pos, 0, 2, nullptr) == TQ_ERR_ARG);
  CHECK(tq_append(&c, &ck, &cv, sb, kn, kn, 0, pos, 0, 2, nullptr) == TQ_OK);
  CHECK(launches == before + 2);

  /* decode, sparse decode, prefill */
  before = launches;
  const uint16_t* q = (const uint16_t*)fake(16);
  float* out = (float*)fake(16);
  const int32_t* lens = (const int32_t*)fake(4);
  const size_t ws = tq_decode_workspace_bytes(&c, 16, 1024, 2);
  CHECK(ws == 0);
  CHECK(tq_decode_attn(&c, &ck, &cv, sb, q, 16, lens, 1024, 2, out, nullptr, 0, nullptr) == TQ_OK);
  c.capacity = 8192;
  const size_t ws2 = tq_decode_workspace_bytes(&c, 16, 8192, 2);
  CHECK(ws2 > 0);
  CHECK(tq_decode_attn(&c, &ck, &cv, sb, q, 16, lens, 8192, 2, out, nullptr, 0, nullptr) ==
        TQ_ERR_WORKSPACE);
  CHECK(tq_decode_attn(&c, &ck, &cv, sb, q, 16, lens, 8192, 2, out, fake(256), ws2, nullptr) ==
        TQ_OK);
  CHECK(tq_decode_attn(&c, &ck, &cv, sb, q, 16, lens, 8192, 2, out, fake(128), ws2, nullptr) ==
        TQ_ERR_WORKSPACE);
  CHECK(tq_decode_attn(&c, &ck, &cv, sb, q, 10, lens, 8192, 2, out, fake(256), ws2, nullptr) ==
        TQ_ERR_ARG);
  CHECK(tq_decode_attn(&c, &ck, &cv, sb, q, 64, lens, 8192, 2, out, fake(256), ws2, nullptr) ==
        TQ_ERR_UNSUPPORTED);
  CHECK(tq_decode_attn_sparse(&c, &ck, &cv, sb, q, 16, lens, 8192, 2, 1e-4f, (uint32_t*)fake(4),
                              (uint32_t*)fake(4), out, fake(256), ws2, nullptr) == TQ_OK);
  CHECK(tq_decode_attn_sparse(&c, &ck, &cv, sb, q, 16, lens, 8192, 2, NAN, nullptr, nullptr, out,
                              fake(256), ws2, nullptr) == TQ_ERR_ARG);
  CHECK(tq_decode_attn_sparse(&c, &ck, &cv, sb, q, 16, lens, 8192, 2, 1e-4f, nullptr,
                              (uint32_t*)fake(2), out, fake(256), ws2, nullptr) == TQ_ERR_ARG);
  CHECK(tq_decode_attn_noalloc(&c, &ck, &cv, sb, q, 16, lens, 8192, 2, out, nullptr) == TQ_OK);
  CHECK(scratch_lookups == 1);
  CHECK(tq_decode_attn_noalloc(&c, &ck, &cv, sb, q, 10, lens, 8192, 2, out, nullptr) == TQ_ERR_ARG);
  CHECK(tq_decode_attn_noalloc(&c, &ck, &cv, sb, q, 16, lens, 8192, 4096, out, nullptr) ==
        TQ_ERR_WORKSPACE); /* records of 4096 layers exceed the library's array */
  CHECK(scratch_lookups == 1);
  CHECK(tq_prefill_attn(&c, &ck, &cv, sb, q, 16, 7, pos, 2, out, nullptr) == TQ_OK);
  CHECK(tq_prefill_attn(&c, &ck, &cv, sb, q, 16, -1, pos, 2, out, nullptr) == TQ_ERR_ARG);
  CHECK(launches == before + 5);

  /* paged caches */
  tq_kv_cache p = cache(128, 4, 2, 1024);
  p.block_table = (const int32_t*)fake(4);
  p.page_tokens = 256;
  p.max_pages = 4;
  p.num_pages = 10;
  CHECK(tq_cache_layer_bytes(&p, &a, &b2, &n1, &n2) == TQ_OK && a == 10 * 4 * 256 * 64);
  p.page_tokens = 96;
  CHECK(tq_cache_layer_bytes(&p, &a, &b2, &n1, &n2) == TQ_ERR_ARG);
  p.page_tokens = 256;
  p.num_pages = 1 << 17;
  CHECK(tq_cache_layer_bytes(&p, &a, &b2, &n1, &n2) == TQ_ERR_UNSUPPORTED);

  /* QJL */
  before = launches;
  CHECK(tq_qjl_encode(&ck, kn, 10, 128, sb, kn, (uint8_t*)fake(8), (uint8_t*)fake(4),
                      (uint16_t*)fake(2), nullptr) == TQ_OK);
  CHECK(tq_qjl_scores(&ck, q, 4, sb, kn, (uint8_t*)fake(8), (uint16_t*)fake(2), (uint8_t*)fake(4),
                      (uint16_t*)fake(2), 10, out, nullptr) == TQ_OK);
  CHECK(tq_qjl_scores(&ck, q, 9, sb, kn, (uint8_t*)fake(8), (uint16_t*)fake(2), (uint8_t*)fake(4),
                      (uint16_t*)fake(2), 10, out, nullptr) == TQ_ERR_UNSUPPORTED);
  CHECK(launches == before + 2);
  printf("host harness ok\n");
  return 0;
}
