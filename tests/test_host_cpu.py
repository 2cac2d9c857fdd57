"""Host-side checks that need no GPU: the C ABI loads and exports every
declared symbol, argument validation happens before any device work, the
library's codebook agrees with the oracle's, and the decode planning."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import kv_cache_quantization_tq_amd as tq
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", src)))


def test_header_declarations_are_exported():
    names = _declared()
    assert set(names) == set(tq.EXPORTS)
    L = tq.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = tq.lib()
    for code, name in tq.STATUS.items():
        assert L.tq_status_str(code).decode() == name


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_library_codebook_matches_oracle(d, bits):
    """Independent Lloyd-Max implementations (erfc closed forms vs Simpson
    quadrature) agree to fp32 rounding."""
    c, t = tq.codebook_compute(d, bits)
    oc, ot = oracle.codebook(d, bits)
    assert np.abs(np.array(c) - oc).max() <= 1e-7 * np.abs(oc).max()
    assert np.abs(np.array(t) - ot).max() <= 1e-7 * np.abs(oc).max()


def test_codebook_compute_rejects_unsupported():
    L = tq.lib()
    buf = (ctypes.c_float * 16)()
    assert L.tq_codebook_compute(96, 4, buf, buf) == 2
    assert L.tq_codebook_compute(128, 5, buf, buf) == 2
    assert L.tq_codebook_compute(128, 4, None, buf) == 1


def _fake_cache(**kw):
    s = tq.KVCacheStruct()
    s.k_codes = s.v_codes = s.k_norms = s.v_norms = 1 << 20
    s.batch, s.kv_heads, s.head_dim, s.bits_k, s.bits_v, s.capacity = 1, 8, 128, 4, 2, 1024
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def test_validation_before_device_work():
    """Bad caches and sizes are rejected on the host (no GPU is touched)."""
    L = tq.lib()
    vp = ctypes.c_void_p
    bad = [dict(capacity=1000), dict(head_dim=96), dict(bits_k=5), dict(batch=0),
           dict(k_codes=(1 << 20) + 4), dict(layer_stride_k_codes=8),
           dict(capacity=1 << 25)]  # one stream of key codes reaches 2 GiB
    for kw in bad:
        s = _fake_cache(**kw)
        rc = L.tq_append(ctypes.byref(s), None, None, vp(1), vp(16), vp(16), 1, vp(4), 0, 1, None)
        assert rc in (1, 2), kw
        rc = L.tq_decode_attn(ctypes.byref(s), None, None, vp(1), vp(16), 8, vp(4), 16, 1, vp(16),
                              None, 0, None)
        assert rc in (1, 2), kw
    s = _fake_cache()
    # group size 16 is unsupported; q_heads not a multiple of kv_heads is an error
    assert L.tq_decode_attn(ctypes.byref(s), None, None, vp(1), vp(16), 128, vp(4), 16, 1, vp(16),
                            None, 0, None) == 2
    assert L.tq_decode_attn(ctypes.byref(s), None, None, vp(1), vp(16), 12, vp(4), 16, 1, vp(16),
                            None, 0, None) == 1
    # max_len beyond capacity
    assert L.tq_decode_attn(ctypes.byref(s), None, None, vp(1), vp(16), 32, vp(4), 2048, 1,
                            vp(16), None, 0, None) == 1
    # null codebook handles
    assert L.tq_encode(None, vp(16), 4, 128, vp(1), vp(16), vp(16), None) == 1
    assert L.tq_append(ctypes.byref(s), None, None, vp(1), vp(16), vp(16), 1, vp(4), 0, 1,
                       None) == 1


def test_sparse_decode_validation():
    """tq_decode_attn_sparse rejects a NaN, negative or infinite threshold and a
    misaligned count array or skip bitmap before anything else (an
    unsupported head dim would otherwise answer TQ_ERR_UNSUPPORTED); valid
    thresholds reach the ordinary checks."""
    L = tq.lib()
    vp = ctypes.c_void_p
    s = _fake_cache(head_dim=96)
    def call(eps, counts=None, tiles=None):
        return L.tq_decode_attn_sparse(ctypes.byref(s), None, None, vp(1), vp(16), 8, vp(4), 16,
                                       1, eps, counts, tiles, vp(16), None, 0, None)
    for eps in (float("nan"), -1e-6, float("inf")):
        assert call(eps) == 1, eps
    assert call(1e-6, vp(2)) == 1
    assert call(1e-6, None, vp(6)) == 1
    for eps in (0.0, 1e-6, 1.0, 3.0):
        assert call(eps) == 2, eps
        assert call(eps, vp(4), vp(8)) == 2, eps


def test_prefill_validation():
    """tq_prefill_attn checks the cache, the group size and t_new before any
    device work."""
    L = tq.lib()
    vp = ctypes.c_void_p
    for kw in (dict(capacity=1000), dict(head_dim=96), dict(bits_v=1)):
        s = _fake_cache(**kw)
        assert L.tq_prefill_attn(ctypes.byref(s), None, None, vp(1), vp(16), 8, 4, vp(4), 1,
                                 vp(16), None) in (1, 2), kw
    s = _fake_cache()
    assert L.tq_prefill_attn(ctypes.byref(s), None, None, vp(1), vp(16), 12, 4, vp(4), 1,
                             vp(16), None) == 1          # q_heads not a multiple of kv_heads
    assert L.tq_prefill_attn(ctypes.byref(s), None, None, vp(1), vp(16), 128, 4, vp(4), 1,
                             vp(16), None) == 2          # group of 16
    assert L.tq_prefill_attn(ctypes.byref(s), None, None, vp(1), vp(16), 8, -1, vp(4), 1,
                             vp(16), None) == 1          # negative t_new
    assert L.tq_prefill_attn(ctypes.byref(s), None, None, vp(1), vp(16), 8, 4, vp(4), 0,
                             vp(16), None) == 1          # no layers


def test_qjl_validation():
    """The QJL entry points reject null handles and pointers, misaligned
    buffers and unsupported query counts before any device work."""
    L = tq.lib()
    vp = ctypes.c_void_p
    assert L.tq_qjl_encode(None, vp(16), 4, 128, vp(4), vp(16), vp(16), vp(16), vp(16), None) == 1
    assert L.tq_qjl_scores(None, vp(16), 4, vp(4), vp(16), vp(16), vp(16), vp(16), vp(16), 8,
                           vp(16), None) == 1
    assert L.tq_qjl_encode(None, vp(16), -1, 128, vp(4), vp(16), vp(16), vp(16), vp(16), None) == 1


def test_workspace_planning():
    L = tq.lib()
    s = _fake_cache(capacity=32768)
    # one layer, 8 KV heads, 32K tokens: several splits -> records of (d + 2) floats
    nb = L.tq_decode_workspace_bytes(ctypes.byref(s), 32, 32768, 1)
    assert nb > 0 and (nb - 256) % (32 * 130 * 4) == 0
    # many units -> one split, no workspace
    s.batch = 64
    assert L.tq_decode_workspace_bytes(ctypes.byref(s), 32, 8192, 32) == 0
    # layer bytes: the page's 100 B per token per KV head at d = 128, K4/V2
    s = _fake_cache(batch=1, kv_heads=1, capacity=32)
    k, v, kn, vn = (ctypes.c_int64() for _ in range(4))
    assert L.tq_cache_layer_bytes(ctypes.byref(s), ctypes.byref(k), ctypes.byref(v),
                                  ctypes.byref(kn), ctypes.byref(vn)) == 0
    assert (k.value + v.value + kn.value + vn.value) // 32 == 100


def _paged(**kw):
    s = _fake_cache(capacity=1024)
    s.block_table = 1 << 16
    s.page_tokens, s.max_pages, s.num_pages = 256, 4, 10
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def test_paged_cache_layer_bytes():
    """Paged storage: the layer arrays are the page pools."""
    L = tq.lib()
    s = _paged()
    kc, vc, kn, vn = (ctypes.c_int64() for _ in range(4))
    assert L.tq_cache_layer_bytes(ctypes.byref(s), ctypes.byref(kc), ctypes.byref(vc),
                                  ctypes.byref(kn), ctypes.byref(vn)) == 0
    rows = 10 * 8 * 256
    assert (kc.value, vc.value, kn.value, vn.value) == (rows * 64, rows * 32, rows * 2, rows * 2)


def test_paged_validation():
    """Bad paging parameters are rejected on the host."""
    L = tq.lib()
    vp = ctypes.c_void_p
    bad = [dict(page_tokens=96), dict(page_tokens=16, max_pages=64), dict(max_pages=3),
           dict(num_pages=0), dict(block_table=(1 << 16) + 2)]
    for kw in bad:
        s = _paged(**kw)
        rc = L.tq_append(ctypes.byref(s), None, None, vp(1), vp(16), vp(16), 1, vp(4), 0, 1, None)
        assert rc == 1, kw
        rc = L.tq_decode_attn(ctypes.byref(s), None, None, vp(1), vp(16), 8, vp(4), 16, 1, vp(16),
                              None, 0, None)
        assert rc == 1, kw
    # a layer's pool of 2 GiB or more is unsupported
    s = _paged(num_pages=1 << 17)
    assert L.tq_decode_attn(ctypes.byref(s), None, None, vp(1), vp(16), 8, vp(4), 16, 1, vp(16),
                            None, 0, None) == 2


_ROWS_HARNESS = r"""
#define __host__
#define __device__
#include <stdio.h>
#include "tq_append_rows.h"
int main(void) {
  long long p0, t_new, cap, slot;
  while (scanf("%lld %lld %lld %lld", &p0, &t_new, &cap, &slot) == 4) {
    int32_t tile, jlo, jhi;
    bool ok = tq_append_tile_rows((int32_t)p0, (int32_t)t_new, (int32_t)cap, (int32_t)slot,
                                  &tile, &jlo, &jhi);
    const int32_t fe = tq_append_full_end((int32_t)p0, (int32_t)t_new, (int32_t)cap);
    const bool nf = ok && tq_append_next_full(tile, jlo, jhi, fe, 2);
    printf("%d %d %d %d %d\n", ok ? 1 : 0, tile, jlo, jhi, nf ? 1 : 0);
  }
  return 0;
}
"""


def test_append_tile_rows_arithmetic(tmp_path):
    """The append kernel's per-slot row arithmetic (tq_append_rows.h, compiled
    here for the host) against a brute-force statement of what an append
    writes: rows p0 .. p0 + t_new - 1 that are below capacity, cut into
    32-token tiles; and its shortcut for a wave's next task (the slot two
    further on), taken exactly when both tiles are written in all 32 rows.  Includes positions within 64 of INT32_MAX, where 32-bit
    row arithmetic would wrap and write far past the stream."""
    import subprocess
    src = tmp_path / "rows.cpp"
    src.write_text(_ROWS_HARNESS)
    exe = tmp_path / "rows"
    inc = os.path.join(ROOT, "kv_cache_quantization_tq_amd", "csrc")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", inc, str(src), "-o", str(exe)], check=True)
    imax = 2 ** 31 - 1
    cases = []
    rng = np.random.default_rng(9)
    for cap in (32, 2048, 32768, 1 << 26):
        starts = [0, 1, 31, 32, cap - 33, cap - 1, cap, cap + 5, -1, -40]
        starts += list(range(imax - 64, imax + 1, 7)) + [imax - 4, imax]
        starts += rng.integers(0, cap, 5).tolist()
        for p0 in starts:
            for t_new in (1, 7, 8, 32, 40, 2049, imax - 3):
                nslots = min((t_new + 31) // 32 + 1, 70)
                for slot in sorted(set(list(range(min(nslots, 6))) + [nslots - 3, nslots - 1])):
                    cases.append((p0, t_new, cap, slot))
    inp = "\n".join(" ".join(map(str, c)) for c in cases) + "\n"
    res = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True)
    lines = res.stdout.split("\n")
    got = {}
    for (p0, t_new, cap, slot), line in zip(cases, lines):
        got[(p0, t_new, cap, slot)] = tuple(map(int, line.split()))
    for (p0, t_new, cap, slot), line in zip(cases, lines):
        ok, tile, jlo, jhi, nf = map(int, line.split())
        # brute force: appended rows below capacity, within this slot's tile
        want = None
        if 0 <= p0 < cap:
            t = p0 // 32 + slot
            lo, hi = max(p0, 32 * t), min(p0 + t_new, 32 * t + 32, cap)
            if hi > lo:
                want = (t, lo - 32 * t, hi - 32 * t)
        if want is None:
            assert ok == 0, (p0, t_new, cap, slot, line)
        else:
            assert ok == 1 and (tile, jlo, jhi) == want, (p0, t_new, cap, slot, line, want)
            assert 32 * tile + jhi <= cap and 0 <= jlo < jhi <= 32
        # the kernel's shortcut: when tq_append_next_full says so, the slot two
        # further on is the next-but-one tile, written in all 32 rows
        full2 = (0 <= p0 < cap and 32 * (p0 // 32 + slot + 2) >= p0
                 and 32 * (p0 // 32 + slot + 2) + 32 <= min(p0 + t_new, cap))
        if nf:
            assert want is not None and (want[1], want[2]) == (0, 32) and full2, \
                (p0, t_new, cap, slot, line)
        elif want is not None and (want[1], want[2]) == (0, 32) and full2:
            raise AssertionError(("shortcut missed", p0, t_new, cap, slot, line))
        if (p0, t_new, cap, slot + 2) in got and nf:
            assert got[(p0, t_new, cap, slot + 2)][:4] == (1, tile + 2, 0, 32), \
                (p0, t_new, cap, slot, got[(p0, t_new, cap, slot + 2)])
    assert len(lines) >= len(cases)
