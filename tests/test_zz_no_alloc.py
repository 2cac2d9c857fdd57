"""tq_decode_attn_noalloc (the decode for callers that cannot allocate: the
split workspace is the library's own device array) against tq_decode_attn
with a caller workspace, through the C ABI: two calls in a row, the second
with a smaller input, each bit-identical to the workspace path (same kernels,
same split plan, so the same arithmetic), plus a call whose workspace would
exceed the library's array, rejected before any launch."""
import ctypes

import numpy as np
import pytest

import kv_cache_quantization_tq_amd as tq
import synth
from helpers import require_gpu

pytestmark = pytest.mark.gpu
SEED = 1021


def _case(torch, L, B, H, G, d, bk, bv, T):
    cache = tq.KVCache(L, B, H, d, bk, bv, ((T + 31) // 32) * 32)
    sbd = torch.from_numpy(np.stack([synth.sign_bits(SEED, l, d) for l in range(L)])).cuda()
    cbk, cbv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    for l in range(L):
        k = torch.empty((1, B, H, T, d), dtype=torch.int16, device="cuda")
        v = torch.empty_like(k)
        synth.kv_dev(SEED, 0, l, k[0])
        synth.kv_dev(SEED, 1, l, v[0])
        tq.append(cache, cbk, cbv, sbd[l:l + 1], k, v,
                  torch.zeros(B, dtype=torch.int32, device="cuda"), host_max_pos=0, layer0=l,
                  n_layers=1)
    q = torch.empty((L, B, G * H, d), dtype=torch.int16, device="cuda")
    for l in range(L):
        synth.q_dev(SEED, 0, l, q[l])
    return cache, sbd, cbk, cbv, q


def test_noalloc_equals_workspace_decode():
    torch = require_gpu()
    # a larger call, then a smaller one (fewer layers, sequences and tokens)
    for L, B, H, G, d, bk, bv, lens in ((2, 2, 2, 4, 128, 4, 2, [6000, 3100]),
                                        (1, 1, 2, 8, 64, 3, 3, [2500])):
        T = max(lens)
        cache, sbd, cbk, cbv, q = _case(torch, L, B, H, G, d, bk, bv, T)
        lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
        assert tq.decode_workspace_bytes(cache, G * H, T) > 0, "the case must use split records"
        ref = torch.empty((L, B, G * H, d), dtype=torch.float32, device="cuda")
        tq.decode(cache, cbk, cbv, sbd, q, lens_d, T, ref, tq.workspace(cache, G * H, T))
        got = torch.full_like(ref, float("nan"))
        tq.decode_noalloc(cache, cbk, cbv, sbd, q, lens_d, T, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (L, B, H, G, d, lens)
        # a repeat on the same array (its counters returned to zero)
        got.fill_(float("nan"))
        tq.decode_noalloc(cache, cbk, cbv, sbd, q, lens_d, T, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), ("repeat", L, B, H, G, d, lens)


def _plan_bytes(B, H, G, d, T):
    """The decode workspace of a (1-layer) shape, from the planner alone (a
    cache description with placeholder addresses; nothing is touched)."""
    s = tq.KVCacheStruct()
    s.k_codes = s.v_codes = s.k_norms = s.v_norms = 1 << 20
    s.batch, s.kv_heads, s.head_dim, s.bits_k, s.bits_v, s.capacity = B, H, d, 4, 2, T
    return tq.lib().tq_decode_workspace_bytes(ctypes.byref(s), G * H, T, 1)


def test_noalloc_rejects_oversized_workspace():
    """A shape whose split records exceed the library's 16 MiB array: the call
    returns TQ_ERR_WORKSPACE and launches nothing (the output keeps its
    contents).  Every buffer is allocated for the shape, so the call's
    arguments are valid in full."""
    torch = require_gpu()
    # many units just short of full rounds of blocks take the most split
    # records: about 1840 (layer, sequence, KV head) units at 2 splits
    H, G, d, T = 8, 8, 256, 1024
    B = next((b for b in range(200, 260) if _plan_bytes(b, H, G, d, T) > 16 << 20), None)
    if B is None:
        pytest.skip("no batch size in 200..259 needs more than 16 MiB of split records here")
    cache = tq.KVCache(1, B, H, d, 4, 2, T)
    sbd = torch.from_numpy(synth.sign_bits(SEED, 0, d)[None]).cuda()
    cbk, cbv = tq.Codebook(d, 4), tq.Codebook(d, 2)
    q = torch.zeros((1, B, G * H, d), dtype=torch.int16, device="cuda")
    out = torch.full((1, B, G * H, d), 7.0, dtype=torch.float32, device="cuda")
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    assert tq.decode_workspace_bytes(cache, G * H, T) > 16 << 20
    with pytest.raises(tq.TQError) as e:
        tq.decode_noalloc(cache, cbk, cbv, sbd, q, lens, T, out)
    assert e.value.code == 4  # TQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
