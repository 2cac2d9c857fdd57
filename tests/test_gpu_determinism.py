"""Repeated launches give bit-identical results.  Each kernel runs on the same
inputs twice, with launches of other kernels and shapes (other LDS contents,
other workspace use) in between.  A kernel that read LDS, registers or
workspace it had not written in the same launch, or whose waves or blocks
raced, would show up here as a difference; the parity tests, which compare
with the oracle within tolerances, could miss a small one."""
import numpy as np
import pytest

import kv_cache_quantization_tq_amd as tq
import synth
from helpers import require_gpu

pytestmark = pytest.mark.gpu
SEED = 1009

# few long units (the decode splits the context and merges through the
# workspace), many short units, and 256-dim heads
CONFIGS = [
    dict(d=128, bk=4, bv=2, L=1, B=1, H=2, G=4, T=8192),
    dict(d=64, bk=3, bv=3, L=4, B=8, H=4, G=8, T=300),
    dict(d=256, bk=2, bv=4, L=1, B=2, H=2, G=2, T=2000),
]
T_NEW = 64


def _setup(torch, c):
    d, L, B, H, G, T = c["d"], c["L"], c["B"], c["H"], c["G"], c["T"]
    cache = tq.KVCache(L, B, H, d, c["bk"], c["bv"], (T + 31) // 32 * 32)
    cbk, cbv = tq.Codebook(d, c["bk"]), tq.Codebook(d, c["bv"])
    sbd = torch.from_numpy(np.stack([synth.sign_bits(SEED, l, d) for l in range(L)])).cuda()
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    for l in range(L):
        k = torch.empty((1, B, H, T, d), dtype=torch.int16, device="cuda")
        v = torch.empty_like(k)
        synth.kv_dev(SEED, 0, l, k[0])
        synth.kv_dev(SEED, 1, l, v[0])
        tq.append(cache, cbk, cbv, sbd[l:l + 1], k, v, zero, host_max_pos=0, layer0=l,
                  n_layers=1)
    q = torch.empty((L, B, H * G, d), dtype=torch.int16, device="cuda")
    qp = torch.empty((L, B, H * G, T_NEW, d), dtype=torch.int16, device="cuda")
    qs = torch.empty((B, H * G, d), dtype=torch.int16, device="cuda")
    for l in range(L):
        synth.q_dev(SEED, 7, l, q[l])
        for i in range(T_NEW):
            synth.q_dev(SEED, 100 + i, l, qs)
            qp[l, :, :, i] = qs
    # ragged lengths for the decode; the prefill's new tokens are the last T_NEW
    lens = torch.tensor([T - 37 * b for b in range(B)], dtype=torch.int32, device="cuda")
    pos = torch.tensor([T - T_NEW] * B, dtype=torch.int32, device="cuda")
    return dict(cache=cache, cbk=cbk, cbv=cbv, sbd=sbd, q=q, qp=qp, lens=lens, pos=pos,
                ws=tq.workspace(cache, H * G, T), **c)


def _run(torch, s):
    """Dense decode, Sparse V decode (with its skip bitmap) and prefill."""
    L, B, H, G, d, T = s["L"], s["B"], s["H"], s["G"], s["d"], s["T"]
    out = torch.empty((L, B, H * G, d), dtype=torch.float32, device="cuda")
    tq.decode(s["cache"], s["cbk"], s["cbv"], s["sbd"], s["q"], s["lens"], T, out, s["ws"])
    outs = torch.empty_like(out)
    tiles = torch.zeros((L, B, H, tq.skip_words(T)), dtype=torch.int32, device="cuda")
    tq.decode_sparse(s["cache"], s["cbk"], s["cbv"], s["sbd"], s["q"], s["lens"], T, outs, 1e-4,
                     s["ws"], skip_tiles=tiles)
    outp = torch.empty((L, B, H * G, T_NEW, d), dtype=torch.float32, device="cuda")
    tq.prefill(s["cache"], s["cbk"], s["cbv"], s["sbd"], s["qp"], s["pos"], outp)
    torch.cuda.synchronize()
    return [out, outs, tiles, outp]


def test_repeat_launches_bit_identical():
    torch = require_gpu()
    states = [_setup(torch, c) for c in CONFIGS]
    first = [_run(torch, s) for s in states]
    # again, in the opposite order, so that every launch follows other shapes
    second = [_run(torch, s) for s in reversed(states)][::-1]
    for c, a, b in zip(CONFIGS, first, second):
        for name, x, y in (("decode", a[0], b[0]), ("prefill", a[3], b[3])):
            assert torch.isfinite(x).all(), (c, name)
            assert torch.equal(x, y), (c, name, float((x - y).abs().max()))
        # Sparse V: which tiles a launch skips depends on when its waves see
        # each other's running maxima (a race by design, on a reference that
        # is valid either way), so only launches that skipped the same tiles
        # must agree bit for bit
        if torch.equal(a[2], b[2]):
            assert torch.equal(a[1], b[1]), (c, "sparse decode", float((a[1] - b[1]).abs().max()))
        print(f"{c}: sparse skip bitmaps {'equal' if torch.equal(a[2], b[2]) else 'differ'}")


def test_qjl_repeat_bit_identical():
    torch = require_gpu()
    d, bits, n, G = 128, 4, 3000, 4
    rng = np.random.default_rng(5)
    cb = tq.Codebook(d, bits)
    xd = torch.from_numpy(synth.kv_host(SEED, 0, 0, 0, 0, d, 0, n).view(np.int16)).cuda()
    sbd = torch.from_numpy(synth.sign_bits(SEED, 0, d)).cuda()
    S16 = rng.standard_normal((d, d)).astype(np.float16)
    Sd = torch.from_numpy(S16.view(np.int16)).cuda()
    qd = torch.from_numpy(np.stack([synth.q_host(SEED, 0, 0, 0, g, d)
                                    for g in range(G)]).view(np.int16)).cuda()
    codes = torch.empty((n, d * bits // 8), dtype=torch.uint8, device="cuda")
    norms = torch.empty(n, dtype=torch.int16, device="cuda")
    tq.encode(cb, xd, sbd, codes, norms)
    res = []
    other = _setup(torch, CONFIGS[1])
    for rep in range(2):
        signs = torch.empty((n, d // 8), dtype=torch.uint8, device="cuda")
        gamma = torch.empty(n, dtype=torch.int16, device="cuda")
        out = torch.empty((G, n), dtype=torch.float32, device="cuda")
        tq.qjl_encode(cb, xd, sbd, Sd, codes, signs, gamma)
        tq.qjl_scores(cb, qd, sbd, Sd, codes, norms, signs, gamma, out)
        torch.cuda.synchronize()
        res.append((signs, gamma, out))
        _run(torch, other)  # other kernels between the two
    for x, y in zip(*res):
        assert torch.equal(x, y)
