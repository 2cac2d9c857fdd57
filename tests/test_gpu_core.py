"""GPU parity of the HIP path against the CPU oracle on small shapes that span
several tiles and ragged tails: encode (codes, norms), append (== encode, bit
for bit, nothing else touched) and decode attention."""
import math

import numpy as np
import pytest

import kv_cache_quantization_tq_amd as tq
import oracle
import synth
from helpers import (attention_errors, check_attention, compare_codes,
                     oracle_attention_with_bound, require_gpu)

pytestmark = pytest.mark.gpu
SEED = 1001


def _dev_kv(torch, seed, kind, layer, B, H, nt, d):
    t = torch.empty((B, H, nt, d), dtype=torch.int16, device="cuda")
    synth.kv_dev(seed, kind, layer, t)
    return t


def test_generator_device_matches_host():
    torch = require_gpu()
    d = 128
    t = _dev_kv(torch, SEED, 1, 3, 2, 3, 200, d)
    torch.cuda.synchronize()
    got = t.cpu().numpy().view(np.uint16)
    for b in range(2):
        for h in range(3):
            ref = synth.kv_host(SEED, 1, 3, b, h, d, 0, 200)
            assert np.array_equal(got[b, h], ref)
    q = torch.empty((2, 4, d), dtype=torch.int16, device="cuda")
    synth.q_dev(SEED, 5, 3, q)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy().view(np.uint16)[1, 2], synth.q_host(SEED, 5, 3, 1, 2, d))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_encode_parity(d, bits):
    torch = require_gpu()
    n = 3001
    x = synth.kv_host(SEED, 0, d, bits, 0, d, 0, n)
    sb = synth.sign_bits(SEED, 7, d)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    cb = tq.Codebook(d, bits)
    codes = torch.empty((n, d * bits // 8), dtype=torch.uint8, device="cuda")
    norms = torch.empty(n, dtype=torch.int16, device="cuda")
    tq.encode(cb, xd, torch.from_numpy(sb).cuda(), codes, norms)
    torch.cuda.synchronize()
    oc, on, ob = oracle.encode(x, bits, sb)
    assert np.array_equal(norms.cpu().numpy().view(np.uint16), on)
    gc = oracle.unpack_rows(codes.cpu().numpy(), d, bits)
    compare_codes(gc, oc, ob, f"d={d} b={bits}")


def test_encode_special_vectors():
    """Zero vectors, exact-midpoint norms, subnormals, fp16 extremes, a single
    spike, and a row stride larger than d."""
    torch = require_gpu()
    d, bits = 128, 4
    rows = []
    rows.append(np.zeros(d, np.float16))
    r = np.zeros(d, np.float16); r[3], r[77] = 1233, 1644; rows.append(r)       # norm 2055: tie
    r = np.zeros(d, np.float16); r[0], r[1] = 1239, 1652; rows.append(r)        # norm 2065: tie
    r = np.zeros(d, np.float16); r[5] = 2 ** -24; rows.append(r)                # one subnormal
    r = np.full(d, 2 ** -24, np.float16); rows.append(r)                        # all subnormal
    r = np.zeros(d, np.float16); r[9] = -65504; rows.append(r)                  # extreme
    r = np.full(d, 3000, np.float16); rows.append(r)                            # large norm
    r = np.zeros(d, np.float16); r[100] = 1.0; rows.append(r)                   # spike
    rng = np.random.default_rng(3)
    for _ in range(57):
        rows.append((rng.standard_normal(d) * 10 ** rng.uniform(-6, 3)).astype(np.float16))
    x = np.stack(rows).view(np.uint16)
    n = x.shape[0]
    sb = synth.sign_bits(SEED, 2, d)
    stride = d + 64
    buf = np.zeros((n, stride), np.uint16)
    buf[:, :d] = x
    xd = torch.from_numpy(buf.view(np.int16)).cuda()
    cb = tq.Codebook(d, bits)
    codes = torch.empty((n, d * bits // 8), dtype=torch.uint8, device="cuda")
    norms = torch.empty(n, dtype=torch.int16, device="cuda")
    tq.encode(cb, xd, torch.from_numpy(sb).cuda(), codes, norms)
    torch.cuda.synchronize()
    oc, on, ob = oracle.encode(x, bits, sb)
    assert np.array_equal(norms.cpu().numpy().view(np.uint16), on)
    gc = oracle.unpack_rows(codes.cpu().numpy(), d, bits)
    # structured rows (constant vectors, a spike) put coordinates exactly on
    # thresholds, where either neighbouring code is correct: band check only
    compare_codes(gc, oc, ob, "special", max_frac=None)
    assert np.all(gc[0] == 7)


@pytest.mark.parametrize("d,bk,bv", [(128, 4, 3), (128, 3, 2), (64, 4, 2), (256, 2, 4)])
def test_append_equals_encode(d, bk, bv):
    """Chunked appends at ragged positions write exactly tq_encode's codes (keys
    as rows, values rearranged into tiles) and leave every other byte alone."""
    torch = require_gpu()
    Lyr, B, H, cap = 2, 2, 2, 2304
    start = [0, 45]
    chunks = [1, 7, 31, 33, 2049, 1]
    total = sum(chunks)
    cache = tq.KVCache(Lyr, B, H, d, bk, bv, cap)
    g = torch.Generator(device="cuda").manual_seed(0)
    for t in (cache.k_codes, cache.v_codes):
        t.copy_(torch.randint(0, 256, t.shape, dtype=torch.uint8, device="cuda", generator=g))
    for t in (cache.k_norms, cache.v_norms):
        t.copy_(torch.randint(-2 ** 15, 2 ** 15, t.shape, dtype=torch.int16, device="cuda",
                              generator=g))
    before = [t.clone() for t in (cache.k_codes, cache.v_codes, cache.k_norms, cache.v_norms)]
    sbs = np.stack([synth.sign_bits(SEED, l, d) for l in range(Lyr)])
    sbd = torch.from_numpy(sbs).cuda()
    cbk, cbv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    kall = torch.stack([_dev_kv(torch, SEED, 0, l, B, H, total, d) for l in range(Lyr)])
    vall = torch.stack([_dev_kv(torch, SEED, 1, l, B, H, total, d) for l in range(Lyr)])
    off = 0
    for c in chunks:
        pos = torch.tensor([start[b] + off for b in range(B)], dtype=torch.int32, device="cuda")
        tq.append(cache, cbk, cbv, sbd, kall[:, :, :, off:off + c].contiguous(),
                  vall[:, :, :, off:off + c].contiguous(), pos,
                  host_max_pos=max(start) + off)
        off += c
    torch.cuda.synchronize()
    for l in range(Lyr):
        for b in range(B):
            for h in range(H):
                rows = slice(start[b], start[b] + total)
                for kind, cb, bits in ((0, cbk, bk), (1, cbv, bv)):
                    src = (kall if kind == 0 else vall)[l, b, h]
                    codes = torch.empty((total, d * bits // 8), dtype=torch.uint8, device="cuda")
                    norms = torch.empty(total, dtype=torch.int16, device="cuda")
                    tq.encode(cb, src, sbd[l], codes, norms)
                    torch.cuda.synchronize()
                    ref = codes.cpu().numpy()
                    nrm = (cache.k_norms if kind == 0 else cache.v_norms)[l, b, h].cpu().numpy()
                    assert np.array_equal(nrm[rows], norms.cpu().numpy())
                    old = before[2 + kind][l, b, h].cpu().numpy()
                    keep = np.ones(cap, bool)
                    keep[rows] = False
                    assert np.array_equal(nrm[keep], old[keep])
                    if kind == 0:
                        got = cache.k_codes[l, b, h].cpu().numpy()
                        assert np.array_equal(got[rows], ref)
                        assert np.array_equal(got[keep], before[0][l, b, h].cpu().numpy()[keep])
                    else:
                        tiles = cache.v_codes[l, b, h].cpu().numpy()
                        got = oracle.unpack_vtiles(tiles, d, bits)
                        want = oracle.unpack_rows(ref, d, bits)
                        assert np.array_equal(got[rows], want)
                        old_codes = oracle.unpack_vtiles(before[1][l, b, h].cpu().numpy(), d, bits)
                        assert np.array_equal(got[keep], old_codes[keep])


def _decode_case(torch, d, bk, bv, G, lens, Lyr=2, H=2, seed=SEED):
    B = len(lens)
    T = max(lens)
    cap = ((T + 31) // 32) * 32 + 32
    Hq = G * H
    cache = tq.KVCache(Lyr, B, H, d, bk, bv, cap)
    sbs = np.stack([synth.sign_bits(seed, l, d) for l in range(Lyr)])
    sbd = torch.from_numpy(sbs).cuda()
    cbk, cbv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    kall = torch.stack([_dev_kv(torch, seed, 0, l, B, H, T, d) for l in range(Lyr)])
    vall = torch.stack([_dev_kv(torch, seed, 1, l, B, H, T, d) for l in range(Lyr)])
    tq.append(cache, cbk, cbv, sbd, kall, vall, torch.zeros(B, dtype=torch.int32, device="cuda"),
              host_max_pos=0)
    q = torch.empty((Lyr, B, Hq, d), dtype=torch.int16, device="cuda")
    for l in range(Lyr):
        synth.q_dev(seed, 0, l, q[l])
    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.empty((Lyr, B, Hq, d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(cache, Hq, T)
    tq.decode(cache, cbk, cbv, sbd, q, lens_d, T, out, ws)
    torch.cuda.synchronize()
    return cache, sbs, q.cpu().numpy().view(np.uint16), out.cpu().numpy(), (cbk, cbv, sbd, lens_d, T)


def _oracle_decode(seed, d, bk, bv, G, lens, sbs, q16, Lyr=2, H=2):
    ref = np.zeros((Lyr, len(lens), G * H, d))
    bound = np.zeros_like(ref)
    for l in range(Lyr):
        for b, n in enumerate(lens):
            for h in range(H):
                k = synth.kv_host(seed, 0, l, b, h, d, 0, n)
                v = synth.kv_host(seed, 1, l, b, h, d, 0, n)
                o, bd, _ = oracle_attention_with_bound(k, v, q16[l, b, h * G:(h + 1) * G], bk, bv,
                                                       sbs[l])
                ref[l, b, h * G:(h + 1) * G] = o
                bound[l, b, h * G:(h + 1) * G] = bd
    return ref, bound


@pytest.mark.parametrize("d,bk,bv,G,lens", [
    (128, 4, 2, 1, [512]),
    (128, 4, 2, 4, [1, 257, 700]),
    (128, 3, 2, 4, [31, 32, 33]),
    (128, 4, 3, 8, [300, 0, 65]),
    (64, 4, 2, 8, [255, 256]),
    (256, 4, 2, 8, [129, 7]),
    (256, 2, 4, 2, [97]),
    (64, 3, 3, 1, [200]),
])
def test_decode_parity(d, bk, bv, G, lens):
    torch = require_gpu()
    _, sbs, q16, out, _ = _decode_case(torch, d, bk, bv, G, lens)
    ref, bound = _oracle_decode(SEED, d, bk, bv, G, lens, sbs, q16)
    check_attention(out, ref, bound, f"decode d={d} K{bk}/V{bv} G={G} lens={lens}")
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(out[:, b] == 0)


def test_decode_split_invariance():
    """Per-layer calls (more token splits) agree with one all-layer call."""
    torch = require_gpu()
    d, bk, bv, G, lens = 128, 4, 2, 4, [4000, 2500]
    cache, sbs, q16, out, (cbk, cbv, sbd, lens_d, T) = _decode_case(torch, d, bk, bv, G, lens)
    Lyr, B, Hq = out.shape[0], len(lens), G * 2
    qd = torch.from_numpy(q16.view(np.int16)).cuda()
    for l in range(Lyr):
        o = torch.empty((1, B, Hq, d), dtype=torch.float32, device="cuda")
        ws = tq.workspace(cache, Hq, T, n_layers=1, layer0=l)
        tq.decode(cache, cbk, cbv, sbd[l:l + 1], qd[l:l + 1].contiguous(), lens_d, T, o, ws,
                  layer0=l, n_layers=1)
        torch.cuda.synchronize()
        rel, mx = attention_errors(o.cpu().numpy()[0], out[l])
        assert rel < 1e-5 and mx < 1e-4, (rel, mx)
