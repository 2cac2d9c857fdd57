"""GPU parity of prefill (extend) attention over the compressed cache
(tq_prefill_attn) against the oracle: every new query attends causally to its
sequence's cached tokens, so query i of sequence b is the oracle's attention
over the first pos[b] + i + 1 dequantized tokens.  Shapes span several query
chunks and key tiles with ragged ends, every group size class (including a
group that is not a power of two), all head dims, plain prefill (pos 0) and
extension of an existing context, and paged storage."""
import numpy as np
import pytest

import kv_cache_quantization_tq_amd as tq
import oracle
import synth
from helpers import (check_attention, check_mismatch_fraction, gpu_stream, oracle_stream,
                     require_gpu)

pytestmark = pytest.mark.gpu
SEED = 1003


def _grow_exps(n, grow):
    """Per-token power-of-two scale exponents of K and V (zero unless grow):
    keys double every 20 tokens, values every 48 (outputs stay in the range
    the absolute max-abs bar is meant for)."""
    t = np.arange(n)
    return (t // 20, t // 48) if grow else (0 * t, 0 * t)


def _scaled(h16, e):
    """fp16 bits times 2^e per row (exact: no value leaves the normal range)."""
    x = h16.view(np.float16).astype(np.float32) * np.exp2(e)[:, None].astype(np.float32)
    y = x.astype(np.float16)
    assert np.all(np.isfinite(y)) and np.array_equal(y.astype(np.float32), x)
    return y.view(np.uint16)


def _case(torch, d, bk, bv, G, H, pos, t_new, Lyr=1, paged_tokens=None, seed=SEED, grow=False):
    B = len(pos)
    T = max(pos) + t_new
    cap = ((T + 31) // 32) * 32
    if paged_tokens:
        P = paged_tokens
        cap = (cap + P - 1) // P * P
        maxp = cap // P
        rng = np.random.default_rng(seed)
        table = rng.permutation(B * maxp).reshape(B, maxp).astype(np.int32)
        cache = tq.PagedKVCache(Lyr, B, H, d, bk, bv, P, maxp, B * maxp, table)
    else:
        cache = tq.KVCache(Lyr, B, H, d, bk, bv, cap)
    sbs = np.stack([synth.sign_bits(seed, l, d) for l in range(Lyr)])
    sbd = torch.from_numpy(sbs).cuda()
    cbk, cbv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    for l in range(Lyr):
        k = torch.empty((1, B, H, T, d), dtype=torch.int16, device="cuda")
        v = torch.empty_like(k)
        synth.kv_dev(seed, 0, l, k[0])
        synth.kv_dev(seed, 1, l, v[0])
        if grow:
            ke, ve = _grow_exps(T, True)
            for x, e in ((k, ke), (v, ve)):
                sc = torch.from_numpy(np.exp2(e).astype(np.float16)).cuda()
                x.view(torch.float16).mul_(sc[:, None])
        tq.append(cache, cbk, cbv, sbd[l:l + 1], k, v,
                  torch.zeros(B, dtype=torch.int32, device="cuda"), host_max_pos=0, layer0=l,
                  n_layers=1)
    q16 = np.empty((Lyr, B, G * H, t_new, d), dtype=np.uint16)
    for l in range(Lyr):
        for b in range(B):
            for hq in range(G * H):
                for i in range(t_new):
                    q16[l, b, hq, i] = synth.q_host(seed, i, l, b, hq, d)
    qd = torch.from_numpy(q16.view(np.int16)).cuda()
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    out = torch.empty((Lyr, B, G * H, t_new, d), dtype=torch.float32, device="cuda")
    tq.prefill(cache, cbk, cbv, sbd, qd, posd, out)
    torch.cuda.synchronize()
    return dict(cache=cache, sbs=sbs, sbd=sbd, cbk=cbk, cbv=cbv, q16=q16, qd=qd, posd=posd,
                out=out.cpu().numpy(), Lyr=Lyr, B=B, H=H, G=G, d=d, bk=bk, bv=bv, pos=pos,
                t_new=t_new, seed=seed, grow=grow)


def _oracle(c, what=""):
    """Every query row's attention over its causal prefix of the cache,
    resolved against the GPU's codes; returns (ref, band codes resolved)."""
    d, G, H, t_new = c["d"], c["G"], c["H"], c["t_new"]
    ref = np.zeros(c["out"].shape)
    n_alt = n_coords = 0
    for l in range(c["Lyr"]):
        for b, p in enumerate(c["pos"]):
            for h in range(H):
                n_all = p + t_new
                k = synth.kv_host(c["seed"], 0, l, b, h, d, 0, n_all)
                v = synth.kv_host(c["seed"], 1, l, b, h, d, 0, n_all)
                if c["grow"]:
                    ke, ve = _grow_exps(n_all, True)
                    k, v = _scaled(k, ke), _scaled(v, ve)
                sl = slice(h * G, (h + 1) * G)
                st = oracle_stream(k, v, c["bk"], c["bv"], c["sbs"][l],
                                   gpu_stream(c["cache"], l, b, h, n_all), f"{what} {l},{b},{h}")
                n_alt += st["n_alt"]
                n_coords += st["n_coords"]
                for i in range(t_new):
                    n = p + i + 1
                    q64 = oracle.halves_to_double(c["q16"][l, b, sl, i])
                    ref[l, b, sl, i] = oracle.attention(q64, st["K"][:n], st["V"][:n])
    check_mismatch_fraction(n_alt, n_coords, what)
    return ref, n_alt


@pytest.mark.parametrize("d,bk,bv,G,H,pos,t_new,Lyr", [
    (128, 4, 2, 4, 2, [0, 300], 77, 2),
    (64, 3, 3, 8, 1, [5], 40, 1),
    (256, 2, 4, 1, 2, [1000], 130, 1),
    (128, 4, 3, 3, 2, [33], 50, 1),
    (128, 3, 2, 2, 1, [62, 0, 17], 33, 1),
    # one new query; a chunk whose first query is the last token of a tile
    (128, 4, 2, 4, 1, [40, 0], 1, 1),
    (128, 2, 4, 4, 1, [31, 63], 2, 1),
    (64, 4, 2, 2, 2, [95], 70, 1),
])
def test_prefill_parity(d, bk, bv, G, H, pos, t_new, Lyr):
    torch = require_gpu()
    c = _case(torch, d, bk, bv, G, H, pos, t_new, Lyr)
    what = f"prefill d={d} K{bk}/V{bv} G={G} pos={pos} t_new={t_new}"
    ref, n_alt = _oracle(c, what)
    check_attention(c["out"], ref, what, n_alt)


@pytest.mark.parametrize("P,d", [(32, 128), (128, 128), (64, 64)])
def test_prefill_paged(P, d):
    """Shuffled pages: the oracle's bars, and bit for bit the contiguous
    cache's output (the kernels differ only in row addressing)."""
    torch = require_gpu()
    c = _case(torch, d, 4, 2, 4, 2, [0, 300], 77, 2, paged_tokens=P)
    ref, n_alt = _oracle(c, f"prefill paged P={P} d={d}")
    check_attention(c["out"], ref, f"prefill paged P={P} d={d}", n_alt)
    cc = _case(torch, d, 4, 2, 4, 2, [0, 300], 77, 2)
    assert np.array_equal(c["out"], cc["out"]), float(np.abs(c["out"] - cc["out"]).max())


@pytest.mark.parametrize("d,bk,bv,G,pos,t_new", [
    (128, 4, 2, 4, [0, 40], 100),
    (64, 3, 3, 8, [5], 90),
])
def test_prefill_growing_scales(d, bk, bv, G, pos, t_new):
    """Key and value scales that double every 20 and 48 tokens: each column's
    running softmax reference moves many times, by more than the rescale
    threshold within a tile too, and the block's value-norm exponent moves."""
    torch = require_gpu()
    c = _case(torch, d, bk, bv, G, 1, pos, t_new, grow=True)
    what = f"prefill growing scales d={d}"
    ref, n_alt = _oracle(c, what)
    check_attention(c["out"], ref, what, n_alt)


def test_prefill_row_equals_decode():
    """Query i of the prefill equals a decode step with that query and
    length pos + i + 1 (both on the GPU, same cache)."""
    torch = require_gpu()
    c = _case(torch, 128, 4, 2, 4, 2, [200, 40], 70, 1)
    for i in (0, 1, 31, 32, 69):
        q = c["qd"][:, :, :, i].contiguous()
        lens = c["posd"] + (i + 1)
        out = torch.empty((1, c["B"], c["G"] * c["H"], c["d"]), dtype=torch.float32, device="cuda")
        ws = tq.workspace(c["cache"], c["G"] * c["H"], max(c["pos"]) + i + 1)
        tq.decode(c["cache"], c["cbk"], c["cbv"], c["sbd"], q, lens, max(c["pos"]) + i + 1, out,
                  ws)
        torch.cuda.synchronize()
        got = c["out"][:, :, :, i]
        want = out.cpu().numpy()
        rel = np.linalg.norm(got - want) / np.linalg.norm(want)
        mx = np.abs(got - want).max()
        print(f"prefill row {i} vs decode: rel {rel:.2e} max-abs {mx:.2e}")
        assert rel < 1e-4 and mx < 1e-3, (i, rel, mx)


def test_prefill_full_size_sampled():
    """The benchmark's prefill launch at its full prompt (32768 tokens, 8 KV
    heads, groups of 4, d 128, K4/V2; one layer: the launch configuration per
    block does not depend on the layer count), checked on sampled query rows
    of two KV heads against the oracle's attention over their whole prefix."""
    torch = require_gpu()
    d, bk, bv, G, H, T = 128, 4, 2, 4, 8, 32768
    seed = 1002
    cache = tq.KVCache(1, 1, H, d, bk, bv, T)
    sbs = np.stack([synth.sign_bits(seed, 0, d)])
    sbd = torch.from_numpy(sbs).cuda()
    cbk, cbv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    k = torch.empty((1, 1, H, T, d), dtype=torch.int16, device="cuda")
    v = torch.empty_like(k)
    synth.kv_dev(seed, 0, 0, k[0])
    synth.kv_dev(seed, 1, 0, v[0])
    tq.append(cache, cbk, cbv, sbd, k, v, torch.zeros(1, dtype=torch.int32, device="cuda"),
              host_max_pos=0)
    del k, v
    rows = [0, 31, 32, 4095, 16384, 32767]
    q16 = np.empty((1, 1, G * H, T, d), dtype=np.uint16)
    qs = np.stack([synth.q_host(seed, 0, 0, 0, hq, d) for hq in range(G * H)])
    q16[0, 0] = qs[:, None, :]
    for hq in range(G * H):  # distinct queries on the sampled rows
        for i in rows:
            q16[0, 0, hq, i] = synth.q_host(seed, i + 1, 0, 0, hq, d)
    qd = torch.from_numpy(q16.view(np.int16)).cuda()
    out = torch.empty((1, 1, G * H, T, d), dtype=torch.float32, device="cuda")
    tq.prefill(cache, cbk, cbv, sbd, qd, torch.zeros(1, dtype=torch.int32, device="cuda"), out)
    torch.cuda.synchronize()
    for h in (0, 5):
        kk = synth.kv_host(seed, 0, 0, 0, h, d, 0, T)
        vv = synth.kv_host(seed, 1, 0, 0, h, d, 0, T)
        sl = slice(h * G, (h + 1) * G)
        what = f"prefill 32K, KV head {h}, rows {rows}"
        st = oracle_stream(kk, vv, bk, bv, sbs[0], gpu_stream(cache, 0, 0, h, T), what)
        check_mismatch_fraction(st["n_alt"], st["n_coords"], what)
        got = np.stack([out[0, 0, sl, i].cpu().numpy() for i in rows])
        ref = np.zeros_like(got, dtype=np.float64)
        for r, i in enumerate(rows):
            q64 = oracle.halves_to_double(q16[0, 0, sl, i])
            ref[r] = oracle.attention(q64, st["K"][:i + 1], st["V"][:i + 1])
        check_attention(got, ref, what, st["n_alt"])
