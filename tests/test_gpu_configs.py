"""Parity of the HIP path at the five workload configurations' full sizes, in
the launch configuration the benchmark uses (one append call and one decode
call covering all layers), checked on sampled outputs the oracle computes one
stream at a time:

  1. tiny: 1 layer, 2 KV heads, 2 query heads, d 128, 512 tokens, K4/V2
     (everything checked);
  2. 32 layers, 32 query / 8 KV heads, d 128, batch 1, 32K context, K4/V2;
  3. 32 layers, 32 / 8 heads, d 128, batch 16, 8K context, K3/V2, 64 decode
     steps each appending one token per sequence;
  4. 48 layers, 8 KV heads, d 128, 32K tokens, K4/V3: bulk encode and 16
     chunked appends of 2048 tokens, which must agree bit for bit;
  5. 80 layers, 64 query / 8 KV heads, d 128, batch 4, 128K context, K4/V2
     (33.5 GB cache), plus one layer at d 64 and one at d 256.

Inputs come from the seeded generator (seed 1000 + config number); the oracle
reads the same fp16 values on the host.  Codes are compared bit for bit
outside the 1e-6 threshold band, norms bit for bit, attention within 2e-3
relative L2 and 1e-2 max-abs over the sampled heads.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import kv_cache_quantization_tq_amd as tq
import oracle
import synth
from helpers import (check_attention, check_mismatch_fraction, compare_codes, gpu_stream,
                     oracle_attention_stream, oracle_stream, require_gpu)

pytestmark = pytest.mark.gpu
WORKERS = min(16, os.cpu_count() or 4)


def _pool():
    return ThreadPoolExecutor(max_workers=WORKERS)


def _gen_layer(torch, seed, layer, B, H, T, d, t0=0):
    k = torch.empty((B, H, T, d), dtype=torch.int16, device="cuda")
    v = torch.empty_like(k)
    synth.kv_dev(seed, 0, layer, k, t0=t0)
    synth.kv_dev(seed, 1, layer, v, t0=t0)
    return k, v


def _sign_table(torch, seed, layers, d):
    sbs = np.stack([synth.sign_bits(seed, l, d) for l in layers])
    return sbs, torch.from_numpy(sbs).cuda()


def _check_rows(cache, seed, layer, b, h, rows, sb, d, bk, bv, what, cache_layer=None):
    """Codes and norms of sampled rows of one stream against the oracle
    (generator layer `layer`, stored at cache layer `cache_layer`)."""
    cl = layer if cache_layer is None else cache_layer
    for kind, bits in ((0, bk), (1, bv)):
        x = np.concatenate([synth.kv_host(seed, kind, layer, b, h, d, r, 1) for r in rows])
        oc, on, ob = oracle.encode(x, bits, sb)
        if kind == 0:
            packed = cache.k_codes[cl, b, h].cpu().numpy()[rows]
            gc = oracle.unpack_rows(packed, d, bits)
            gn = cache.k_norms[cl, b, h].cpu().numpy().view(np.uint16)[rows]
        else:
            tiles = sorted(set(r // 32 for r in rows))
            tile_codes = oracle.unpack_vtiles(cache.v_codes[cl, b, h].cpu().numpy()[tiles], d, bits)
            pos = {t: i for i, t in enumerate(tiles)}
            gc = np.stack([tile_codes[pos[r // 32] * 32 + r % 32] for r in rows])
            gn = cache.v_norms[cl, b, h].cpu().numpy().view(np.uint16)[rows]
        assert np.array_equal(gn, on), f"{what} kind {kind}: norms differ"
        compare_codes(gc, oc, ob, f"{what} kind {kind}")


def _decode_check(seed, cache, out, q, samples, lens, sbs, d, bk, bv, G, what):
    """out, q: host arrays [L][B][Hq][d]; samples: (layer, b, kv) units.  The
    GPU streams are read back here, the oracle runs on a thread per unit."""
    streams = [gpu_stream(cache, l, b, h, lens[b]) for (l, b, h) in samples]
    with _pool() as ex:
        futs = [ex.submit(oracle_attention_stream, seed, l, b, h, lens[b], bk, bv, sbs[l],
                          q[l, b, h * G:(h + 1) * G], g, f"{what} unit {l},{b},{h}")
                for (l, b, h), g in zip(samples, streams)]
        got, ref, n_alt, n_coords = [], [], 0, 0
        for (l, b, h), f in zip(samples, futs):
            o, na, nc = f.result()
            ref.append(o)
            n_alt += na
            n_coords += nc
            got.append(out[l, b, h * G:(h + 1) * G])
    check_mismatch_fraction(n_alt, n_coords, f"{what}: {len(samples)} sampled units")
    check_attention(np.stack(got), np.stack(ref), f"{what}: {len(samples)} sampled units", n_alt)


def test_config1_tiny_full():
    torch = require_gpu()
    seed, L, B, H, G, d, T, bk, bv = 1001, 1, 1, 2, 1, 128, 512, 4, 2
    sbs, sbd = _sign_table(torch, seed, range(L), d)
    cache = tq.KVCache(L, B, H, d, bk, bv, T)
    cbk, cbv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    k, v = _gen_layer(torch, seed, 0, B, H, T, d)
    tq.append(cache, cbk, cbv, sbd, k[None], v[None], torch.zeros(B, dtype=torch.int32,
                                                                   device="cuda"), host_max_pos=0)
    q = torch.empty((L, B, H * G, d), dtype=torch.int16, device="cuda")
    synth.q_dev(seed, 0, 0, q[0])
    out = torch.empty((L, B, H * G, d), dtype=torch.float32, device="cuda")
    tq.decode(cache, cbk, cbv, sbd, q, torch.full((B,), T, dtype=torch.int32, device="cuda"), T,
              out, tq.workspace(cache, H * G, T))
    torch.cuda.synchronize()
    for h in range(H):
        _check_rows(cache, seed, 0, 0, h, list(range(T)), sbs[0], d, bk, bv, f"cfg1 head {h}")
    _decode_check(seed, cache, out.cpu().numpy(), q.cpu().numpy().view(np.uint16),
                  [(0, 0, h) for h in range(H)], [T], sbs, d, bk, bv, G, "cfg1")


def test_config2_llama8b_32k():
    torch = require_gpu()
    seed, L, B, H, G, d, T, bk, bv = 1002, 32, 1, 8, 4, 128, 32768, 4, 2
    sbs, sbd = _sign_table(torch, seed, range(L), d)
    cache = tq.KVCache(L, B, H, d, bk, bv, T + 32)
    cbk, cbv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    kp = torch.empty((L, B, H, T, d), dtype=torch.int16, device="cuda")
    vp = torch.empty_like(kp)
    kn = torch.empty((L, B, H, 1, d), dtype=torch.int16, device="cuda")
    vn = torch.empty_like(kn)
    for l in range(L):
        synth.kv_dev(seed, 0, l, kp[l])
        synth.kv_dev(seed, 1, l, vp[l])
        synth.kv_dev(seed, 0, l, kn[l], t0=T)
        synth.kv_dev(seed, 1, l, vn[l], t0=T)
    tq.append(cache, cbk, cbv, sbd, kp, vp, torch.zeros(B, dtype=torch.int32, device="cuda"),
              host_max_pos=0)
    tq.append(cache, cbk, cbv, sbd, kn, vn, torch.full((B,), T, dtype=torch.int32, device="cuda"),
              host_max_pos=T)
    del kp, vp
    q = torch.empty((L, B, H * G, d), dtype=torch.int16, device="cuda")
    for l in range(L):
        synth.q_dev(seed, 0, l, q[l])
    ctx = T + 1
    out = torch.empty((L, B, H * G, d), dtype=torch.float32, device="cuda")
    tq.decode(cache, cbk, cbv, sbd, q, torch.full((B,), ctx, dtype=torch.int32, device="cuda"),
              ctx, out, tq.workspace(cache, H * G, ctx))
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    for (l, h) in ((0, 0), (17, 5), (31, 7)):
        rows = sorted(set(rng.integers(0, ctx, 300).tolist()) | {0, 31, 32, T - 1, T})
        _check_rows(cache, seed, l, 0, h, rows, sbs[l], d, bk, bv, f"cfg2 layer {l} head {h}")
    units = [(0, 0, 0), (3, 0, 2), (7, 0, 5), (12, 0, 1), (17, 0, 4), (22, 0, 7), (27, 0, 3),
             (31, 0, 6)]
    _decode_check(seed, cache, out.cpu().numpy(), q.cpu().numpy().view(np.uint16), units, [ctx],
                  sbs, d, bk, bv, G, "cfg2")
    assert np.isfinite(out.cpu().numpy()).all()


def test_config3_batched_decode_64_steps():
    torch = require_gpu()
    seed, L, B, H, G, d, T0, steps, bk, bv = 1003, 32, 16, 8, 4, 128, 8192, 64, 3, 2
    sbs, sbd = _sign_table(torch, seed, range(L), d)
    cap = T0 + steps
    cache = tq.KVCache(L, B, H, d, bk, bv, ((cap + 31) // 32) * 32)
    cbk, cbv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    for l in range(L):
        k, v = _gen_layer(torch, seed, l, B, H, T0, d)
        tq.append(cache, cbk, cbv, sbd[l:l + 1], k[None], v[None], zero, host_max_pos=0,
                  layer0=l, n_layers=1)
    torch.cuda.synchronize()
    del k, v
    kn = torch.empty((L, B, H, 1, d), dtype=torch.int16, device="cuda")
    vn = torch.empty_like(kn)
    q = torch.empty((L, B, H * G, d), dtype=torch.int16, device="cuda")
    out = torch.empty((L, B, H * G, d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(cache, H * G, cap)
    sample_layers = (0, 31)
    outs, qs = [], []
    for s in range(steps):
        for l in range(L):
            synth.kv_dev(seed, 0, l, kn[l], t0=T0 + s)
            synth.kv_dev(seed, 1, l, vn[l], t0=T0 + s)
            synth.q_dev(seed, s, l, q[l])
        pos = torch.full((B,), T0 + s, dtype=torch.int32, device="cuda")
        tq.append(cache, cbk, cbv, sbd, kn, vn, pos, host_max_pos=T0 + s)
        ctx = T0 + s + 1
        tq.decode(cache, cbk, cbv, sbd, q, torch.full((B,), ctx, dtype=torch.int32,
                                                      device="cuda"), ctx, out, ws)
        outs.append(out[list(sample_layers)].cpu().numpy())
        qs.append(q[list(sample_layers)].cpu().numpy().view(np.uint16))
    torch.cuda.synchronize()
    # appended rows and a few prefill rows against the oracle
    for l, b, h in ((0, 0, 0), (31, 15, 7), (0, 9, 3)):
        rows = [0, 5, T0 - 1] + list(range(T0, T0 + steps))
        _check_rows(cache, seed, l, b, h, rows, sbs[l], d, bk, bv, f"cfg3 stream {l},{b},{h}")
    # attention on every step for sampled streams: encode and dequantize each
    # stream once with the oracle (resolved against the GPU's codes of all
    # its rows), then attend with each step's queries over its prefix
    units = [(li, b, h) for li in range(len(sample_layers)) for b in (0, 7, 15) for h in (0, 5)]
    streams = {u: gpu_stream(cache, sample_layers[u[0]], u[1], u[2], cap) for u in units}

    def stream(u):
        li, b, h = u
        l = sample_layers[li]
        k = synth.kv_host(seed, 0, l, b, h, d, 0, cap)
        v = synth.kv_host(seed, 1, l, b, h, d, 0, cap)
        st = oracle_stream(k, v, bk, bv, sbs[l], streams[u], f"cfg3 stream {l},{b},{h}")
        res = []
        for s in range(steps):
            n = T0 + s + 1
            q64 = oracle.halves_to_double(qs[s][li, b, h * G:(h + 1) * G])
            res.append(oracle.attention(q64, st["K"][:n], st["V"][:n]))
        return u, res, st["n_alt"], st["n_coords"]

    got, ref, n_alt, n_coords = [], [], 0, 0
    with _pool() as ex:
        for (li, b, h), res, na, nc in ex.map(stream, units):
            n_alt += na
            n_coords += nc
            for s in range(steps):
                ref.append(res[s])
                got.append(outs[s][li, b, h * G:(h + 1) * G])
    what = f"cfg3: {steps} steps x {len(units)} streams"
    check_mismatch_fraction(n_alt, n_coords, what)
    check_attention(np.stack(got), np.stack(ref), what, n_alt)


def test_config4_encode_bulk_equals_chunked():
    torch = require_gpu()
    seed, L, B, H, d, T, bk, bv, chunk = 1004, 48, 1, 8, 128, 32768, 4, 3, 2048
    sbs, sbd = _sign_table(torch, seed, range(L), d)
    bulk = tq.KVCache(L, B, H, d, bk, bv, T)
    chunked = tq.KVCache(L, B, H, d, bk, bv, T)
    cbk, cbv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    kp = torch.empty((L, B, H, T, d), dtype=torch.int16, device="cuda")
    vp = torch.empty_like(kp)
    for l in range(L):
        synth.kv_dev(seed, 0, l, kp[l])
        synth.kv_dev(seed, 1, l, vp[l])
    tq.append(bulk, cbk, cbv, sbd, kp, vp, zero, host_max_pos=0)
    for c in range(T // chunk):
        kc = kp[:, :, :, c * chunk:(c + 1) * chunk].contiguous()
        vc = vp[:, :, :, c * chunk:(c + 1) * chunk].contiguous()
        tq.append(chunked, cbk, cbv, sbd, kc, vc, torch.full((B,), c * chunk, dtype=torch.int32,
                                                              device="cuda"), host_max_pos=c * chunk)
    torch.cuda.synchronize()
    for name in ("k_codes", "v_codes", "k_norms", "v_norms"):
        assert torch.equal(getattr(bulk, name), getattr(chunked, name)), name
    rng = np.random.default_rng(4)
    for (l, h) in ((0, 0), (23, 3), (47, 7)):
        rows = sorted(set(rng.integers(0, T, 400).tolist()) | {0, 2047, 2048, T - 1})
        _check_rows(bulk, seed, l, 0, h, rows, sbs[l], d, bk, bv, f"cfg4 layer {l} head {h}")


def test_config5_70b_long_context():
    torch = require_gpu()
    seed, L, B, H, G, d, T, bk, bv = 1005, 80, 4, 8, 8, 128, 131072, 4, 2
    sbs, sbd = _sign_table(torch, seed, range(L), d)
    cache = tq.KVCache(L, B, H, d, bk, bv, T)
    cbk, cbv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    for l in range(L):
        k, v = _gen_layer(torch, seed, l, B, H, T, d)
        tq.append(cache, cbk, cbv, sbd[l:l + 1], k[None], v[None], zero, host_max_pos=0,
                  layer0=l, n_layers=1)
        del k, v
        if l % 20 == 19:
            torch.cuda.synchronize()
            print(f"cfg5: {l + 1} of {L} layers encoded", flush=True)
    q = torch.empty((L, B, H * G, d), dtype=torch.int16, device="cuda")
    for l in range(L):
        synth.q_dev(seed, 0, l, q[l])
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    out = torch.empty((L, B, H * G, d), dtype=torch.float32, device="cuda")
    tq.decode(cache, cbk, cbv, sbd, q, lens, T, out, tq.workspace(cache, H * G, T))
    torch.cuda.synchronize()
    outh, qh = out.cpu().numpy(), q.cpu().numpy().view(np.uint16)
    assert np.isfinite(outh).all()
    _check_rows(cache, seed, 79, 3, 7, [0, 1, 4097, T - 1], sbs[79], d, bk, bv, "cfg5 rows")
    units = [(0, 0, 0), (10, 1, 3), (20, 2, 6), (30, 3, 1), (40, 0, 4), (50, 1, 7), (60, 2, 2),
             (79, 3, 7)]
    _decode_check(seed, cache, outh, qh, units, [T] * B, sbs, d, bk, bv, G, "cfg5 d128")
    del cache, out
    # the extra layers at d = 64 and d = 256 (layer indices 80 and 81 of the seed)
    for dd, layer in ((64, 80), (256, 81)):
        c1 = tq.KVCache(1, B, H, dd, bk, bv, T)
        cb1k, cb1v = tq.Codebook(dd, bk), tq.Codebook(dd, bv)
        sb1 = synth.sign_bits(seed, layer, dd)
        sb1d = torch.from_numpy(sb1[None]).cuda()
        k, v = _gen_layer(torch, seed, layer, B, H, T, dd)
        tq.append(c1, cb1k, cb1v, sb1d, k[None], v[None], zero, host_max_pos=0)
        del k, v
        q1 = torch.empty((1, B, H * G, dd), dtype=torch.int16, device="cuda")
        synth.q_dev(seed, 0, layer, q1[0])
        o1 = torch.empty((1, B, H * G, dd), dtype=torch.float32, device="cuda")
        tq.decode(c1, cb1k, cb1v, sb1d, q1, lens, T, o1, tq.workspace(c1, H * G, T))
        torch.cuda.synchronize()
        _check_rows(c1, seed, layer, 1, 2, [0, 77, T - 1], sb1, dd, bk, bv, f"cfg5 d{dd} rows",
                    cache_layer=0)
        # the oracle streams of this layer are indexed by its own layer number
        o1h, q1h = o1.cpu().numpy(), q1.cpu().numpy().view(np.uint16)
        what = f"cfg5 d{dd}"
        ref, na, nc = oracle_attention_stream(seed, layer, 2, 5, T, bk, bv, sb1,
                                              q1h[0, 2, 5 * G:6 * G], gpu_stream(c1, 0, 2, 5, T),
                                              what)
        check_mismatch_fraction(na, nc, what)
        check_attention(o1h[0, 2, 5 * G:6 * G], ref, what, na)
        del c1, o1
