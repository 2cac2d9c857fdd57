"""Benchmark of the compressed-KV hot path on one MI355X.

Workload (Llama-3-8B-shaped, 32K context): 32 layers, 32 query heads, 8 KV
heads (GQA group 4), head dim 128, batch 1, keys 4-bit / values 2-bit, seeded
synthetic fp16 K/V with 4 outlier channels (x10) per head and a per-token
lognormal(0, 0.5) scale.

One step = the whole hot path over one batch: compress the 32768-token prefill
of all 32 layers (tq_append), append the next token (tq_append), and one decode
step of attention over the 32769-token compressed cache of all 32 layers
(tq_decode_attn).  Inputs are resident in HBM before timing starts.

``value`` is the decode-attention throughput in GB/s of packed cache bytes
(codes + norms) per step; the line also carries encode tokens/s, the decode
kernel's roofline fraction against the 8 TB/s HBM peak, the 48-layer K4/V3
32K prefill encode (timed after the steps, bulk and in 16 chunks of 2048
tokens), and the CPU oracle timed on a bounded sample on this host's cores,
with the same sample's GPU codes and outputs compared against it.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

L, B, HKV, HQ, D, T, BK, BV = 32, 1, 8, 32, 128, 32768, 4, 2
SEED = 1002
HBM_PEAK_GBS = 8000.0


def per_token_head_bytes(d=D, bk=BK, bv=BV):
    """Algorithmic decode bytes per token per KV head: codes + two fp16 norms."""
    return d * (bk + bv) // 8 + 4


def encode_bytes_per_token_head(d=D, bk=BK, bv=BV):
    """fp16 K+V read + packed codes and norms written."""
    return 4 * d + d * (bk + bv) // 8 + 4


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE scaled by a
    plain copy's readings), or None when the kernel's source has changed since
    the counters were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)["kernels"][kernel]
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes"] if h.hexdigest() == rec["source_sha256"] else None


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_threads():
    """Threads for the oracle: the cores in this process's affinity mask, at
    most 16 (one GPU's share of a host's cores)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n)), n


def cpu_baseline(gpu=None, seconds_budget=20.0):
    """The oracle (plain loops, fp64) on this host's cores, on a sample of the
    same workload: whole (layer, KV head) streams of the decoded context (the
    32768-token prefill plus the appended token), each encoded (keys and
    values: norm, explicit rotation, argmin), then dequantized and attended by
    its 4 query heads.  One stream per thread, rounds of `threads` streams
    (streams spread over the layers) until the budget is spent; each phase is
    timed by the wall clock over a round.  Rates are scaled to the metric's
    units: decode GB/s of packed bytes, encode tokens/s over all layers and
    heads.

    With `gpu` = (cache, out, q) the same streams are also compared with the
    GPU's: norms bit for bit, codes (any difference must lie within 1e-6 of a
    threshold; those are counted), and the attention outputs against the
    oracle's over its cache, resolved to the GPU's neighbouring code at those
    band coordinates."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    import synth
    ctx = T + 1
    threads, n_aff = _oracle_threads()
    order = np.random.default_rng(SEED).permutation(L * HKV)
    units = [(int(u) // HKV, int(u) % HKV) for u in order]
    sbs = {l: synth.sign_bits(SEED, l, D) for l in range(L)}
    enc_s = dec_s = 0.0
    done = 0
    par = dict(streams=0, codes=0, band_diff=0, outside_band_diff=0, norms_diff=0,
               num=0.0, den=0.0, max_abs=0.0)

    def inputs_unit(u):
        l, h = u
        return [synth.kv_host(SEED, kind, l, 0, h, D, 0, ctx) for kind in (0, 1)]

    def encode_unit(args):
        (l, h), xs = args
        return [oracle.encode(x, bits, sbs[l], want_alt=True) for x, bits in zip(xs, (BK, BV))]

    def decode_unit(args):
        (l, h), enc, resolved = args
        (kc, kn, _, _), (vc, vn, _, _) = enc
        K = oracle.dequant(resolved[0] if resolved else kc, kn, BK, sbs[l])
        V = oracle.dequant(resolved[1] if resolved else vc, vn, BV, sbs[l])
        q = np.stack([synth.q_host(SEED, 0, l, 0, h * (HQ // HKV) + g, D)
                      for g in range(HQ // HKV)])
        return oracle.attention(oracle.halves_to_double(q), K, V)

    # the oracle's codebooks (Lloyd iterations, computed once and kept) are
    # built before timing
    oracle.codebook(D, BK)
    oracle.codebook(D, BV)
    t_start = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while done < len(units) and time.perf_counter() - t_start < seconds_budget:
            batch = units[done:done + threads]
            xs = list(ex.map(inputs_unit, batch))  # the seeded inputs, not timed
            t0 = time.perf_counter()
            encs = list(ex.map(encode_unit, zip(batch, xs)))
            t1 = time.perf_counter()
            del xs
            resolved = []
            for (l, h), enc in zip(batch, encs):
                if gpu is None:
                    resolved.append(None)
                    continue
                cache = gpu[0]
                g_k = oracle.unpack_rows(cache.k_codes[l, 0, h, :ctx].cpu().numpy(), D, BK)
                g_v = oracle.unpack_vtiles(cache.v_codes[l, 0, h, :(ctx + 31) // 32].cpu().numpy(),
                                           D, BV)[:ctx]
                g_norms = (cache.k_norms[l, 0, h, :ctx].cpu().numpy().view(np.uint16),
                           cache.v_norms[l, 0, h, :ctx].cpu().numpy().view(np.uint16))
                res = []
                for (codes, norms, band, alt), gc, gn in zip(enc, (g_k, g_v), g_norms):
                    diff = gc != codes
                    inside = diff & (band < 1e-6) & (gc == alt)
                    par["codes"] += codes.size
                    par["band_diff"] += int(inside.sum())
                    par["outside_band_diff"] += int((diff & ~inside).sum())
                    par["norms_diff"] += int((gn != norms).sum())
                    rc = codes.copy()
                    rc[inside] = alt[inside]
                    res.append(rc)
                resolved.append(res)
            t2 = time.perf_counter()
            outs = list(ex.map(decode_unit, zip(batch, encs, resolved)))
            t3 = time.perf_counter()
            enc_s += t1 - t0
            dec_s += t3 - t2
            done += len(batch)
            if gpu is not None:
                out_gpu = gpu[1]
                G = HQ // HKV
                for (l, h), o in zip(batch, outs):
                    g = out_gpu[l, 0, h * G:(h + 1) * G].cpu().numpy().astype(np.float64)
                    par["num"] += float(((g - o) ** 2).sum())
                    par["den"] += float((o ** 2).sum())
                    par["max_abs"] = max(par["max_abs"], float(np.abs(g - o).max()))
                par["streams"] = done
    dec_gbs = done * ctx * per_token_head_bytes() / dec_s / 1e9
    enc_tok_s = done * ctx / enc_s / (L * HKV)  # context tokens/s over all layers and heads
    r = {
        "value": dec_gbs, "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"{done} of {L * HKV} (layer, KV head) streams of the {ctx}-token context, "
                  f"each encoded (keys and values), dequantized and attended by "
                  f"{HQ // HKV} query heads; {threads} streams at a time, one per thread",
        "cpu_model": _cpu_model(), "cores_in_affinity_mask": n_aff,
        "encode_tokens_per_s": enc_tok_s,
        "seconds": enc_s + dec_s,
    }
    if gpu is not None:
        r["parity"] = {
            "streams": par["streams"], "codes": par["codes"],
            "band_codes_gpu_took_other_neighbour": par["band_diff"],
            "codes_differing_outside_band": par["outside_band_diff"],
            "norms_differing": par["norms_diff"],
            "attention_rel_l2": (par["num"] / par["den"]) ** 0.5 if par["den"] else 0.0,
            "attention_max_abs": par["max_abs"],
            "bars": "codes: differences only within 1e-6 of a threshold, under 1e-5 of codes; "
                    "norms bit-exact; attention rel-L2 <= 2e-3, max-abs <= 1e-2"}
    return r


def _report(workload, metric, value, unit, higher, extra, args, ms_per_step):
    line = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": higher,
            "scaling": "weak", "vs_baseline": None,
            "data": "synthetic (seeded fp16 K/V with outlier channels and lognormal token scale)",
            "config": workload}
    line.update(extra)
    print(json.dumps(line), flush=True)


def _timed(torch, fn, steps, warmup):
    """Median over `steps` calls of fn issued back to back (after `warmup`
    calls), each bracketed by its own events, in ms."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    ts = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    return ts[len(ts) // 2]


def _fill_cache(torch, tq, synth, cache, cbk, cbv, sbd, seed, L, B, H, T, d):
    """Encode the seeded prefill of every layer into `cache`, one layer at a
    time (bounded device memory)."""
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    for l in range(L):
        k = torch.empty((1, B, H, T, d), dtype=torch.int16, device="cuda")
        v = torch.empty_like(k)
        synth.kv_dev(seed, 0, l, k[0])
        synth.kv_dev(seed, 1, l, v[0])
        tq.append(cache, cbk, cbv, sbd[l:l + 1], k, v, zero, host_max_pos=0, layer0=l, n_layers=1)
        del k, v
    torch.cuda.synchronize()


def workload_batched_decode(args):
    """32 layers, 32 query / 8 KV heads, d 128, batch 16, 8192-token context,
    K3/V2: 64 consecutive steps, each appending one token per sequence to all
    layers (one tq_append) and attending over all layers (one tq_decode_attn).
    Reports decode tokens/s (batch x steps / time) and GB/s of packed cache
    read over the 64 steps."""
    import numpy as np
    import torch
    import kv_cache_quantization_tq_amd as tq
    import synth
    seed, L, B, H, HQ, d, T0, steps, bk, bv = 1003, 32, 16, 8, 32, 128, 8192, 64, 3, 2
    torch.cuda.set_device(0)
    cap = ((T0 + steps + 31) // 32) * 32
    cache = tq.KVCache(L, B, H, d, bk, bv, cap)
    cbk, cbv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    sbd = torch.from_numpy(np.stack([synth.sign_bits(seed, l, d) for l in range(L)])).cuda()
    _fill_cache(torch, tq, synth, cache, cbk, cbv, sbd, seed, L, B, H, T0, d)
    kn = torch.empty((steps, L, B, H, 1, d), dtype=torch.int16, device="cuda")
    vn = torch.empty_like(kn)
    q = torch.empty((steps, L, B, HQ, d), dtype=torch.int16, device="cuda")
    for s in range(steps):
        for l in range(L):
            synth.kv_dev(seed, 0, l, kn[s, l], t0=T0 + s)
            synth.kv_dev(seed, 1, l, vn[s, l], t0=T0 + s)
            synth.q_dev(seed, s, l, q[s, l])
    pos = [torch.full((B,), T0 + s, dtype=torch.int32, device="cuda") for s in range(steps)]
    lens = [torch.full((B,), T0 + s + 1, dtype=torch.int32, device="cuda") for s in range(steps)]
    out = torch.empty((L, B, HQ, d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(cache, HQ, cap)
    torch.cuda.synchronize()

    def run64():
        for s in range(steps):
            tq.append(cache, cbk, cbv, sbd, kn[s], vn[s], pos[s], host_max_pos=T0 + s)
            tq.decode(cache, cbk, cbv, sbd, q[s], lens[s], T0 + s + 1, out, ws)

    ms = _timed(torch, run64, args.steps, args.warmup)
    nbytes = sum(L * B * H * (T0 + s + 1) * per_token_head_bytes(d, bk, bv) for s in range(steps))
    gbs = nbytes / (ms * 1e-3) / 1e9
    _report({"workload": "batched decode, 64 steps with appends", "layers": L, "q_heads": HQ,
             "kv_heads": H, "head_dim": d, "batch": B, "context": f"{T0 + 1}..{T0 + steps}",
             "bits_k": bk, "bits_v": bv},
            "decode tokens/s (batch x 64 steps, append + decode per step)", B * steps / (ms * 1e-3),
            "tokens/s", True,
            {"dtype": "f32 (f16 matrix-core operands; packed 3-bit K, 2-bit V)",
             "ms_per_64_steps": ms, "packed_gbs": gbs, "pct_hbm_peak": 100 * gbs / HBM_PEAK_GBS,
             "packed_bytes_64_steps": nbytes}, args, ms / steps)


def encode_48l(args):
    """48 layers, 8 KV heads, d 128, 32768 tokens, K4/V3: the whole prefill in
    one tq_append over all layers, and the same prefill as 16 chunked appends
    of 2048 tokens, each timed (median of `steps` after `warmup`).  Returns
    the figures; the inputs are freed before returning."""
    import numpy as np
    import torch
    import kv_cache_quantization_tq_amd as tq
    import synth
    seed, L4, B4, H, d, T4, bk, bv, chunk = 1004, 48, 1, 8, 128, 32768, 4, 3, 2048
    cache = tq.KVCache(L4, B4, H, d, bk, bv, T4)
    cbk, cbv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    sbd = torch.from_numpy(np.stack([synth.sign_bits(seed, l, d) for l in range(L4)])).cuda()
    kp = torch.empty((L4, B4, H, T4, d), dtype=torch.int16, device="cuda")
    vp = torch.empty_like(kp)
    for l in range(L4):
        synth.kv_dev(seed, 0, l, kp[l])
        synth.kv_dev(seed, 1, l, vp[l])
    kc = [kp[:, :, :, c * chunk:(c + 1) * chunk].contiguous() for c in range(T4 // chunk)]
    vc = [vp[:, :, :, c * chunk:(c + 1) * chunk].contiguous() for c in range(T4 // chunk)]
    zero = torch.zeros(B4, dtype=torch.int32, device="cuda")
    cpos = [torch.full((B4,), c * chunk, dtype=torch.int32, device="cuda")
            for c in range(T4 // chunk)]
    torch.cuda.synchronize()
    bulk_ms = _timed(torch, lambda: tq.append(cache, cbk, cbv, sbd, kp, vp, zero, host_max_pos=0),
                     args.steps, args.warmup)

    def chunked():
        for c in range(T4 // chunk):
            tq.append(cache, cbk, cbv, sbd, kc[c], vc[c], cpos[c], host_max_pos=c * chunk)

    chunk_ms = _timed(torch, chunked, args.steps, args.warmup)
    nbytes = L4 * B4 * H * T4 * encode_bytes_per_token_head(d, bk, bv)
    gbs = nbytes / (bulk_ms * 1e-3) / 1e9
    del kp, vp, kc, vc, cache
    torch.cuda.synchronize()
    return {"layers": L4, "kv_heads": H, "head_dim": d, "batch": B4, "tokens": T4,
            "bits_k": bk, "bits_v": bv, "encode_ms": bulk_ms,
            "encode_tokens_per_s": T4 * B4 / (bulk_ms * 1e-3), "encode_gbs": gbs,
            "pct_hbm_peak": 100 * gbs / HBM_PEAK_GBS, "bytes_per_launch": nbytes,
            "chunked_16x2048_ms": chunk_ms,
            "chunked_pct_hbm_peak": 100 * nbytes / (chunk_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def workload_encode_48l(args):
    """The 48-layer K4/V3 prefill encode on a line of its own (encode_48l)."""
    import torch
    torch.cuda.set_device(0)
    r = encode_48l(args)
    _report({"workload": "48-layer 32K prefill encode", "layers": r["layers"],
             "kv_heads": r["kv_heads"], "head_dim": r["head_dim"], "batch": r["batch"],
             "tokens": r["tokens"], "bits_k": r["bits_k"], "bits_v": r["bits_v"]},
            "encode tokens/s (32K prefill, all 48 layers, one tq_append)",
            r["encode_tokens_per_s"], "tokens/s", True,
            {"dtype": "f32 (f16 matrix-core transform; packed 4-bit K, 3-bit V)",
             "encode_ms": r["encode_ms"], "encode_gbs": r["encode_gbs"],
             "pct_hbm_peak": r["pct_hbm_peak"], "bytes_per_launch": r["bytes_per_launch"],
             "chunked_16x2048_ms": r["chunked_16x2048_ms"],
             "chunked_pct_hbm_peak": r["chunked_pct_hbm_peak"]}, args, r["encode_ms"])


def workload_70b_128k(args):
    """80 layers, 64 query / 8 KV heads (group 8), d 128, batch 4, 131072-token
    context, K4/V2 (33.5 GB packed cache): one decode step over all layers
    (timed); plus one layer at d 64 and one at d 256 with the same batch,
    heads and context (timed on their own)."""
    import numpy as np
    import torch
    import kv_cache_quantization_tq_amd as tq
    import synth
    seed, L, B, H, HQ, d, T, bk, bv = 1005, 80, 4, 8, 64, 128, 131072, 4, 2
    torch.cuda.set_device(0)
    res = {}
    for dd, layers, first in ((d, L, 0), (64, 1, 80), (256, 1, 81)):
        cache = tq.KVCache(layers, B, H, dd, bk, bv, T)
        cbk, cbv = tq.Codebook(dd, bk), tq.Codebook(dd, bv)
        sbd = torch.from_numpy(np.stack([synth.sign_bits(seed, first + l, dd)
                                         for l in range(layers)])).cuda()
        zero = torch.zeros(B, dtype=torch.int32, device="cuda")
        for l in range(layers):
            k = torch.empty((1, B, H, T, dd), dtype=torch.int16, device="cuda")
            v = torch.empty_like(k)
            synth.kv_dev(seed, 0, first + l, k[0])
            synth.kv_dev(seed, 1, first + l, v[0])
            tq.append(cache, cbk, cbv, sbd[l:l + 1], k, v, zero, host_max_pos=0, layer0=l,
                      n_layers=1)
            del k, v
        q = torch.empty((layers, B, HQ, dd), dtype=torch.int16, device="cuda")
        for l in range(layers):
            synth.q_dev(seed, 0, first + l, q[l])
        lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
        out = torch.empty((layers, B, HQ, dd), dtype=torch.float32, device="cuda")
        ws = tq.workspace(cache, HQ, T)
        torch.cuda.synchronize()
        ms = _timed(torch, lambda: tq.decode(cache, cbk, cbv, sbd, q, lens, T, out, ws),
                    args.steps, args.warmup)
        nbytes = layers * B * H * T * per_token_head_bytes(dd, bk, bv)
        res[dd] = (ms, nbytes)
        del cache, q, out, ws
        torch.cuda.synchronize()
        print(f"70b-128k: d {dd}: {ms * 1e3:.1f} us per step", file=sys.stderr, flush=True)
    ms, nbytes = res[d]
    gbs = nbytes / (ms * 1e-3) / 1e9
    extra = {"dtype": "f32 (f16 matrix-core operands; packed 4-bit K, 2-bit V)",
             "decode_us": ms * 1e3, "packed_gbs": gbs, "pct_hbm_peak": 100 * gbs / HBM_PEAK_GBS,
             "bytes_per_step": nbytes}
    for dd in (64, 256):
        m2, b2 = res[dd]
        extra[f"d{dd}_layer_decode_us"] = m2 * 1e3
        extra[f"d{dd}_layer_pct_hbm_peak"] = 100 * b2 / (m2 * 1e-3) / 1e9 / HBM_PEAK_GBS
    _report({"workload": "70b-shaped 128K-context decode", "layers": L, "q_heads": HQ,
             "kv_heads": H, "head_dim": d, "batch": B, "context": T, "bits_k": bk, "bits_v": bv},
            "decode tokens/s (batch / step time, all 80 layers)", B / (ms * 1e-3), "tokens/s",
            True, extra, args, ms)


def workload_tiny(args):
    """1 layer, 2 KV and 2 query heads, d 128, 512 tokens, K4/V2: encode of
    the 512 tokens and one decode step, timed (latency-bound)."""
    import numpy as np
    import torch
    import kv_cache_quantization_tq_amd as tq
    import synth
    seed, L, B, H, HQ, d, T, bk, bv = 1001, 1, 1, 2, 2, 128, 512, 4, 2
    torch.cuda.set_device(0)
    cache = tq.KVCache(L, B, H, d, bk, bv, T)
    cbk, cbv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    sbd = torch.from_numpy(synth.sign_bits(seed, 0, d)[None]).cuda()
    k = torch.empty((1, B, H, T, d), dtype=torch.int16, device="cuda")
    v = torch.empty_like(k)
    synth.kv_dev(seed, 0, 0, k[0])
    synth.kv_dev(seed, 1, 0, v[0])
    q = torch.empty((1, B, HQ, d), dtype=torch.int16, device="cuda")
    synth.q_dev(seed, 0, 0, q[0])
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    out = torch.empty((1, B, HQ, d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(cache, HQ, T)
    enc_ms = _timed(torch, lambda: tq.append(cache, cbk, cbv, sbd, k, v, zero, host_max_pos=0),
                    args.steps, args.warmup)
    dec_ms = _timed(torch, lambda: tq.decode(cache, cbk, cbv, sbd, q, lens, T, out, ws),
                    args.steps, args.warmup)
    _report({"workload": "tiny single layer", "layers": L, "q_heads": HQ, "kv_heads": H,
             "head_dim": d, "batch": B, "context": T, "bits_k": bk, "bits_v": bv},
            "decode-step latency (us, latency-bound; no roofline claim)", dec_ms * 1e3, "us", False,
            {"dtype": "f32 (f16 matrix-core operands; packed 4-bit K, 2-bit V)",
             "encode_us": enc_ms * 1e3, "decode_us": dec_ms * 1e3}, args, enc_ms + dec_ms)


def workload_paged_llama8b(args):
    """The 32K workload (32 layers, 32 query / 8 KV heads, d 128, K4/V2) in
    paged storage: 256-token pages, the pool's pages assigned to the batch in
    shuffled order.  Times the 32K prefill append and one decode step, as the
    default line does, so the two layouts can be compared."""
    import numpy as np
    import torch
    import kv_cache_quantization_tq_amd as tq
    import synth
    P = 256
    torch.cuda.set_device(0)
    cap = T + 256
    maxp = cap // P
    rng = np.random.default_rng(7)
    num_pages = B * maxp
    table = rng.permutation(num_pages).reshape(B, maxp).astype(np.int32)
    cache = tq.PagedKVCache(L, B, HKV, D, BK, BV, P, maxp, num_pages, table)
    cbk, cbv = tq.Codebook(D, BK), tq.Codebook(D, BV)
    sbs = torch.from_numpy(np.stack([synth.sign_bits(SEED, l, D) for l in range(L)])).cuda()
    k = torch.empty((L, B, HKV, T, D), dtype=torch.int16, device="cuda")
    v = torch.empty_like(k)
    for l in range(L):
        synth.kv_dev(SEED, 0, l, k[l])
        synth.kv_dev(SEED, 1, l, v[l])
    q = torch.empty((L, B, HQ, D), dtype=torch.int16, device="cuda")
    for l in range(L):
        synth.q_dev(SEED, 0, l, q[l])
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    out = torch.empty((L, B, HQ, D), dtype=torch.float32, device="cuda")
    ws = tq.workspace(cache, HQ, T)
    torch.cuda.synchronize()
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    enc_ms = _timed(torch, lambda: tq.append(cache, cbk, cbv, sbs, k, v, zero, host_max_pos=0),
                    args.steps, args.warmup)
    dec_ms = _timed(torch, lambda: tq.decode(cache, cbk, cbv, sbs, q, lens, T, out, ws),
                    args.steps, args.warmup)
    dec_bytes = L * B * HKV * T * per_token_head_bytes()
    enc_bytes = L * B * HKV * T * encode_bytes_per_token_head()
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    _report({"workload": "llama3-8b-shaped 32K decode + prefill, paged (256-token pages, "
                         "shuffled)", "layers": L, "q_heads": HQ, "kv_heads": HKV, "head_dim": D,
             "batch": B, "context": T, "bits_k": BK, "bits_v": BV, "page_tokens": P},
            "decode-attn GB/s over packed KV, paged storage", dec_gbs, "GB/s", True,
            {"dtype": "f32 (f16 matrix-core operands; packed 4-bit K, 2-bit V)",
             "decode_us": dec_ms * 1e3, "decode_pct_hbm_peak": 100 * dec_gbs / HBM_PEAK_GBS,
             "encode_ms": enc_ms,
             "encode_pct_hbm_peak": 100 * enc_bytes / (enc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
            args, enc_ms + dec_ms)


def workload_sparse_v(args):
    """The 32K decode (32 layers, 32 query / 8 KV heads, d 128, K4/V2) with the
    Sparse V gate at thresholds 1e-6, 1e-4 and 1e-3 against the dense decode
    on the same cache; reports the tiles skipped and the time of each.  The
    four are timed interleaved: in each round every one runs 5 launches
    (order reversed every other round), and the reported time is the median
    over the rounds of the per-launch mean.  Launch times drift by up to ~50%
    over runs of a few milliseconds of back-to-back decodes (the clock
    following the load), so timing the thresholds one after another would
    compare different clock states."""
    import numpy as np
    import torch
    import kv_cache_quantization_tq_amd as tq
    import synth
    torch.cuda.set_device(0)
    cache = tq.KVCache(L, B, HKV, D, BK, BV, T + 32)
    cbk, cbv = tq.Codebook(D, BK), tq.Codebook(D, BV)
    sbs = torch.from_numpy(np.stack([synth.sign_bits(SEED, l, D) for l in range(L)])).cuda()
    _fill_cache(torch, tq, synth, cache, cbk, cbv, sbs, SEED, L, B, HKV, T, D)
    q = torch.empty((L, B, HQ, D), dtype=torch.int16, device="cuda")
    for l in range(L):
        synth.q_dev(SEED, 0, l, q[l])
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    out = torch.empty((L, B, HQ, D), dtype=torch.float32, device="cuda")
    ws = tq.workspace(cache, HQ, T)
    torch.cuda.synchronize()
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    dec_bytes = L * B * HKV * T * per_token_head_bytes()
    tiles = L * B * HKV * (T // 32)
    v_tile_bytes = 32 * (D * BV // 8 + 2)
    thresholds = (1e-6, 1e-4, 1e-3)
    skipped = {}
    for eps in thresholds:
        cnt = torch.zeros((L, B, HKV), dtype=torch.int32, device="cuda")
        tq.decode_sparse(cache, cbk, cbv, sbs, q, lens, T, out, eps, ws, skip_counts=cnt)
        torch.cuda.synchronize()
        skipped[eps] = int(cnt.sum().item())
    runs = [(0.0, lambda: tq.decode(cache, cbk, cbv, sbs, q, lens, T, out, ws))]
    runs += [(eps, lambda e=eps: tq.decode_sparse(cache, cbk, cbv, sbs, q, lens, T, out, e, ws))
             for eps in thresholds]
    per, rounds = 5, max(args.steps, 10)
    times = {eps: [] for eps, _ in runs}
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for r in range(args.warmup + rounds):
        for eps, fn in (runs if r % 2 == 0 else runs[::-1]):
            ev0.record()
            for _ in range(per):
                fn()
            ev1.record()
            torch.cuda.synchronize()
            if r >= args.warmup:
                times[eps].append(ev0.elapsed_time(ev1) / per)
    med = {eps: float(np.median(t)) for eps, t in times.items()}
    res = {"dense_us": med[0.0] * 1e3}
    for eps in thresholds:
        key = f"eps_{eps:g}"
        ms = med[eps]
        res[key + "_us"] = ms * 1e3
        res[key + "_skipped_tile_frac"] = skipped[eps] / tiles
        res[key + "_bytes_read_gbs"] = (dec_bytes - skipped[eps] * v_tile_bytes) / (ms * 1e-3) / 1e9
        res[key + "_vs_dense"] = med[0.0] / ms
    best = med[1e-3]
    _report({"workload": "llama3-8b-shaped 32K decode with the Sparse V gate", "layers": L,
             "q_heads": HQ, "kv_heads": HKV, "head_dim": D, "batch": B, "context": T,
             "bits_k": BK, "bits_v": BV, "eps": 1e-3},
            "decode-attn dense-equivalent GB/s (packed KV bytes a dense decode reads / time), "
            "Sparse V at eps 1e-3", dec_bytes / (best * 1e-3) / 1e9, "GB/s", True,
            dict(dtype="f32 (f16 matrix-core operands; packed 4-bit K, 2-bit V)",
                 timing=f"interleaved: {rounds} rounds x {per} launches per threshold, medians",
                 **res),
            argparse.Namespace(steps=rounds, warmup=args.warmup), best)


def workload_prefill(args):
    """Causal prefill attention over the compressed cache for the 32K workload
    (32 layers, 32 query / 8 KV heads, d 128, K4/V2): the whole 32768-token
    prompt is appended, then every prompt token attends to its prefix
    (tq_prefill_attn, one call for all layers).  Matrix-core bound: reported
    against the fp16 dense peak with the algorithmic flops of causal
    attention, 4 d per (query, key) pair."""
    import numpy as np
    import torch
    import kv_cache_quantization_tq_amd as tq
    import synth
    torch.cuda.set_device(0)
    Tp = int(os.environ.get("TQ_PREFILL_TOKENS", T))
    cache = tq.KVCache(L, B, HKV, D, BK, BV, Tp)
    cbk, cbv = tq.Codebook(D, BK), tq.Codebook(D, BV)
    sbs = torch.from_numpy(np.stack([synth.sign_bits(SEED, l, D) for l in range(L)])).cuda()
    _fill_cache(torch, tq, synth, cache, cbk, cbv, sbs, SEED, L, B, HKV, Tp, D)
    # queries: the decode query generator, one step per prompt position
    q = torch.empty((L, B, HQ, Tp, D), dtype=torch.int16, device="cuda")
    qs = torch.empty((B, HQ, D), dtype=torch.int16, device="cuda")
    for l in range(L):
        synth.q_dev(SEED, 0, l, qs)
        q[l] = qs[:, :, None, :]
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.empty((L, B, HQ, Tp, D), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    ms = _timed(torch, lambda: tq.prefill(cache, cbk, cbv, sbs, q, pos, out), args.steps,
                args.warmup)
    pairs = Tp * (Tp + 1) // 2
    flops = 4.0 * D * pairs * HQ * L * B
    tfs = flops / (ms * 1e-3) / 1e12
    _report({"workload": "llama3-8b-shaped 32K causal prefill attention over the packed cache",
             "layers": L, "q_heads": HQ, "kv_heads": HKV, "head_dim": D, "batch": B,
             "prompt": Tp, "bits_k": BK, "bits_v": BV},
            "prefill-attn TFLOP/s (4 d flops per causal query-key pair)", tfs, "TFLOP/s", True,
            {"dtype": "f32 (f16 matrix-core operands; packed 4-bit K, 2-bit V)",
             "prefill_ms": ms, "tokens_per_s": Tp * B / (ms * 1e-3),
             "roofline": {"bound": "mfma", "kernel": "prefill32_kernel<128,4,2>", "achieved": tfs,
                          "peak": 2500.0, "unit": "TFLOP/s", "frac": tfs / 2500.0,
                          "traffic": None}},
            args, ms)


def workload_qjl(args):
    """The QJL stage on the keys of the 32K workload (32 layers x 8 KV heads x
    32768 tokens, d 128, 4-bit keys): tq_qjl_encode over all 8.4M keys (after
    tq_encode), then tq_qjl_scores of 4 queries against all of them.  Both
    stream HBM: per key the sketch reads the fp16 key and its codes and
    writes d/8 sign bytes and gamma; the estimate reads codes, signs, norm and
    gamma and writes 4 floats."""
    import numpy as np
    import torch
    import kv_cache_quantization_tq_amd as tq
    import synth
    torch.cuda.set_device(0)
    n = L * B * HKV * T
    x = torch.empty((L, B, HKV, T, D), dtype=torch.int16, device="cuda")
    for l in range(L):
        synth.kv_dev(SEED, 0, l, x[l])
    x = x.view(n, D)
    cb = tq.Codebook(D, BK)
    sb = torch.from_numpy(synth.sign_bits(SEED, 0, D)).cuda()
    rng = np.random.default_rng(SEED)
    S = torch.from_numpy(rng.standard_normal((D, D)).astype(np.float16).view(np.int16)).cuda()
    codes = torch.empty((n, D * BK // 8), dtype=torch.uint8, device="cuda")
    norms = torch.empty(n, dtype=torch.int16, device="cuda")
    signs = torch.empty((n, D // 8), dtype=torch.uint8, device="cuda")
    gamma = torch.empty(n, dtype=torch.int16, device="cuda")
    tq.encode(cb, x, sb, codes, norms)
    q = torch.empty((1, 4, D), dtype=torch.int16, device="cuda")
    synth.q_dev(SEED, 0, 0, q)
    q = q.view(4, D)
    out = torch.empty((4, n), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    enc_ms = _timed(torch, lambda: tq.qjl_encode(cb, x, sb, S, codes, signs, gamma), args.steps,
                    args.warmup)
    sc_ms = _timed(torch, lambda: tq.qjl_scores(cb, q, sb, S, codes, norms, signs, gamma, out),
                   args.steps, args.warmup)
    enc_b = n * (2 * D + D * BK // 8 + D // 8 + 2)
    sc_b = n * (D * BK // 8 + D // 8 + 2 + 2 + 4 * 4)
    enc_gbs = enc_b / (enc_ms * 1e-3) / 1e9
    sc_gbs = sc_b / (sc_ms * 1e-3) / 1e9
    _report({"workload": "QJL sketch and estimate over the keys of the 32K workload",
             "keys": n, "head_dim": D, "bits_k": BK, "queries": 4},
            "QJL sketch GB/s (fp16 keys + codes read, signs + gamma written)", enc_gbs, "GB/s",
            True,
            {"dtype": "f32 (f16 matrix-core operands for S r)",
             "qjl_encode_ms": enc_ms, "qjl_encode_keys_per_s": n / (enc_ms * 1e-3),
             "qjl_scores_ms": sc_ms, "qjl_scores_gbs": sc_gbs,
             "roofline": {"bound": "hbm", "kernel": "qjl_encode_kernel<128,4>",
                          "achieved": enc_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": enc_gbs / HBM_PEAK_GBS,
                          "traffic": measured_traffic("qjl_encode_kernel<128,4>")},
             "roofline_scores": {"bound": "hbm", "kernel": "qjl_scores_kernel<128,4>",
                                 "achieved": sc_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": sc_gbs / HBM_PEAK_GBS,
                                 "traffic": measured_traffic("qjl_scores_kernel<128,4>")}},
            args, enc_ms + sc_ms)


WORKLOADS = {
    "llama8b-32k": None,
    "tiny": workload_tiny,
    "batched-decode-b16-8k": workload_batched_decode,
    "encode-48l-32k": workload_encode_48l,
    "70b-128k-b4": workload_70b_128k,
    "paged-llama8b-32k": workload_paged_llama8b,
    "sparse-v-llama8b-32k": workload_sparse_v,
    "prefill-llama8b-32k": workload_prefill,
    "qjl-llama8b-32k": workload_qjl,
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--workload", default="llama8b-32k", choices=sorted(WORKLOADS),
                    help="llama8b-32k (the metric's workload, default) or one of the other "
                         "workload shapes, timed and reported on a line of its own")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported (across "
              "GPUs the path would shard by KV head, with no exchange between them)",
              file=sys.stderr)
        sys.exit(2)

    if args.workload != "llama8b-32k":
        WORKLOADS[args.workload](args)
        return

    import torch
    import kv_cache_quantization_tq_amd as tq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    cap = T + 32
    cache = tq.KVCache(L, B, HKV, D, BK, BV, cap)
    cbk, cbv = tq.Codebook(D, BK), tq.Codebook(D, BV)
    import numpy as np
    sbs = torch.from_numpy(np.stack([synth.sign_bits(SEED, l, D) for l in range(L)])).cuda()
    k_pre = torch.empty((L, B, HKV, T, D), dtype=torch.int16, device=dev)
    v_pre = torch.empty_like(k_pre)
    k_new = torch.empty((L, B, HKV, 1, D), dtype=torch.int16, device=dev)
    v_new = torch.empty_like(k_new)
    for l in range(L):
        synth.kv_dev(SEED, 0, l, k_pre[l])
        synth.kv_dev(SEED, 1, l, v_pre[l])
        synth.kv_dev(SEED, 0, l, k_new[l], t0=T)
        synth.kv_dev(SEED, 1, l, v_new[l], t0=T)
    q = torch.empty((L, B, HQ, D), dtype=torch.int16, device=dev)
    for l in range(L):
        synth.q_dev(SEED, 0, l, q[l])
    pos0 = torch.zeros(B, dtype=torch.int32, device=dev)
    posT = torch.full((B,), T, dtype=torch.int32, device=dev)
    ctx = T + 1
    lens = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    out = torch.empty((L, B, HQ, D), dtype=torch.float32, device=dev)
    ws = tq.workspace(cache, HQ, ctx)
    torch.cuda.synchronize()

    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev):
        ev[0].record(stream)
        tq.append(cache, cbk, cbv, sbs, k_pre, v_pre, pos0, host_max_pos=0)
        ev[1].record(stream)
        tq.append(cache, cbk, cbv, sbs, k_new, v_new, posT, host_max_pos=T)
        ev[2].record(stream)
        tq.decode(cache, cbk, cbv, sbs, q, lens, ctx, out, ws)
        ev[3].record(stream)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
           for _ in range(args.warmup + args.steps)]
    for i in range(args.warmup):
        step(evs[i])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[args.warmup + i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    timed = evs[args.warmup:]
    enc_ms = sum(e[0].elapsed_time(e[1]) for e in timed) / args.steps
    app_ms = sum(e[1].elapsed_time(e[2]) for e in timed) / args.steps
    dec_ms = sum(e[2].elapsed_time(e[3]) for e in timed) / args.steps
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    dec_bytes = L * B * HKV * ctx * per_token_head_bytes()
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    enc_bytes = L * B * HKV * T * encode_bytes_per_token_head()
    enc_gbs = enc_bytes / (enc_ms * 1e-3) / 1e9
    line = {
        "metric": "decode-attn GB/s over packed KV (% of HBM peak); encode tokens/s at 32K ctx",
        "value": dec_gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (f16 matrix-core operands; packed 4-bit K, 2-bit V)",
        "data": "synthetic (seeded fp16 K/V with outlier channels and lognormal token scale)",
        "config": {"workload": "llama3-8b-shaped decode + 32K prefill encode", "layers": L,
                   "q_heads": HQ, "kv_heads": HKV, "head_dim": D, "batch": B,
                   "context": ctx, "bits_k": BK, "bits_v": BV, "parallelism": "none"},
        "decode_us": dec_ms * 1e3,
        "decode_pct_hbm_peak": 100 * dec_gbs / HBM_PEAK_GBS,
        "decode_tokens_per_s": B / (dec_ms * 1e-3),
        "encode_ms": enc_ms,
        "encode_tokens_per_s": T * B / (enc_ms * 1e-3),
        "encode_gbs": enc_gbs,
        "encode_pct_hbm_peak": 100 * enc_gbs / HBM_PEAK_GBS,
        "append_us": app_ms * 1e3,
        "roofline": {"bound": "hbm", "kernel": "decode_kernel<128,4,2,4>",
                     "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dec_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic("decode_kernel<128,4,2,4>"),
                     "bytes_per_launch": dec_bytes, "avg_launch_us": dec_ms * 1e3},
        "roofline_encode": {"bound": "hbm", "kernel": "append_kernel<128,4,2>",
                            "achieved": enc_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": enc_gbs / HBM_PEAK_GBS,
                            "traffic": measured_traffic("append_kernel<128,4,2>"),
                            "bytes_per_launch": enc_bytes, "avg_launch_us": enc_ms * 1e3},
    }
    # the 48-layer K4/V3 prefill encode (the dedicated encode workload), timed
    # after the steps above
    e48 = encode_48l(args)
    line["encode_48l_k4v3"] = {k: e48[k] for k in (
        "encode_ms", "encode_tokens_per_s", "pct_hbm_peak", "chunked_16x2048_ms",
        "chunked_pct_hbm_peak")}
    line["roofline_encode_48l"] = {
        "bound": "hbm", "kernel": "append_kernel<128,4,3>", "achieved": e48["encode_gbs"],
        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": e48["encode_gbs"] / HBM_PEAK_GBS,
        "traffic": measured_traffic("append_kernel<128,4,3>"),
        "bytes_per_launch": e48["bytes_per_launch"], "avg_launch_us": e48["encode_ms"] * 1e3}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline((cache, out, q))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
