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
kernel's roofline fraction against the 8 TB/s HBM peak, and the CPU oracle
timed on a bounded sample on this host.
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


def cpu_baseline(seconds_budget=20.0):
    """The oracle (single thread, plain loops, fp64) on a sample of the same
    workload: whole (layer 0, KV head h) streams, 32768 tokens each, encoded and
    then attended by their 4 query heads; streams are added until the budget is
    spent.  Scaled to the metric's units."""
    import numpy as np
    import oracle
    import synth
    sb = synth.sign_bits(SEED, 0, D)
    enc_s = dec_s = 0.0
    n_streams = 0
    t_start = time.perf_counter()
    for h in range(HKV):
        k = synth.kv_host(SEED, 0, 0, 0, h, D, 0, T)
        v = synth.kv_host(SEED, 1, 0, 0, h, D, 0, T)
        q = np.stack([synth.q_host(SEED, 0, 0, 0, h * 4 + g, D) for g in range(4)])
        t0 = time.perf_counter()
        kc, kn, _ = oracle.encode(k, BK, sb, want_band=False)
        vc, vn, _ = oracle.encode(v, BV, sb, want_band=False)
        t1 = time.perf_counter()
        K = oracle.dequant(kc, kn, BK, sb)
        V = oracle.dequant(vc, vn, BV, sb)
        oracle.attention(oracle.halves_to_double(q), K, V)
        t2 = time.perf_counter()
        enc_s += t1 - t0
        dec_s += t2 - t1
        n_streams += 1
        if time.perf_counter() - t_start > seconds_budget:
            break
    dec_gbs = n_streams * T * per_token_head_bytes() / dec_s / 1e9
    enc_tok_s = n_streams * T / enc_s / (L * HKV)  # context tokens/s over all layers and heads
    return {
        "value": dec_gbs, "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"{n_streams} of {L * HKV} (layer, KV head) streams, {T} tokens each, "
                  f"encode + dequantize + attention by 4 query heads",
        "encode_tokens_per_s": enc_tok_s,
        "seconds": enc_s + dec_s,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by KV head with no exchange; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

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
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
