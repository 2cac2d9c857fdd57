"""Shared helpers for the GPU tests: seeded inputs, GPU/oracle comparisons."""
import math

import numpy as np

import oracle
import synth


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (none visible)")
    return torch


def kv_stream_host(seed, kind, layer, seq, head, d, t0, nt):
    return synth.kv_host(seed, kind, layer, seq, head, d, t0, nt)


def compare_codes(gpu_codes, ora_codes, ora_band, what="", max_frac=1e-5):
    """Codes equal except within 1e-6 of a threshold; on the seeded random
    workloads those mismatches must also stay under 1e-5 of all codes
    (max_frac=None for hand-built inputs that sit on thresholds on purpose)."""
    mism = gpu_codes != ora_codes
    n_mis = int(mism.sum())
    total = gpu_codes.size
    if n_mis:
        worst = float(ora_band[mism].max())
        assert worst < 1e-6, f"{what}: code mismatch {worst:.3g} away from a threshold"
    if max_frac is not None:
        assert n_mis < max_frac * total or n_mis == 0, f"{what}: {n_mis} of {total} codes differ"
    return n_mis


def attention_errors(gpu_out, ref_out):
    g = np.asarray(gpu_out, dtype=np.float64)
    r = np.asarray(ref_out, dtype=np.float64)
    rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    mx = float(np.abs(g - r).max()) if g.size else 0.0
    return rel, mx


REL_L2 = 2e-3
MAX_ABS = 1e-2


def _alt_codes(x16, codes, band, bits, sign_bits, rows_cols):
    """For band coordinates (row j, coord i), the neighbouring code across the
    nearest threshold (both readings are correct within the 1e-6 band)."""
    d = codes.shape[1]
    R = oracle.rotation(d, sign_bits)
    _, t = oracle.codebook(d, bits)
    out = []
    for j, i in rows_cols:
        x = np.asarray(x16[j], np.uint16).view(np.float16).astype(np.float64)
        nrm = np.linalg.norm(x)
        y = (R[i] @ x) / nrm if nrm > 0 else 0.0
        k = int(np.argmin(np.abs(y - t)))
        c = int(codes[j, i])
        out.append(k + 1 if c == k else k)
    return out


def band_flip_bound(q64, k16, v16, st, bits_k, bits_v, sign_bits, threshold=1e-6):
    """Elementwise bound [G][d] on how far the attention output can move when
    the oracle's band-ambiguous codes (within `threshold` of a decision
    threshold, where either neighbouring code is a correct encoding) are read
    the other way: the sum over those coordinates of the exact output change
    of flipping each one alone.  st: oracle.decode_stream(..., full=True)."""
    d = q64.shape[1]
    R = oracle.rotation(d, sign_bits)
    ck, _ = oracle.codebook(d, bits_k)
    cv, _ = oracle.codebook(d, bits_v)
    K, V, o = st["K"], st["V"], st["out"]
    if K.shape[0] == 0:
        return np.zeros_like(o), 0
    s = (q64 @ K.T) / math.sqrt(d)
    w = np.exp(s - s.max(1, keepdims=True))
    l = w.sum(1)
    p = w / l[:, None]
    bound = np.zeros_like(o)
    kb = np.argwhere(st["k_band"] < threshold)
    if len(kb):
        alt = _alt_codes(k16, st["k_codes"], st["k_band"], bits_k, sign_bits, kb)
        kn = oracle.halves_to_double(st["k_norms"])
        for (j, i), a in zip(kb, alt):
            dk = kn[j] * (ck[a] - ck[st["k_codes"][j, i]]) * R[i]
            ds = (q64 @ dk) / math.sqrt(d)
            w2 = w[:, j] * np.exp(ds)
            o2 = (o * l[:, None] + (w2 - w[:, j])[:, None] * V[j][None]) / (l + w2 - w[:, j])[:, None]
            bound += np.abs(o2 - o)
    vb = np.argwhere(st["v_band"] < threshold)
    if len(vb):
        alt = _alt_codes(v16, st["v_codes"], st["v_band"], bits_v, sign_bits, vb)
        vn = oracle.halves_to_double(st["v_norms"])
        for (j, i), a in zip(vb, alt):
            dv = vn[j] * (cv[a] - cv[st["v_codes"][j, i]]) * R[i]
            bound += np.abs(p[:, j][:, None] * dv[None])
    return bound, len(kb) + len(vb)


def check_attention(gpu, ref, bound, what=""):
    """GPU output within the bars of the oracle's, widened only by the
    band-flip bound (zero when no band coordinate exists)."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    err = np.abs(g - r)
    rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    rel_allow = REL_L2 + np.linalg.norm(bound) / max(np.linalg.norm(r), 1e-300)
    excess = float((err - bound).max()) if err.size else 0.0
    print(f"{what}: rel-L2 {rel:.3e} (allowed {rel_allow:.3e}), max-abs {err.max():.3e}, "
          f"max-abs beyond band-flip bound {excess:.3e} (bound max {bound.max():.3e})", flush=True)
    assert rel <= rel_allow, (rel, rel_allow)
    assert excess <= MAX_ABS, excess


def oracle_attention_with_bound(k16, v16, q16, bits_k, bits_v, sign_bits):
    """The oracle's attention for one stream and its band-flip bound."""
    st = oracle.decode_stream(k16, v16, q16, bits_k, bits_v, sign_bits, full=True)
    q64 = oracle.halves_to_double(q16)
    bound, nb = band_flip_bound(q64, k16, v16, st, bits_k, bits_v, sign_bits)
    return st["out"], bound, nb


def prefix(st, n):
    """The decode_stream record restricted to the first n tokens."""
    r = {k: st[k][:n] for k in ("k_codes", "k_norms", "k_band", "v_codes", "v_norms", "v_band",
                                 "K", "V")}
    return r
