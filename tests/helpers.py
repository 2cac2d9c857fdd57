"""Shared helpers for the GPU tests: seeded inputs and GPU/oracle comparisons.

Attention parity follows the target's bars with nothing widened: the GPU's
output is within 2e-3 relative L2 and 1e-2 max-abs of the oracle's attention
over the same dequantized cache.  "The same cache" is the oracle's own
encoding of the same seeded fp16 inputs, taken code for code; only at a
coordinate within 1e-6 of a decision threshold, where either neighbouring
code is a correct encoding, may the GPU have taken the other one, and there
the oracle takes its own alternative code (the neighbour across that
threshold, computed by the oracle).  Every GPU code is checked to be one of
the oracle's two candidates first, and norms are checked bit for bit, so no
value the oracle attends over comes from the GPU path.
"""
import numpy as np

import oracle
import synth

REL_L2 = 2e-3
MAX_ABS = 1e-2
BAND = 1e-6
MISMATCH_FRAC = 1e-5


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (none visible)")
    return torch


def kv_stream_host(seed, kind, layer, seq, head, d, t0, nt):
    return synth.kv_host(seed, kind, layer, seq, head, d, t0, nt)


def compare_codes(gpu_codes, ora_codes, ora_band, what="", max_frac=MISMATCH_FRAC):
    """Codes equal except within 1e-6 of a threshold; on the seeded random
    workloads those mismatches must also stay under 1e-5 of all codes
    (max_frac=None for hand-built inputs that sit on thresholds on purpose).
    Returns the number of mismatches."""
    mism = gpu_codes != ora_codes
    n_mis = int(mism.sum())
    total = gpu_codes.size
    if n_mis:
        worst = float(ora_band[mism].max())
        assert worst < BAND, f"{what}: code mismatch {worst:.3g} away from a threshold"
    if max_frac is not None:
        assert n_mis < max_frac * total or n_mis == 0, f"{what}: {n_mis} of {total} codes differ"
    return n_mis


def resolve_codes(gpu_codes, ora_codes, ora_band, ora_alt, what=""):
    """The codes the oracle attends over: its own, except at band coordinates
    (within 1e-6 of a threshold) where the GPU took the other neighbouring
    code, where it takes its own alternative.  Fails if any GPU code is
    neither of the oracle's two candidates.  Returns (codes, number taken from
    the alternatives)."""
    mism = gpu_codes != ora_codes
    n = int(mism.sum())
    if n:
        worst = float(ora_band[mism].max())
        assert worst < BAND, f"{what}: code mismatch {worst:.3g} away from a threshold"
        bad = gpu_codes[mism] != ora_alt[mism]
        assert not bad.any(), f"{what}: {int(bad.sum())} band codes are not the neighbouring code"
        out = ora_codes.copy()
        out[mism] = ora_alt[mism]
        return out, n
    return ora_codes, 0


def gpu_stream(cache, layer, b, h, n):
    """The first n tokens of one (layer, sequence, KV head) stream of a GPU
    cache (contiguous or paged), read back and unpacked with the oracle's
    unpackers: dict(k_codes [n][d], k_norms [n], v_codes [n][d], v_norms [n])."""
    d, bk, bv = cache.head_dim, cache.bits_k, cache.bits_v
    if hasattr(cache, "gather"):
        kc, vc, kn, vn = cache.gather(layer, b, h)
    else:
        kc, vc = cache.k_codes[layer, b, h], cache.v_codes[layer, b, h]
        kn, vn = cache.k_norms[layer, b, h], cache.v_norms[layer, b, h]
    nt = (n + 31) // 32
    return dict(
        k_codes=oracle.unpack_rows(kc[:n].cpu().numpy(), d, bk),
        k_norms=kn[:n].cpu().numpy().view(np.uint16),
        v_codes=oracle.unpack_vtiles(vc[:nt].cpu().numpy(), d, bv)[:n],
        v_norms=vn[:n].cpu().numpy().view(np.uint16))


def oracle_stream(k16, v16, bk, bv, sign_bits, gpu, what=""):
    """Encode one stream with the oracle, check the GPU's norms (bit for bit)
    and codes (the band rule) of it, and dequantize the oracle's codes,
    resolved where the GPU took the other band neighbour.

    Returns dict(K [n][d], V [n][d] (original domain, fp64), n_alt (codes
    taken from the oracle's alternatives), n_coords)."""
    kc, kn, kb, ka = oracle.encode(k16, bk, sign_bits, want_alt=True)
    vc, vn, vb, va = oracle.encode(v16, bv, sign_bits, want_alt=True)
    assert np.array_equal(gpu["k_norms"], kn), f"{what}: key norms differ"
    assert np.array_equal(gpu["v_norms"], vn), f"{what}: value norms differ"
    kr, nk = resolve_codes(gpu["k_codes"], kc, kb, ka, what + " keys")
    vr, nv = resolve_codes(gpu["v_codes"], vc, vb, va, what + " values")
    return dict(K=oracle.dequant(kr, kn, bk, sign_bits), V=oracle.dequant(vr, vn, bv, sign_bits),
                n_alt=nk + nv, n_coords=kc.size + vc.size)


def check_mismatch_fraction(n_alt, n_coords, what=""):
    """The band mismatches of a test's streams stay under 1e-5 of their coordinates."""
    print(f"{what}: {n_alt} band coordinates of {n_coords} where the GPU took the other "
          f"neighbouring code", flush=True)
    assert n_alt < MISMATCH_FRAC * n_coords or n_alt == 0, (n_alt, n_coords)


def attention_errors(gpu_out, ref_out):
    g = np.asarray(gpu_out, dtype=np.float64)
    r = np.asarray(ref_out, dtype=np.float64)
    rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    mx = float(np.abs(g - r).max()) if g.size else 0.0
    return rel, mx


def check_attention(gpu, ref, what="", n_alt=0):
    """GPU output within 2e-3 relative L2 and 1e-2 max-abs of the oracle's."""
    rel, mx = attention_errors(gpu, ref)
    print(f"{what}: rel-L2 {rel:.3e} (bar {REL_L2:.0e}), max-abs {mx:.3e} (bar {MAX_ABS:.0e}), "
          f"{n_alt} band codes resolved to the GPU's neighbour", flush=True)
    assert rel <= REL_L2, (what, rel)
    assert mx <= MAX_ABS, (what, mx)


def oracle_attention_stream(seed, layer, b, h, n, bk, bv, sign_bits, q16, gpu, what=""):
    """The oracle's attention of the G queries q16[G][d] over the first n
    tokens of the seeded stream (generator layer `layer`, sequence b, head h),
    over the cache resolved against `gpu` (gpu_stream of that stream).
    Returns (out [G][d], n_alt, n_coords)."""
    d = q16.shape[-1]
    k = synth.kv_host(seed, 0, layer, b, h, d, 0, n)
    v = synth.kv_host(seed, 1, layer, b, h, d, 0, n)
    st = oracle_stream(k, v, bk, bv, sign_bits, gpu, what)
    out = oracle.attention(oracle.halves_to_double(q16), st["K"], st["V"])
    return out, st["n_alt"], st["n_coords"]
