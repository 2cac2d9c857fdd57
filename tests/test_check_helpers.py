"""The attention check's band-flip bound, tested on the CPU against brute
force: each band coordinate's code is flipped alone in the oracle's cache, the
attention recomputed, and the bound must be the sum of those exact changes."""
import numpy as np
import pytest

import oracle
import synth
from helpers import band_flip_bound


@pytest.mark.parametrize("d,bk,bv", [(64, 4, 2), (128, 3, 3)])
def test_band_flip_bound_matches_single_flips(d, bk, bv):
    seed, T, G = 77, 40, 3
    k = synth.kv_host(seed, 0, 0, 0, 0, d, 0, T)
    v = synth.kv_host(seed, 1, 0, 0, 0, d, 0, T)
    q16 = np.stack([synth.q_host(seed, 0, 0, 0, g, d) for g in range(G)])
    sb = synth.sign_bits(seed, 0, d)
    st = oracle.decode_stream(k, v, q16, bk, bv, sb, full=True)
    q64 = oracle.halves_to_double(q16)
    thr = 4e-3  # wide enough that a few coordinates of this tiny stream are "band"
    bound, nb = band_flip_bound(q64, k, v, st, bk, bv, sb, threshold=thr)
    assert nb > 0
    ck, tk = oracle.codebook(d, bk)
    cv, tv = oracle.codebook(d, bv)
    R = oracle.rotation(d, sb)
    total = np.zeros_like(bound)
    for kind, codes, band, x16, t in (("k", st["k_codes"], st["k_band"], k, tk),
                                      ("v", st["v_codes"], st["v_band"], v, tv)):
        for j, i in np.argwhere(band < thr):
            x = x16[j].view(np.float16).astype(np.float64)
            y = R[i] @ x / np.linalg.norm(x)
            near = int(np.argmin(np.abs(y - t)))
            c2 = codes.copy()
            c2[j, i] = near + 1 if codes[j, i] == near else near
            if kind == "k":
                K2 = oracle.dequant(c2, st["k_norms"], bk, sb)
                o2 = oracle.attention(q64, K2, st["V"])
            else:
                V2 = oracle.dequant(c2, st["v_norms"], bv, sb)
                o2 = oracle.attention(q64, st["K"], V2)
            assert abs(int(c2[j, i]) - int(codes[j, i])) == 1
            total += np.abs(o2 - st["out"])
    np.testing.assert_allclose(bound, total, rtol=1e-9, atol=1e-15)


def test_band_flip_bound_empty_and_bandless():
    d = 64
    sb = synth.sign_bits(5, 0, d)
    q16 = np.stack([synth.q_host(5, 0, 0, 0, 0, d)])
    k = synth.kv_host(5, 0, 0, 0, 0, d, 0, 8)
    st = oracle.decode_stream(k, k, q16, 2, 2, sb, full=True)
    b, nb = band_flip_bound(oracle.halves_to_double(q16), k, k, st, 2, 2, sb, threshold=0.0)
    assert nb == 0 and not b.any()
    e = k[:0]
    st0 = oracle.decode_stream(e, e, q16, 2, 2, sb, full=True)
    b0, nb0 = band_flip_bound(oracle.halves_to_double(q16), e, e, st0, 2, 2, sb)
    assert nb0 == 0 and b0.shape == (1, d) and not b0.any()
