"""The GPU tests' comparison helpers, tested on the CPU: the attention check
resolves band codes only to the oracle's own neighbouring code, and rejects
every other difference (a code outside the band, a band code two levels away,
a norm off by one ulp).  The "GPU" inputs here are planted on the CPU."""
import numpy as np
import pytest

import oracle
import synth
from helpers import check_attention, oracle_stream, resolve_codes


def _stream(seed=77, d=64, T=40):
    k = synth.kv_host(seed, 0, 0, 0, 0, d, 0, T)
    v = synth.kv_host(seed, 1, 0, 0, 0, d, 0, T)
    return k, v, synth.sign_bits(seed, 0, d)


def test_resolve_takes_the_oracles_neighbour_at_band_coordinates():
    k, _, sb = _stream()
    codes, _, band, alt = oracle.encode(k, 4, sb, want_alt=True)
    # a coordinate nearest its threshold stands in for a band coordinate
    j, i = np.unravel_index(int(np.argmin(band)), band.shape)
    gpu = codes.copy()
    gpu[j, i] = alt[j, i]
    band_wide = band.copy()
    band_wide[j, i] = 0.0
    out, n = resolve_codes(gpu, codes, band_wide, alt)
    assert n == 1 and np.array_equal(out, gpu) and out is not codes
    same, n0 = resolve_codes(codes.copy(), codes, band, alt)
    assert n0 == 0 and np.array_equal(same, codes)


def test_resolve_rejects_codes_that_are_not_correct_encodings():
    k, _, sb = _stream()
    codes, _, band, alt = oracle.encode(k, 4, sb, want_alt=True)
    # outside the band: any difference fails
    far = np.argwhere(band > 1e-3)[0]
    gpu = codes.copy()
    gpu[tuple(far)] = alt[tuple(far)]
    with pytest.raises(AssertionError):
        resolve_codes(gpu, codes, band, alt)
    # in the band, but two levels away from the oracle's code
    j, i = np.unravel_index(int(np.argmin(band)), band.shape)
    band_wide = band.copy()
    band_wide[j, i] = 0.0
    gpu = codes.copy()
    gpu[j, i] = (int(alt[j, i]) * 2 - int(codes[j, i])) % 16
    with pytest.raises(AssertionError):
        resolve_codes(gpu, codes, band_wide, alt)


def test_oracle_stream_checks_norms_and_dequantizes():
    k, v, sb = _stream()
    d = k.shape[1]
    kc, kn, _ = oracle.encode(k, 4, sb)
    vc, vn, _ = oracle.encode(v, 2, sb)
    gpu = dict(k_codes=kc, k_norms=kn, v_codes=vc, v_norms=vn)
    st = oracle_stream(k, v, 4, 2, sb, gpu, "cpu")
    assert st["n_alt"] == 0 and st["n_coords"] == 2 * k.size
    assert np.array_equal(st["K"], oracle.dequant(kc, kn, 4, sb))
    assert np.array_equal(st["V"], oracle.dequant(vc, vn, 2, sb))
    bad = dict(gpu, v_norms=vn + np.uint16(1))
    with pytest.raises(AssertionError):
        oracle_stream(k, v, 4, 2, sb, bad, "cpu")
    assert st["K"].shape == (k.shape[0], d)


def test_check_attention_plain_bars():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((4, 64))
    check_attention(ref + 1e-4, ref, "within")
    with pytest.raises(AssertionError):
        check_attention(ref * (1 + 3e-3), ref, "rel-L2 above 2e-3")
    off = ref.copy()
    off[0, 0] += 0.02
    with pytest.raises(AssertionError):
        check_attention(off, ref, "max-abs above 1e-2")
