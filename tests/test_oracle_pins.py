"""Pins of the CPU oracle against facts it does not produce itself.

Each test names what it pins and where the fact comes from: the pages (their
worked byte count, config table and fidelity figures), closed forms, textbook
values, algebraic identities, and brute force on tiny inputs.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import integrate, stats

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _figures():
    out = {}
    with open(os.path.join(GOLDEN, "page_figures.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                out[k] = float(v)
    return out


def _rand_signs(rng, d):
    return rng.integers(0, 256, size=d // 8, dtype=np.uint8)


# ------------------------------------------------------------------ Hadamard


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 64, 128, 256])
def test_hadamard_closed_form_and_orthogonality(d):
    """Sylvester matrix: H[i][j] = (-1)^popcount(i & j), H = H^T, H H = d I."""
    H = oracle.hadamard(d)
    ref = np.array([[(-1) ** bin(i & j).count("1") for j in range(d)] for i in range(d)])
    assert np.array_equal(H, ref)
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H, d * np.eye(d))


def test_fwht_brute_force_small():
    """A textbook in-place butterfly FWHT on the basis vectors reproduces H (d <= 16)."""
    for d in (2, 4, 8, 16):
        H = oracle.hadamard(d)
        for k in range(d):
            v = np.zeros(d)
            v[k] = 1.0
            h = 1
            while h < d:
                for i in range(0, d, 2 * h):
                    for j in range(i, i + h):
                        a, b = v[j], v[j + h]
                        v[j], v[j + h] = a + b, a - b
                h *= 2
            assert np.array_equal(v, H[:, k])


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotation_orthogonal_and_inner_products(d):
    """R = H D / sqrt(d) is orthogonal; it keeps norms and q.k = (Rq).(Rk)."""
    rng = np.random.default_rng(d)
    sb = _rand_signs(rng, d)
    R = oracle.rotation(d, sb)
    assert np.abs(R.T @ R - np.eye(d)).max() < 1e-14
    s = np.array([-1.0 if (sb[j // 8] >> (j % 8)) & 1 else 1.0 for j in range(d)])
    H = np.array([[(-1) ** bin(i & j).count("1") for j in range(d)] for i in range(d)])
    assert np.abs(R - H * s[None, :] / math.sqrt(d)).max() < 1e-15
    x, q, k = rng.standard_normal((3, d))
    assert abs(np.linalg.norm(R @ x) - np.linalg.norm(x)) < 1e-12
    assert abs((R @ q) @ (R @ k) - q @ k) < 1e-12


# ----------------------------------------------------------------- codebooks


def _golden_levels():
    rows = {}
    with open(os.path.join(GOLDEN, "lloyd_max_gaussian.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                v = line.split()
                dec = len(v[1].split(".")[1])
                rows[int(v[0])] = (float(v[1]), [float(x) for x in v[2:]], 0.6 * 10.0 ** -dec)
    return rows


def test_lloyd_max_one_bit_closed_form():
    """b = 1: levels +-sqrt(2/pi), distortion 1 - 2/pi (exact)."""
    c, t, mse, _ = oracle.lloyd_max_unit(1)
    assert abs(c[1] - math.sqrt(2 / math.pi)) < 1e-12 and c[0] == -c[1]
    assert t[0] == 0.0
    assert abs(mse - (1 - 2 / math.pi)) < 1e-12


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_max_textbook_levels(bits):
    """Levels and distortion agree with the textbook Gaussian table."""
    mse_ref, lv, mse_tol = _golden_levels()[bits]
    c, _, mse, _ = oracle.lloyd_max_unit(bits)
    L = 1 << bits
    assert np.abs(c[L // 2:] - np.array(lv)).max() < 2e-4
    assert abs(mse - mse_ref) < mse_tol  # the table's last printed digit


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_optimality_conditions(bits):
    """Centroid condition by an independent adaptive quadrature (scipy), the
    midpoint condition, antisymmetry, and cell probabilities summing to 1."""
    c, t, mse, _ = oracle.lloyd_max_unit(bits)
    L = 1 << bits
    edges = [-np.inf] + list(t) + [np.inf]
    tot = 0.0
    dist = 0.0
    for k in range(L):
        a, b = edges[k], edges[k + 1]
        mass = stats.norm.cdf(b) - stats.norm.cdf(a)
        mom = stats.norm.pdf(a) - stats.norm.pdf(b)  # integral of z phi(z)
        assert abs(mom / mass - c[k]) < 1e-11
        tot += mass
        dist += integrate.quad(lambda z: (z - c[k]) ** 2 * stats.norm.pdf(z), a, b,
                               epsabs=1e-14, epsrel=1e-12)[0]
    assert abs(tot - 1.0) < 1e-14
    assert abs(dist - mse) < 1e-10
    assert np.allclose(t, 0.5 * (c[1:] + c[:-1]), rtol=0, atol=0)
    assert np.array_equal(c, -c[::-1])
    assert np.all(np.diff(c) > 0)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_distortion_within_stated_bound(bits):
    """Unit-variance distortion below the bound (sqrt(3) pi / 2) 4^-b that the
    tqai page's test suite states ("Test Suite", first item)."""
    _, _, mse, _ = oracle.lloyd_max_unit(bits)
    bound = math.sqrt(3) * math.pi / 2 * 4.0 ** (-bits)
    assert mse < bound
    # and the bound is not slack by an order of magnitude (it would be for a
    # wrong density or a dropped term)
    assert mse > 0.5 * bound


def test_codebook_scaling_with_dimension():
    """N(0, 1/d) codebook = unit codebook / sqrt(d)."""
    c1, t1, _, _ = oracle.lloyd_max_unit(4)
    c, t = oracle.codebook(128, 4)
    assert np.allclose(c * math.sqrt(128), c1, atol=1e-15)
    assert np.allclose(t * math.sqrt(128), t1, atol=1e-15)


# ---------------------------------------------------------------------- norm

_POS = np.arange(0, 0x7C00, dtype=np.uint16)
_QUANTA = [int(Fraction(float(v)) * (1 << 24)) for v in _POS.view(np.float16)]


def _norm16_exact(x16):
    """Independent exact RNE: binary search of 4 S among the squared sums of
    neighbouring fp16 values (all in units of 2^-24), Python integers."""
    S = 0
    for v in np.asarray(x16, np.uint16).view(np.float16):
        m = int(Fraction(float(v)) * (1 << 24))
        S += m * m
    S4 = 4 * S
    lo, hi = 0, len(_QUANTA) - 1
    # largest p with (A_{p-1} + A_p)^2 <= 4S (p = 0 if none)
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if (_QUANTA[mid - 1] + _QUANTA[mid]) ** 2 <= S4:
            lo = mid
        else:
            hi = mid - 1
    p = lo
    if p > 0 and (_QUANTA[p - 1] + _QUANTA[p]) ** 2 == S4 and p % 2 == 1:
        p -= 1  # exact midpoint: the even pattern wins
    if p == len(_QUANTA) - 1 and (2 * _QUANTA[p] + 2 ** 24 * 32) ** 2 <= S4:
        return 0x7C00
    return p


def test_norm_exact_random():
    """fp16 norm equals an independent exact computation on random vectors of
    the workload's distribution, including near-tie cases."""
    rng = np.random.default_rng(7)
    for trial in range(3000):
        d = [64, 128, 256][trial % 3]
        x = (rng.standard_normal(d) * math.exp(rng.standard_normal())).astype(np.float16)
        if trial % 5 == 0:
            x[rng.integers(0, d, 4)] *= 10
        xb = x.view(np.uint16)
        h, _ = oracle.norm16(xb)
        assert h == _norm16_exact(xb)


def test_norm_ties_and_special_cases():
    """Exact midpoints round to even; zero, single element, subnormals."""
    tie = np.array([1233, 1644], np.float16).view(np.uint16)  # 3-4-5: norm 2055
    assert oracle.norm16(tie)[0] == np.float16(2056).view(np.uint16)
    tie2 = np.array([1239, 1652], np.float16).view(np.uint16)  # norm 2065 -> 2064
    assert oracle.norm16(tie2)[0] == np.float16(2064).view(np.uint16)
    above = np.array([1233, 1644, 2 ** -24], np.float16).view(np.uint16)
    assert oracle.norm16(above)[0] == np.float16(2056).view(np.uint16)
    below = np.array([1239, 1652, 0.0], np.float16).view(np.uint16)
    assert oracle.norm16(below)[0] == np.float16(2064).view(np.uint16)
    assert oracle.norm16(np.zeros(128, np.uint16))[0] == 0
    for v in [1.5, -3.25, 6.1e-5, 2 ** -24, 65504.0]:
        x = np.zeros(64, np.float16)
        x[17] = v
        assert oracle.norm16(x.view(np.uint16))[0] == np.float16(abs(v)).view(np.uint16)
    big = np.full(4, 65504, np.float16).view(np.uint16)  # norm 131008 -> inf
    assert oracle.norm16(big)[0] == 0x7C00
    for trial in range(200):
        rng = np.random.default_rng(trial)
        x = (rng.standard_normal(128) * 1e-6).astype(np.float16).view(np.uint16)
        assert oracle.norm16(x)[0] == _norm16_exact(x)


# ------------------------------------------------------------------ quantize


def test_quantize_argmin_equals_threshold_count():
    """Scalar argmin (the oracle's rule) equals the count of thresholds below y
    outside the 1e-6 band; the band is the distance to the nearest threshold."""
    d, bits = 128, 4
    rng = np.random.default_rng(3)
    sb = _rand_signs(rng, d)
    x = rng.standard_normal((400, d)).astype(np.float16).view(np.uint16)
    codes, norms, band = oracle.encode(x, bits, sb)
    R = oracle.rotation(d, sb)
    c, t = oracle.codebook(d, bits)
    xf = x.view(np.float16).astype(np.float64)
    y = (xf @ R.T) / np.linalg.norm(xf, axis=1, keepdims=True)
    cnt = np.searchsorted(t, y, side="left")
    far = band > 1e-6
    assert np.array_equal(codes[far], cnt[far])
    assert np.allclose(band, np.abs(y[..., None] - t).min(-1), atol=1e-13)


def test_alternative_code_against_textbook_thresholds():
    """The alternative code (the neighbour across the nearest threshold) on a
    spike input x = e_j at d = 64: every rotated coordinate is +-1/8 exactly
    (R = H D / 8), so code, alternative and band follow from the thresholds
    of the textbook table (midpoints of its levels, scaled by 1/8)."""
    d = 64
    rng = np.random.default_rng(5)
    sb = _rand_signs(rng, d)
    x = np.zeros((1, d), np.float16)
    x[0, 9] = 1.0
    R = oracle.rotation(d, sb)
    sign = np.sign(R[:, 9])  # +-1/8 per coordinate: the sign is all that varies
    assert np.allclose(np.abs(R[:, 9]), 1 / 8, rtol=0, atol=0)
    for bits in (2, 3, 4):
        lv = _golden_levels()[bits][1]
        levels = np.r_[-np.array(lv[::-1]), np.array(lv)] / 8
        thr = (levels[1:] + levels[:-1]) / 2
        y = 1 / 8
        code_pos = int(np.argmin(np.abs(y - levels)))
        kt = int(np.argmin(np.abs(y - thr)))
        # the table's 4-decimal levels decide these with a wide margin
        dist = np.sort(np.abs(y - thr))
        assert dist[0] > 1e-4 and dist[1] - dist[0] > 1e-4
        alt_pos = kt + 1 if code_pos == kt else kt
        L = 1 << bits
        codes, _, band, alt = oracle.encode(x.view(np.uint16), bits, sb, want_alt=True)
        want_c = np.where(sign > 0, code_pos, L - 1 - code_pos)
        want_a = np.where(sign > 0, alt_pos, L - 1 - alt_pos)
        assert np.array_equal(codes[0], want_c), bits
        assert np.array_equal(alt[0], want_a), bits
        assert np.allclose(band[0], dist[0], rtol=0, atol=2e-5)
    # the hand values for 2 bits: y = 1/8 lies just above the threshold
    # 0.9816 / 8 = 0.1227, so the code is the top level and the alternative
    # the one below it
    codes, _, _, alt = oracle.encode(x.view(np.uint16), 2, sb, want_alt=True)
    assert set(zip(codes[0].tolist(), alt[0].tolist())) <= {(3, 2), (0, 1)}


def test_alternative_code_is_the_neighbour_across_the_nearest_threshold():
    """On random inputs: the alternative differs from the code by one level,
    and the threshold between them is the nearest one (its distance is the
    band)."""
    d = 128
    rng = np.random.default_rng(8)
    sb = _rand_signs(rng, d)
    x = rng.standard_normal((300, d)).astype(np.float16).view(np.uint16)
    R = oracle.rotation(d, sb)
    xf = x.view(np.float16).astype(np.float64)
    y = (xf @ R.T) / np.linalg.norm(xf, axis=1, keepdims=True)
    for bits in (2, 3, 4):
        codes, _, band, alt = oracle.encode(x, bits, sb, want_alt=True)
        _, t = oracle.codebook(d, bits)
        assert (np.abs(alt.astype(int) - codes.astype(int)) == 1).all()
        between = t[np.minimum(alt, codes)]
        assert np.allclose(np.abs(y - between), band, rtol=0, atol=1e-13)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_code_histogram_matches_gaussian_cells(bits):
    """After rotation each coordinate is ~N(0, 1/d): code frequencies match the
    Gaussian cell probabilities (chi-square, isotropic inputs)."""
    d = 128
    x = synth.iso_host(4242, bits, 1500, d)
    sb = synth.sign_bits(4242, 0, d)
    codes, _, _ = oracle.encode(x, bits, sb, want_band=False)
    _, t, _, _ = oracle.lloyd_max_unit(bits)
    edges = np.r_[-np.inf, t, np.inf]
    p = np.diff(stats.norm.cdf(edges))
    obs = np.bincount(codes.ravel(), minlength=1 << bits)
    chi2 = ((obs - p * obs.sum()) ** 2 / (p * obs.sum())).sum()
    assert stats.chi2.sf(chi2, (1 << bits) - 1) > 1e-4


def test_zero_vector_and_symmetry():
    """Zero vector: norm 0 and every code 2^(b-1) - 1 (y = 0 sits on the middle
    threshold; the tie goes to the smaller index).  Exact power-of-two scaling
    keeps the codes; negation mirrors them (antisymmetric codebook)."""
    d = 128
    rng = np.random.default_rng(11)
    sb = _rand_signs(rng, d)
    for bits in (2, 3, 4):
        codes, norms, _ = oracle.encode(np.zeros((2, d), np.uint16), bits, sb)
        assert np.all(codes == (1 << (bits - 1)) - 1) and np.all(norms == 0)
        x = rng.standard_normal((50, d)).astype(np.float16)
        c1, n1, b1 = oracle.encode(x.view(np.uint16), bits, sb)
        c2, n2, _ = oracle.encode((x * np.float16(4)).view(np.uint16), bits, sb)
        c3, n3, _ = oracle.encode((-x).view(np.uint16), bits, sb)
        assert np.array_equal(c1, c2)
        assert np.array_equal(n2.view(np.float16), n1.view(np.float16) * np.float16(4))
        far = b1 > 1e-9
        assert np.array_equal(c3[far], ((1 << bits) - 1 - c1)[far])
        assert np.array_equal(n3, n1)


# ------------------------------------------------------------------- packing


def test_bytes_per_token_worked_example():
    """The tqai page's worked example: FP16 K+V at head dim 128 is 512 B per
    token per KV head; K4/V2 with fp16 norms is 100 B.  Also the config
    table's average bits and memory saved."""
    f = _figures()
    d = 128
    rng = np.random.default_rng(0)
    k = oracle.pack_rows(rng.integers(0, 16, (1, d)), 4)
    v = oracle.pack_rows(rng.integers(0, 4, (1, d)), 2)
    per_token = k.nbytes + v.nbytes + 2 + 2
    assert 2 * d * 2 == f["bytes_per_token_fp16"]
    assert per_token == f["bytes_per_token_k4v2"]
    for kb, vb, name in ((4, 2, "k4v2"), (3, 2, "k3v2"), (4, 3, "k4v3")):
        assert (kb + vb) / 2 == f["avg_bits_" + name]
        codes_only = d * (kb + vb) / 8
        with_norms = codes_only + 4
        saved = 100 * (1 - with_norms / 512)
        saved_codes_only = 100 * (1 - codes_only / 512)
        # the table rounds; K4/V3's 78% matches the codes-only saving
        assert abs(saved - f["saved_pct_" + name]) < 1.0 or \
            abs(saved_codes_only - f["saved_pct_" + name]) < 1.0


def test_pack_rows_bit_positions():
    """LSB-first: code i occupies bits [b i, b i + b) of the row."""
    c = np.zeros((1, 64), np.uint8)
    c[0, 1] = 1
    assert oracle.pack_rows(c, 4)[0, 0] == 0x10
    c = np.zeros((1, 64), np.uint8)
    c[0, 2] = 7  # bits 6, 7, 8
    p = oracle.pack_rows(c, 3)[0]
    assert p[0] == 0xC0 and p[1] == 0x01 and p[2:].sum() == 0
    c = np.zeros((1, 64), np.uint8)
    c[0, 3] = 2  # 2-bit code at bits 6..7 -> 0b10 << 6
    assert oracle.pack_rows(c, 2)[0, 0] == 0x80


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_pack_round_trips(bits, d):
    rng = np.random.default_rng(bits * d)
    for n in (1, 7, 33):
        c = rng.integers(0, 1 << bits, (n, d), dtype=np.uint8)
        assert np.array_equal(oracle.unpack_rows(oracle.pack_rows(c, bits), d, bits), c)
    c = rng.integers(0, 1 << bits, (64, d), dtype=np.uint8)
    tiles = oracle.pack_vtiles(c, bits)
    assert tiles.shape == (2, 32 * d * bits // 8)
    assert np.array_equal(oracle.unpack_vtiles(tiles, d, bits), c)


def test_vtile_bit_positions():
    """Value tile: segment 16q + r holds coordinate r*(d/16)+m of token tok(q,u)
    at bit (8m + u) * b; check one hand-placed code."""
    d, bits = 128, 2
    c = np.zeros((32, d), np.uint8)
    # token 13 = 8*1 + 5 -> q = 1, u = 5; coordinate 3*8 + 2 -> r = 3, m = 2
    c[13, 26] = 3
    t = oracle.pack_vtiles(c, bits)[0]
    seg = d * bits // 16
    bit = (8 * 2 + 5) * bits
    nz = np.flatnonzero(t)
    assert list(nz) == [(16 * 1 + 3) * seg + bit // 8]
    assert t[nz[0]] == 3 << (bit % 8)


def test_vtile_fields_across_byte_boundaries():
    """3-bit fields straddle bytes, 4-bit fields fill nibbles: hand-placed codes
    land at the bytes the layout description gives (d = 128)."""
    d = 128
    # 3 bits: segments of 24 bytes
    c = np.zeros((32, d), np.uint8)
    # token 18 = 8*2 + 2 (q 2, u 2), coordinate 56 = 7*8 + 0 (r 7, m 0):
    # segment 39, bits 6..8 of it; code 0b101 -> bit 6 and bit 8
    c[18, 56] = 5
    # token 5 (q 0, u 5), coordinate 2*8 + 2 = 18 (r 2, m 2): segment 2, bits
    # (16 + 5) * 3 = 63..65; code 0b110 -> bits 64 and 65
    c[5, 18] = 6
    t = oracle.pack_vtiles(c, 3)[0]
    want = {39 * 24 + 0: 0x40, 39 * 24 + 1: 0x01, 2 * 24 + 8: 0x03}
    assert {int(i): int(t[i]) for i in np.flatnonzero(t)} == want
    assert np.array_equal(oracle.unpack_vtiles(t[None], d, 3), c)
    # 4 bits: segments of 32 bytes
    c = np.zeros((32, d), np.uint8)
    # token 27 = 8*3 + 3 (q 3, u 3), coordinate 1 (r 0, m 1): segment 48, bits
    # (8 + 3) * 4 = 44..47, the high nibble of byte 5; code 9
    c[27, 1] = 9
    # token 8 (q 1, u 0), coordinate 15*8 + 7 = 127 (r 15, m 7): segment 31,
    # bits 56 * 4 = 224..227, the low nibble of byte 28; code 14
    c[8, 127] = 14
    t = oracle.pack_vtiles(c, 4)[0]
    want = {48 * 32 + 5: 0x90, 31 * 32 + 28: 0x0E}
    assert {int(i): int(t[i]) for i in np.flatnonzero(t)} == want
    assert np.array_equal(oracle.unpack_vtiles(t[None], d, 4), c)


# ------------------------------------------------------------------ fidelity


def test_fidelity_matches_tqai_benchmark():
    """Synthetic accuracy figures of the tqai page ("The CLI"): 4-bit keys and
    2-bit values on isotropic Gaussian vectors, head dim 128.  NMSE within
    1.5%, cosine within 5e-4, SNR within 0.1 dB; SNR = -10 log10 NMSE and
    cos ~ sqrt(1 - NMSE) hold internally."""
    f = _figures()
    d = 128
    x = synth.iso_host(2024, 0, 6000, d)
    sb = synth.sign_bits(2024, 0, d)
    xf = x.view(np.float16).astype(np.float64)
    for bits, key in ((4, "keys4"), (2, "values2")):
        codes, norms, _ = oracle.encode(x, bits, sb, want_band=False)
        xh = oracle.dequant(codes, norms, bits, sb)
        nmse = ((xh - xf) ** 2).sum() / (xf ** 2).sum()
        snr = -10 * math.log10(nmse)
        cos = np.mean((xh * xf).sum(1) / np.linalg.norm(xh, axis=1) / np.linalg.norm(xf, axis=1))
        assert abs(nmse / f[key + "_nmse"] - 1) < 0.015, nmse
        assert abs(snr - f[key + "_snr_db"]) < 0.1
        assert abs(cos - f[key + "_cos"]) < 5e-4, cos
        assert abs(cos - math.sqrt(1 - nmse)) < 2e-3


# ----------------------------------------------------------------- attention


def test_attention_hand_example():
    """d = 4, T = 2: weights are a logistic function of the score gap."""
    q = np.array([[2.0, 0.0, 0.0, 0.0]])
    K = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]])
    V = np.array([[1.0, 2, 3, 4], [-1.0, 0, 1, 0]])
    # scores 2/2 = 1 and 0: p0 = e/(e+1)
    p0 = math.e / (math.e + 1)
    out = oracle.attention(q, K, V)
    assert np.allclose(out[0], p0 * V[0] + (1 - p0) * V[1], atol=1e-15)


def test_attention_special_cases():
    rng = np.random.default_rng(5)
    d, T = 64, 37
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    q = rng.standard_normal((3, d))
    # one token: the output is that value
    assert np.allclose(oracle.attention(q, K[:1], V[:1]), np.repeat(V[:1], 3, 0), atol=1e-15)
    # zero query or identical keys: uniform weights, output = mean value
    assert np.allclose(oracle.attention(np.zeros((1, d)), K, V)[0], V.mean(0), atol=1e-14)
    assert np.allclose(oracle.attention(q, np.repeat(K[:1], T, 0), V), np.repeat(V.mean(0)[None], 3, 0),
                       atol=1e-14)
    # token order does not matter
    perm = rng.permutation(T)
    assert np.allclose(oracle.attention(q, K, V), oracle.attention(q, K[perm], V[perm]), atol=1e-14)
    # no tokens: zeros
    assert np.array_equal(oracle.attention(q, K[:0], V[:0]), np.zeros((3, d)))


def test_sparse_v_hand_example():
    """Scores 0, -1, -20 (d = 2): with eps = 1e-6 the third position (relative
    weight e^-20 ~ 2e-9) leaves the value sum but stays in the denominator;
    the bound is its weighted |V|."""
    r2 = math.sqrt(2.0)
    q = np.array([[r2, 0.0]])
    K = np.array([[0.0, 1.0], [-1.0, 3.0], [-20.0, -2.0]])  # q.k / sqrt 2 = first coordinate
    V = np.array([[1.0, 0.0], [0.0, 1.0], [5.0, -7.0]])
    l = 1 + math.exp(-1) + math.exp(-20)
    out, bound, w = oracle.attention_sparse(q, K, V, 1e-6, want_weights=True)
    assert np.allclose(w[0], [1.0, math.exp(-1), math.exp(-20)], rtol=1e-14, atol=0)
    assert np.allclose(out[0], [1 / l, math.exp(-1) / l], rtol=1e-14, atol=0)
    assert np.allclose(bound[0], [5 * math.exp(-20) / l, 7 * math.exp(-20) / l], rtol=1e-14, atol=0)
    # a threshold between e^-20 and e^-1 gives the same; above e^-1 the
    # second position leaves too
    out2, _ = oracle.attention_sparse(q, K, V, 0.3)
    assert np.allclose(out2[0], out[0], rtol=1e-14, atol=0)
    out3, b3 = oracle.attention_sparse(q, K, V, 0.5)
    assert np.allclose(out3[0], [1 / l, 0.0], rtol=1e-14, atol=1e-300)
    assert np.allclose(b3[0], [5 * math.exp(-20) / l, (math.exp(-1) + 7 * math.exp(-20)) / l],
                       rtol=1e-14, atol=0)


def test_sparse_v_special_cases():
    rng = np.random.default_rng(15)
    d, T = 64, 53
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    q = rng.standard_normal((3, d)) * 4
    dense = oracle.attention(q, K, V)
    # eps <= 0 keeps every position: plain attention, zero bound
    for eps in (0.0, -1.0):
        o, b = oracle.attention_sparse(q, K, V, eps)
        assert np.allclose(o, dense, rtol=0, atol=1e-15) and not b.any()
    # eps = 1 keeps only the maximum (both of a tie): output = V_max / l
    s = q @ K.T / math.sqrt(d)
    o, b = oracle.attention_sparse(q, K, V, 1.0)
    for g in range(3):
        j = int(np.argmax(s[g]))
        l = np.exp(s[g] - s[g, j]).sum()
        assert np.allclose(o[g], V[j] / l, rtol=1e-12, atol=0)
    K2 = np.vstack([K, K[:1]])
    V2 = np.vstack([V, V[5:6]])
    qt = K[:1] * 3  # position 0 and its copy hold the maximum
    o, _ = oracle.attention_sparse(qt, K2, V2, 1.0)
    st = qt @ K2.T / math.sqrt(d)
    l = np.exp(st[0] - st[0].max()).sum()
    assert np.allclose(o[0], (V[0] + V[5]) / l, rtol=1e-12, atol=0)
    # eps above 1 leaves everything out
    o, b = oracle.attention_sparse(q, K, V, 1.5)
    assert not o.any()
    # the bound holds for the dense result, and dense - sparse is exactly the
    # left-out part: |dense - sparse| <= bound, with equality where the
    # left-out values share a sign
    for eps in (1e-3, 1e-2, 0.1):
        o, b = oracle.attention_sparse(q, K, V, eps)
        assert (np.abs(dense - o) <= b + 1e-15).all()
    Vp = np.abs(V)
    o, b = oracle.attention_sparse(q, K, Vp, 1e-2)
    assert np.allclose(oracle.attention(q, K, Vp) - o, b, rtol=1e-12, atol=1e-16)
    # no positions: zeros
    o, b = oracle.attention_sparse(q, K[:0], V[:0], 1e-6)
    assert not o.any() and not b.any()


def test_attention_keep_hand_example_and_reductions():
    """Attention with an explicit left-out set: the hand example of the sparse
    pin with its second position left out, then keep-all equal to plain
    attention and the eps rule's set equal to the sparse reading."""
    r2 = math.sqrt(2.0)
    q = np.array([[r2, 0.0]])
    K = np.array([[0.0, 1.0], [-1.0, 3.0], [-20.0, -2.0]])
    V = np.array([[1.0, 0.0], [0.0, 1.0], [5.0, -7.0]])
    l = 1 + math.exp(-1) + math.exp(-20)
    out, w = oracle.attention_keep(q, K, V, [1, 0, 1], want_weights=True)
    assert np.allclose(w[0], [1.0, math.exp(-1), math.exp(-20)], rtol=1e-14, atol=0)
    assert np.allclose(out[0], [(1 + 5 * math.exp(-20)) / l, -7 * math.exp(-20) / l],
                       rtol=1e-14, atol=0)
    rng = np.random.default_rng(16)
    d, T = 64, 70
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    q = rng.standard_normal((1, d)) * 4
    assert np.allclose(oracle.attention_keep(q, K, V, np.ones(T)), oracle.attention(q, K, V),
                       rtol=0, atol=1e-15)
    for eps in (1e-3, 0.05):
        o, _, w = oracle.attention_sparse(q, K, V, eps, want_weights=True)
        assert np.allclose(oracle.attention_keep(q, K, V, w[0] >= eps), o, rtol=0, atol=1e-15)
    assert not oracle.attention_keep(q, K, V, np.zeros(T)).any()
    assert not oracle.attention_keep(q, K[:0], V[:0], np.zeros(0)).any()


def test_qjl_hand_examples():
    """d = m = 2: S r = (-1, 4) gives bits (0, 1) and gamma = sqrt 5; with
    R = I, levels (-1/2, 1/2), codes (0, 1), n16 = 2 and q = (3, 1) the
    estimate is 2 (-1 + sqrt(pi/2) / 2 * sqrt 5 * <S q, z>), <S q, z> = -4 + 5."""
    S = np.array([[1.0, 1.0], [2.0, -1.0]])
    bits, gamma, proj = oracle.qjl_project(np.array([1.0, -2.0]), S)
    assert bits.tolist() == [2] and abs(gamma - math.sqrt(5)) < 1e-15
    assert proj.tolist() == [-1.0, 4.0]
    # a zero projection counts as non-negative
    bits0, _, _ = oracle.qjl_project(np.array([1.0, -1.0]), np.array([[1.0, 1.0], [0.0, 1.0]]))
    assert bits0.tolist() == [1]
    est = oracle.qjl_estimate(np.array([3.0, 1.0]), np.array([[0, 1]]), np.array([2.0]),
                              np.array([math.sqrt(5)]), np.array([[2]]), S, np.eye(2),
                              np.array([-0.5, 0.5]))
    want = 2 * (-1 + math.sqrt(math.pi / 2) / 2 * math.sqrt(5) * 1.0)
    assert abs(est[0] - want) < 1e-14


def test_qjl_term_unbiased():
    """Over draws of S (i.i.d. N(0,1), m = d = 64) the QJL term
    sqrt(pi/2)/m gamma <S u, z> averages to <u, r>; a wrong constant or sign
    convention moves the mean by many standard errors."""
    rng = np.random.default_rng(21)
    d = 64
    r = rng.standard_normal(d) * 0.05
    u = r / np.linalg.norm(r) * 10 + rng.standard_normal(d)
    est = []
    for _ in range(3000):
        S = rng.standard_normal((d, d))
        bits, gamma, _ = oracle.qjl_project(r, S)
        z = np.where((bits[np.arange(d) // 8] >> (np.arange(d) % 8)) & 1, 1.0, -1.0)
        est.append(math.sqrt(math.pi / 2) / d * gamma * float((S @ u) @ z))
    est = np.array(est)
    se = est.std() / math.sqrt(len(est))
    assert abs(est.mean() - u @ r) < 5 * se, (est.mean(), u @ r, se)
    assert abs(u @ r) > 20 * se  # the test can see a constant off by a few percent


def test_qjl_estimate_unbiased_on_encoded_keys():
    """The whole estimate (stage 1 plus the QJL term) of <q, x> for encoded
    fp16 keys averages, over draws of S, to <q, x> n16 / ||x|| (the stored
    norm against the exact one), while stage 1 alone stays biased."""
    rng = np.random.default_rng(22)
    d = 64
    sb = _rand_signs(rng, d)
    x = (rng.standard_normal((3, d)) * 2).astype(np.float16).view(np.uint16)
    xf = x.view(np.float16).astype(np.float64)
    q = xf[0] * 0.7 + rng.standard_normal(d)
    R = oracle.rotation(d, sb)
    c, _ = oracle.codebook(d, 2)
    draws = []
    for _ in range(400):
        S = rng.standard_normal((d, d))
        codes, norms, signs, gamma, _ = oracle.qjl_encode(x, 2, sb, S)
        n16 = oracle.halves_to_double(norms)
        g16 = np.float16(gamma).astype(np.float64)
        draws.append(oracle.qjl_estimate(q, codes, n16, g16, signs, S, R, c))
    draws = np.array(draws)
    exact = xf @ q * n16 / np.linalg.norm(xf, axis=1)
    mean, se = draws.mean(0), draws.std(0) / math.sqrt(len(draws))
    assert np.all(np.abs(mean - exact) < 5 * se + 1e-3 * np.abs(exact)), (mean, exact, se)
    stage1 = n16 * ((R @ q) @ c[codes].T)
    assert np.abs(stage1 - exact).max() > 10 * se.max()


def test_rotated_domain_evaluation_matches_plain():
    """Attention evaluated in the rotated domain (scores (Rq).c, values summed
    as levels, one R^T at the end) equals the oracle's plain evaluation over
    the dequantized cache."""
    d, T = 128, 300
    rng = np.random.default_rng(9)
    sb = _rand_signs(rng, d)
    k = (rng.standard_normal((T, d)) * 3).astype(np.float16).view(np.uint16)
    v = rng.standard_normal((T, d)).astype(np.float16).view(np.uint16)
    q = rng.standard_normal((4, d))
    kc, kn, _ = oracle.encode(k, 4, sb, want_band=False)
    vc, vn, _ = oracle.encode(v, 2, sb, want_band=False)
    plain = oracle.attention(q, oracle.dequant(kc, kn, 4, sb), oracle.dequant(vc, vn, 2, sb))
    R = oracle.rotation(d, sb)
    ck, _ = oracle.codebook(d, 4)
    cv, _ = oracle.codebook(d, 2)
    knf = kn.view(np.float16).astype(np.float64)
    vnf = vn.view(np.float16).astype(np.float64)
    s = ((q @ R.T) @ ck[kc].T) * knf[None] / math.sqrt(d)
    p = np.exp(s - s.max(1, keepdims=True))
    acc = (p * vnf[None]) @ cv[vc]
    rot = (acc @ R) / p.sum(1, keepdims=True)
    assert np.abs(rot - plain).max() < 1e-12


# ------------------------------------------------------------------ generator


def test_generator_determinism_and_shape():
    a = synth.kv_host(1001, 0, 3, 1, 2, 128, 100, 5)
    b = synth.kv_host(1001, 0, 3, 1, 2, 128, 100, 5)
    c = synth.kv_host(1001, 0, 3, 1, 2, 128, 98, 7)
    assert np.array_equal(a, b) and np.array_equal(a, c[2:])
    assert not np.array_equal(a, synth.kv_host(1001, 1, 3, 1, 2, 128, 100, 5))


def test_generator_distribution():
    """N(0,1) moments, 4 distinct outlier channels x10, lognormal(0, 0.5)
    per-token scale, balanced sign bits."""
    z = synth.normals_host(99, 0, 400000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert abs((z ** 4).mean() - 3) < 0.05
    d = 128
    o = synth.outliers(1002, 0, 5, 3, d)
    assert len(set(o.tolist())) == 4 and o.min() >= 0 and o.max() < d
    x = synth.kv_host(1002, 0, 5, 0, 3, d, 0, 4000).view(np.float16).astype(np.float64)
    rms = np.sqrt((x ** 2).mean(0))
    mask = np.zeros(d, bool)
    mask[o] = True
    ratio = rms[mask].mean() / rms[~mask].mean()
    assert 8.5 < ratio < 11.5
    # token scale: log of the per-token rms of the normal channels ~ N(0, 0.5^2)
    ls = np.log(np.sqrt((x[:, ~mask] ** 2).mean(1)))
    assert abs(ls.std() - 0.5) < 0.03
    bits = np.unpackbits(synth.sign_bits(1002, 0, 4096)[None], axis=1)
    assert abs(bits.mean() - 0.5) < 0.03
