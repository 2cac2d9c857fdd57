"""GPU parity of the QJL stage (tq_qjl_encode, tq_qjl_scores) against the
oracle ("We Built ...", "Why not both stages?"): the residual sketch (sign
bits of S r, gamma = ||r||) and the inner-product estimate.

S is the caller's draw (fp16 N(0,1) entries), passed to both sides.  Keys
whose stage-1 codes differ between the two sides (a coordinate within 1e-6
of a decision threshold, where either code is correct) are left out of the
sketch comparisons and counted; projections within a relative 1e-4 of zero
may take either sign (fp32 against fp64 residuals)."""
import ctypes
import math

import numpy as np
import pytest

import kv_cache_quantization_tq_amd as tq
import oracle
import synth
from helpers import require_gpu

pytestmark = pytest.mark.gpu
SEED = 1004


def _draw_S(rng, d):
    return rng.standard_normal((d, d)).astype(np.float16)


@pytest.mark.parametrize("d,bits,n,G", [(128, 4, 300, 4), (64, 2, 77, 4), (256, 3, 130, 4),
                                        (128, 3, 1000, 4), (64, 3, 45, 8), (256, 4, 64, 1),
                                        (128, 2, 33, 8), (64, 4, 200, 2)])
def test_qjl_parity(d, bits, n, G):
    """Sketch and estimate against the oracle: every head dim and bit width,
    1 to 8 queries, key counts with and without a whole number of 4-key rows
    and 16-key tiles."""
    torch = require_gpu()
    rng = np.random.default_rng(d * 10 + bits)
    x16 = synth.kv_host(SEED, 0, 0, 0, 0, d, 0, n)
    sb = synth.sign_bits(SEED, 0, d)
    S16 = _draw_S(rng, d)
    cb = tq.Codebook(d, bits)
    xd = torch.from_numpy(x16.view(np.int16)).cuda()
    sbd = torch.from_numpy(sb).cuda()
    Sd = torch.from_numpy(S16.view(np.int16)).cuda()
    codes = torch.empty((n, d * bits // 8), dtype=torch.uint8, device="cuda")
    norms = torch.empty(n, dtype=torch.int16, device="cuda")
    signs = torch.empty((n, d // 8), dtype=torch.uint8, device="cuda")
    gamma = torch.empty(n, dtype=torch.int16, device="cuda")
    tq.encode(cb, xd, sbd, codes, norms)
    tq.qjl_encode(cb, xd, sbd, Sd, codes, signs, gamma)
    q16 = np.stack([synth.q_host(SEED, 0, 0, 0, g, d) for g in range(G)])
    qd = torch.from_numpy(q16.view(np.int16)).cuda()
    out = torch.empty((G, n), dtype=torch.float32, device="cuda")
    tq.qjl_scores(cb, qd, sbd, Sd, codes, norms, signs, gamma, out)
    torch.cuda.synchronize()

    S64 = S16.astype(np.float64)
    oc, on, osg, og, proj = oracle.qjl_encode(x16, bits, sb, S64)
    gc = oracle.unpack_rows(codes.cpu().numpy(), d, bits)
    same = np.all(gc == oc, axis=1) & (norms.cpu().numpy().view(np.uint16) == on)
    excluded = int((~same).sum())
    print(f"QJL d={d} b={bits} n={n}: {excluded} keys with a band code left out", flush=True)
    assert excluded <= max(2, n // 50)
    # gamma: fp16 of the residual norm, within one fp16 rounding
    gg = gamma.cpu().numpy().view(np.float16).astype(np.float64)
    assert np.all(np.abs(gg[same] - og[same]) <= 2.0 ** -10 * og[same] + 1e-7)
    # signs: bit-exact away from zero projections
    gbits = np.unpackbits(signs.cpu().numpy(), axis=1, bitorder="little").astype(bool)
    obits = np.unpackbits(osg, axis=1, bitorder="little").astype(bool)
    rown = np.linalg.norm(S64, axis=1)
    near = np.abs(proj) < 1e-4 * rown[None, :] * og[:, None]
    bad = (gbits != obits) & ~near & same[:, None]
    assert not bad.any(), np.argwhere(bad)[:5]
    # estimates: against the oracle's estimate from its own sketch
    R = oracle.rotation(d, sb)
    c, _ = oracle.codebook(d, bits)
    n16 = oracle.halves_to_double(on)
    g16 = np.float16(og).astype(np.float64)
    got = out.cpu().numpy()
    for g in range(G):
        q64 = oracle.halves_to_double(q16[g])
        want = oracle.qjl_estimate(q64, oc, n16, g16, osg, S64, R, c)
        rq = R @ q64
        qjl_scale = n16 * math.sqrt(math.pi / 2) / d * g16 * np.abs(S64 @ rq).sum()
        scale = n16 * (np.abs(rq) @ np.abs(c[oc]).T) + qjl_scale
        err = np.abs(got[g] - want)
        # fp32 sums, plus one fp16 rounding of gamma either way
        assert np.all(err[same] <= 1e-5 * scale[same] + 2.0 ** -10 * qjl_scale[same]), (
            err[same].max(), scale[same].max())


def test_qjl_large_sampled():
    """655,360 keys (8 heads x 81,920 tokens, d 128, 4 bits): more than one
    grid-stride pass of both kernels; sampled keys (including the last ones)
    against the oracle."""
    torch = require_gpu()
    d, bits, H, T = 128, 4, 8, 81920
    n = H * T
    rng = np.random.default_rng(5)
    S16 = _draw_S(rng, d)
    sb = synth.sign_bits(SEED, 0, d)
    cb = tq.Codebook(d, bits)
    x = torch.empty((1, H, T, d), dtype=torch.int16, device="cuda")
    synth.kv_dev(SEED, 0, 0, x)
    xd = x.view(n, d)
    sbd = torch.from_numpy(sb).cuda()
    Sd = torch.from_numpy(S16.view(np.int16)).cuda()
    codes = torch.empty((n, d * bits // 8), dtype=torch.uint8, device="cuda")
    norms = torch.empty(n, dtype=torch.int16, device="cuda")
    signs = torch.empty((n, d // 8), dtype=torch.uint8, device="cuda")
    gamma = torch.empty(n, dtype=torch.int16, device="cuda")
    tq.encode(cb, xd, sbd, codes, norms)
    tq.qjl_encode(cb, xd, sbd, Sd, codes, signs, gamma)
    G = 3
    q16 = np.stack([synth.q_host(SEED, 0, 0, 0, g, d) for g in range(G)])
    out = torch.empty((G, n), dtype=torch.float32, device="cuda")
    tq.qjl_scores(cb, torch.from_numpy(q16.view(np.int16)).cuda(), sbd, Sd, codes, norms, signs,
                  gamma, out)
    torch.cuda.synchronize()
    picks = np.unique(np.concatenate([rng.integers(0, n, 120), np.arange(n - 40, n)]))
    x16 = np.stack([synth.kv_host(SEED, 0, 0, 0, int(k // T), d, int(k % T), 1)[0] for k in picks])
    S64 = S16.astype(np.float64)
    oc, on, osg, og, proj = oracle.qjl_encode(x16, bits, sb, S64)
    gc = oracle.unpack_rows(codes[picks].cpu().numpy(), d, bits)
    same = np.all(gc == oc, axis=1) & (norms[picks].cpu().numpy().view(np.uint16) == on)
    assert (~same).sum() <= 2
    gg = gamma[picks].cpu().numpy().view(np.float16).astype(np.float64)
    assert np.all(np.abs(gg[same] - og[same]) <= 2.0 ** -10 * og[same] + 1e-7)
    gbits = np.unpackbits(signs[picks].cpu().numpy(), axis=1, bitorder="little").astype(bool)
    obits = np.unpackbits(osg, axis=1, bitorder="little").astype(bool)
    near = np.abs(proj) < 1e-4 * np.linalg.norm(S64, axis=1)[None, :] * og[:, None]
    assert not ((gbits != obits) & ~near & same[:, None]).any()
    R = oracle.rotation(d, sb)
    c, _ = oracle.codebook(d, bits)
    n16 = oracle.halves_to_double(on)
    g16 = np.float16(og).astype(np.float64)
    got = out[:, picks].cpu().numpy()
    for g in range(G):
        q64 = oracle.halves_to_double(q16[g])
        want = oracle.qjl_estimate(q64, oc, n16, g16, osg, S64, R, c)
        rq = R @ q64
        qjl_scale = n16 * math.sqrt(math.pi / 2) / d * g16 * np.abs(S64 @ rq).sum()
        scale = n16 * (np.abs(rq) @ np.abs(c[oc]).T) + qjl_scale
        err = np.abs(got[g] - want)
        assert np.all(err[same] <= 1e-5 * scale[same] + 2.0 ** -10 * qjl_scale[same])


def test_qjl_encode_alignment_checks():
    """Misaligned codes (the kernel reads them as aligned words), x or S are
    rejected on the host, before any device work; signs aligned to 4 but not
    16 bytes take the per-word store path and match the aligned result."""
    torch = require_gpu()
    d, bits, n = 128, 4, 40
    L = tq.lib()
    vp = ctypes.c_void_p
    cb = tq.Codebook(d, bits)
    x = torch.empty((1, 1, n, d), dtype=torch.int16, device="cuda")
    synth.kv_dev(SEED, 0, 0, x)
    x = x.view(n, d)
    sbd = torch.from_numpy(synth.sign_bits(SEED, 0, d)).cuda()
    Sd = torch.from_numpy(_draw_S(np.random.default_rng(3), d).view(np.int16)).cuda()
    codes = torch.empty((n + 1) * d * bits // 8, dtype=torch.uint8, device="cuda")
    norms = torch.empty(n, dtype=torch.int16, device="cuda")
    tq.encode(cb, x, sbd, codes[: n * d * bits // 8].view(n, -1), norms)
    signs = torch.zeros(n * d // 8 + 16, dtype=torch.uint8, device="cuda")
    gamma = torch.empty(n, dtype=torch.int16, device="cuda")

    def call(xp, Sp, cp, sp):
        return L.tq_qjl_encode(cb.handle, vp(xp), n, d, vp(sbd.data_ptr()), vp(Sp), vp(cp),
                               vp(sp), vp(gamma.data_ptr()), None)

    base = (x.data_ptr(), Sd.data_ptr(), codes.data_ptr(), signs.data_ptr())
    assert call(base[0], base[1], base[2] + 4, base[3]) == 1
    assert call(base[0] + 8, base[1], base[2], base[3]) == 1
    assert call(base[0], base[1] + 8, base[2], base[3]) == 1
    assert call(*base) == 0
    torch.cuda.synchronize()
    want = signs[: n * d // 8].clone()
    assert call(base[0], base[1], base[2], base[3] + 4) == 0
    torch.cuda.synchronize()
    assert torch.equal(signs[4: 4 + n * d // 8], want)
