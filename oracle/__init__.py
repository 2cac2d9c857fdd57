"""CPU oracle for the KV-cache codec and compressed-cache decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package; the library and its
Python binding never do.  It shares no code with the GPU path: the arithmetic
lives in ``tq_oracle.c`` (plain loops, fp64), this module only marshals numpy
arrays.

Every function is pinned by ``tests/test_oracle_pins.py`` against facts that do
not come from the oracle itself (closed forms, textbook values, the pages'
worked byte count and fidelity figures, brute force on tiny inputs).
"""
import ctypes
import functools
import math
import os

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_lib = None


def _L():
    global _lib
    if _lib is None:
        path = os.path.join(_DIR, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError("oracle/liboracle.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_half_to_double.restype = dbl
        lib.orc_hadamard.argtypes = [i32, vp]
        lib.orc_rotation.argtypes = [i32, vp, vp]
        lib.orc_lloyd_max.argtypes = [i32, vp, vp, vp]
        lib.orc_lloyd_max.restype = i32
        lib.orc_norm16.argtypes = [vp, i32, vp]
        lib.orc_norm16.restype = ctypes.c_uint16
        lib.orc_encode.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp, vp, vp]
        lib.orc_pack_rows.argtypes = [vp, i64, i32, i32, vp]
        lib.orc_unpack_rows.argtypes = [vp, i64, i32, i32, vp]
        lib.orc_pack_vtile.argtypes = [vp, i32, i32, vp]
        lib.orc_unpack_vtile.argtypes = [vp, i32, i32, vp]
        lib.orc_dequant.argtypes = [vp, vp, i64, i32, vp, vp, vp]
        lib.orc_attention.argtypes = [vp, i32, vp, vp, i64, i32, vp]
        lib.orc_attention_sparse.argtypes = [vp, i32, vp, vp, i64, i32, dbl, vp, vp, vp]
        lib.orc_attention_keep.argtypes = [vp, i32, vp, vp, i64, i32, vp, vp, vp]
        lib.orc_qjl_project.argtypes = [vp, i32, vp, i32, vp, vp, vp]
        lib.orc_qjl_encode.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp]
        lib.orc_qjl_estimate.argtypes = [vp, i32, vp, vp, vp, dbl, dbl, vp, vp, i32]
        lib.orc_qjl_estimate.restype = dbl
        _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def half_to_double(h):
    return _L().orc_half_to_double(int(h))


def hadamard(d):
    """Sylvester Hadamard matrix H_d (float64, entries +-1)."""
    H = np.zeros((d, d), dtype=np.float64)
    _L().orc_hadamard(d, _p(H))
    return H


def rotation(d, sign_bits):
    """R = H D / sqrt(d) for the layer's sign bits (d/8 bytes, LSB-first)."""
    sb = _c(sign_bits, np.uint8)
    assert sb.size == d // 8
    R = np.zeros((d, d), dtype=np.float64)
    _L().orc_rotation(d, _p(sb), _p(R))
    return R


@functools.lru_cache(maxsize=None)
def lloyd_max_unit(bits):
    """Lloyd-Max levels, thresholds and distortion for N(0,1), 2^bits levels."""
    L = 1 << bits
    c = np.zeros(L)
    t = np.zeros(max(L - 1, 1))
    mse = np.zeros(1)
    it = _L().orc_lloyd_max(bits, _p(c), _p(t), _p(mse))
    c.setflags(write=False)
    t.setflags(write=False)
    return c, t[: L - 1], float(mse[0]), it


def codebook(d, bits):
    """Levels and thresholds for N(0, 1/d): the unit codebook over sqrt(d)."""
    c, t, _, _ = lloyd_max_unit(bits)
    return c / math.sqrt(d), t / math.sqrt(d)


def norm16(x):
    """fp16 bits of the correctly rounded norm of one fp16 vector (uint16 bits)."""
    xb = _c(x, np.uint16)
    ex = np.zeros(1)
    h = _L().orc_norm16(_p(xb), xb.size, _p(ex))
    return h, float(ex[0])


def encode(x, bits, sign_bits, want_band=True, want_alt=False):
    """Encode fp16 vectors x[n][d] (uint16 bits).

    Returns (codes uint8 [n][d] unpacked, norms uint16 [n], band float64 [n][d])
    and, with want_alt, the alternative codes uint8 [n][d] as a fourth item:
    per coordinate, the code across its nearest threshold (tq_oracle.c,
    orc_encode)."""
    xb = _c(x, np.uint16)
    n, d = xb.shape
    R = rotation(d, sign_bits)
    c, t = codebook(d, bits)
    codes = np.zeros((n, d), dtype=np.uint8)
    norms = np.zeros(n, dtype=np.uint16)
    band = np.zeros((n, d)) if want_band else None
    alt = np.zeros((n, d), dtype=np.uint8) if want_alt else None
    _L().orc_encode(_p(xb), n, d, bits, _p(R), _p(_c(c, np.float64)), _p(_c(t, np.float64)),
                    _p(codes), _p(norms), _p(band) if want_band else None,
                    _p(alt) if want_alt else None)
    if want_alt:
        return codes, norms, band, alt
    return codes, norms, band


def pack_rows(codes, bits):
    cb = _c(codes, np.uint8)
    n, d = cb.shape
    out = np.zeros((n, d * bits // 8), dtype=np.uint8)
    _L().orc_pack_rows(_p(cb), n, d, bits, _p(out))
    return out


def unpack_rows(packed, d, bits):
    pb = _c(packed, np.uint8)
    n = pb.shape[0]
    out = np.zeros((n, d), dtype=np.uint8)
    _L().orc_unpack_rows(_p(pb), n, d, bits, _p(out))
    return out


def pack_vtiles(codes, bits):
    """codes [T][d] (T a multiple of 32) -> value tiles [T/32][32*d*bits/8]."""
    cb = _c(codes, np.uint8)
    T, d = cb.shape
    assert T % 32 == 0
    out = np.zeros((T // 32, 32 * d * bits // 8), dtype=np.uint8)
    for k in range(T // 32):
        tile = np.ascontiguousarray(cb[32 * k: 32 * k + 32])
        row = np.zeros(32 * d * bits // 8, dtype=np.uint8)
        _L().orc_pack_vtile(_p(tile), d, bits, _p(row))
        out[k] = row
    return out


def unpack_vtiles(tiles, d, bits):
    tb = _c(tiles, np.uint8)
    nt = tb.shape[0]
    out = np.zeros((nt * 32, d), dtype=np.uint8)
    for k in range(nt):
        row = np.ascontiguousarray(tb[k])
        cod = np.zeros((32, d), dtype=np.uint8)
        _L().orc_unpack_vtile(_p(row), d, bits, _p(cod))
        out[32 * k: 32 * k + 32] = cod
    return out


def dequant(codes, norms, bits, sign_bits):
    """x_hat[n][d] = n16 * R^T c[codes] in the original domain (float64)."""
    cb = _c(codes, np.uint8)
    n, d = cb.shape
    R = rotation(d, sign_bits)
    c, _ = codebook(d, bits)
    out = np.zeros((n, d))
    _L().orc_dequant(_p(cb), _p(_c(norms, np.uint16)), n, d, _p(R), _p(_c(c, np.float64)),
                     _p(out))
    return out


def attention(q, K, V):
    """softmax(q K^T / sqrt d) V for q[G][d], K[T][d], V[T][d] (float64)."""
    qb = _c(q, np.float64)
    G, d = qb.shape
    Kb = _c(K, np.float64)
    Vb = _c(V, np.float64)
    T = Kb.shape[0]
    out = np.zeros((G, d))
    _L().orc_attention(_p(qb), G, _p(Kb), _p(Vb), T, d, _p(out))
    return out


def attention_sparse(q, K, V, eps, want_weights=False):
    """Attention with the Sparse V gate (tq_oracle.c, orc_attention_sparse):
    positions whose weight exp(s_j - max s) is below eps are left out of the
    value sum, the denominator keeps them.  Returns (out[G][d], bound[G][d])
    and, with want_weights, the relative weights [G][T] as well."""
    qb = _c(q, np.float64)
    G, d = qb.shape
    Kb = _c(K, np.float64)
    Vb = _c(V, np.float64)
    T = Kb.shape[0]
    out = np.zeros((G, d))
    bound = np.zeros((G, d))
    w = np.zeros((G, max(T, 1))) if want_weights else None
    _L().orc_attention_sparse(_p(qb), G, _p(Kb), _p(Vb), T, d, float(eps), _p(out), _p(bound),
                              _p(w) if want_weights else None)
    if want_weights:
        return out, bound, w[:, :T]
    return out, bound


def attention_keep(q, K, V, keep, want_weights=False):
    """Attention whose value sum leaves out the positions with keep[j] == 0
    (the denominator keeps them): out[G][d] (tq_oracle.c,
    orc_attention_keep); with want_weights also exp(s_j - max s) [G][T]."""
    qb = _c(q, np.float64)
    G, d = qb.shape
    Kb = _c(K, np.float64)
    Vb = _c(V, np.float64)
    T = Kb.shape[0]
    kb = _c(np.asarray(keep, dtype=bool).astype(np.uint8), np.uint8)
    assert kb.shape == (T,)
    out = np.zeros((G, d))
    w = np.zeros((G, max(T, 1))) if want_weights else None
    _L().orc_attention_keep(_p(qb), G, _p(Kb), _p(Vb), T, d, _p(kb), _p(out),
                            _p(w) if want_weights else None)
    if want_weights:
        return out, w[:, :T]
    return out


def qjl_project(r, S):
    """Signs of S r as m bits (uint8 [m/8], LSB first), gamma = ||r||, and S r
    (tq_oracle.c, orc_qjl_project)."""
    rb = _c(r, np.float64)
    Sb = _c(S, np.float64)
    m, d = Sb.shape
    bits = np.zeros((m + 7) // 8, dtype=np.uint8)
    gamma = np.zeros(1)
    proj = np.zeros(m)
    _L().orc_qjl_project(_p(rb), d, _p(Sb), m, _p(bits), _p(gamma), _p(proj))
    return bits, float(gamma[0]), proj


def qjl_encode(x, bits, sign_bits, S):
    """Stage 1 and the QJL sketch of fp16 vectors x[n][d] with the m x d
    matrix S: (codes [n][d], norms uint16 [n], signs uint8 [n][m/8],
    gamma float64 [n], projections float64 [n][m])."""
    xb = _c(x, np.uint16)
    n, d = xb.shape
    Sb = _c(S, np.float64)
    m = Sb.shape[0]
    R = rotation(d, sign_bits)
    c, t = codebook(d, bits)
    codes = np.zeros((n, d), dtype=np.uint8)
    norms = np.zeros(n, dtype=np.uint16)
    signs = np.zeros((n, (m + 7) // 8), dtype=np.uint8)
    gamma = np.zeros(n)
    proj = np.zeros((n, m))
    _L().orc_qjl_encode(_p(xb), n, d, bits, _p(R), _p(_c(c, np.float64)), _p(_c(t, np.float64)),
                        _p(Sb), m, _p(codes), _p(norms), _p(signs), _p(gamma), _p(proj))
    return codes, norms, signs, gamma, proj


def qjl_estimate(q, codes, n16, gamma16, signs, S, R, c):
    """Estimates of <q, x_j> for one query q[d] (float64) over encoded keys:
    codes [T][d], n16 / gamma16 float64 [T] (the stored fp16 values), signs
    [T][m/8]; R the rotation, c the levels (tq_oracle.c, orc_qjl_estimate)."""
    qb = _c(q, np.float64)
    d = qb.shape[0]
    Sb = _c(S, np.float64)
    m = Sb.shape[0]
    Rb = _c(R, np.float64)
    cb = _c(c, np.float64)
    cd = _c(codes, np.uint8)
    sg = _c(signs, np.uint8)
    out = np.zeros(cd.shape[0])
    for j in range(cd.shape[0]):
        out[j] = _L().orc_qjl_estimate(_p(qb), d, _p(Rb), _p(cb), _p(cd[j]), float(n16[j]),
                                       float(gamma16[j]), _p(sg[j]), _p(Sb), m)
    return out


def halves_to_double(x):
    """fp16 bit patterns -> float64 values (exact)."""
    return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode_stream(k16, v16, q16, bits_k, bits_v, sign_bits, full=False):
    """The whole path for one (layer, seq, kv head) stream, in the original
    domain: encode K and V, dequantize, attend with the G queries q16[G][d].

    Returns dict(out[G][d], k_codes, k_norms, k_band, v_codes, v_norms, v_band)
    and, with full=True, the dequantized K[T][d] and V[T][d] too."""
    kc, kn, kb = encode(k16, bits_k, sign_bits)
    vc, vn, vb = encode(v16, bits_v, sign_bits)
    K = dequant(kc, kn, bits_k, sign_bits)
    V = dequant(vc, vn, bits_v, sign_bits)
    out = attention(halves_to_double(q16), K, V)
    r = dict(out=out, k_codes=kc, k_norms=kn, k_band=kb, v_codes=vc, v_norms=vn, v_band=vb)
    if full:
        r["K"], r["V"] = K, V
    return r
