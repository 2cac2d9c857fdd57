"""Seeded synthetic inputs for the KV-cache codec (shared by the oracle tests
and the GPU path; holds none of the codec's arithmetic).

Host values come from ``libsynth_host.so`` (gcc); device tensors are filled by
``libsynth_dev.so`` (hipcc).  Both compile ``synth_core.h`` and produce
bit-identical fp16 values for the same (seed, layer, seq, head, token, coord).

Workload recipe (per coordinate of a K or V vector of one (layer, seq, kv head)):
``x = fp16_rne(z * (10 if the coordinate is one of the stream's 4 outlier
channels) * exp(0.5 * z'))`` with z ~ N(0,1) per coordinate and z' ~ N(0,1) per
token.  Queries are fp16 N(0,1).  Sign bits are fair coin flips per layer.
"""
import ctypes
import os

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_host = None
_dev = None

TAG_SCALE_K = 4
TAG_SCALE_V = 5


def _lib_host():
    global _host
    if _host is None:
        path = os.path.join(_DIR, "libsynth_host.so")
        if not os.path.exists(path):
            raise RuntimeError("libsynth_host.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        u64, i32, i64, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        lib.synth_kv_host.argtypes = [u64, i32, i32, i32, i32, i32, i64, i64, vp]
        lib.synth_q_host.argtypes = [u64, i32, i32, i32, i32, i32, vp]
        lib.synth_sign_bits_host.argtypes = [u64, i32, i32, vp]
        lib.synth_outliers_host.argtypes = [u64, i32, i32, i32, i32, vp]
        lib.synth_iso_host.argtypes = [u64, u64, i64, i32, vp]
        lib.synth_normals_host.argtypes = [u64, u64, i64, vp]
        lib.synth_key_host.argtypes = [u64, u64, u64, u64, u64]
        lib.synth_key_host.restype = u64
        lib.synth_f16_rne_host.argtypes = [ctypes.c_double]
        lib.synth_f16_rne_host.restype = ctypes.c_uint16
        for f in ("synth_log_host", "synth_exp_host", "synth_cos2pi_host"):
            getattr(lib, f).argtypes = [ctypes.c_double]
            getattr(lib, f).restype = ctypes.c_double
        _host = lib
    return _host


def _lib_dev():
    global _dev
    if _dev is None:
        path = os.path.join(_DIR, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError("libsynth_dev.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        u64, i32, i64, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        lib.synth_kv_dev.argtypes = [u64, i32, i32, i32, i32, i32, i64, i64, vp, i64, i64, i64, vp]
        lib.synth_q_dev.argtypes = [u64, i32, i32, i32, i32, i32, vp, i64, vp]
        _dev = lib
    return _dev


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def kv_host(seed, kind, layer, seq, head, d, t0, nt):
    """fp16 bits [nt][d] (uint16) of K (kind 0) or V (kind 1)."""
    out = np.empty((nt, d), dtype=np.uint16)
    _lib_host().synth_kv_host(seed, kind, layer, seq, head, d, t0, nt, _ptr(out))
    return out


def q_host(seed, step, layer, seq, qhead, d):
    out = np.empty(d, dtype=np.uint16)
    _lib_host().synth_q_host(seed, step, layer, seq, qhead, d, _ptr(out))
    return out


def sign_bits(seed, layer, d):
    out = np.empty(d // 8, dtype=np.uint8)
    _lib_host().synth_sign_bits_host(seed, layer, d, _ptr(out))
    return out


def outliers(seed, kind, layer, head, d):
    out = np.empty(4, dtype=np.int32)
    _lib_host().synth_outliers_host(seed, kind, layer, head, d, _ptr(out))
    return out


def iso_host(seed, stream_id, n, d):
    out = np.empty((n, d), dtype=np.uint16)
    _lib_host().synth_iso_host(seed, stream_id, n, d, _ptr(out))
    return out


def normals_host(stream, c0, n):
    out = np.empty(n, dtype=np.float64)
    _lib_host().synth_normals_host(stream, c0, n, _ptr(out))
    return out


def key(seed, tag, a, b, c):
    return _lib_host().synth_key_host(seed, tag, a, b, c)


def f16_rne(v):
    return _lib_host().synth_f16_rne_host(float(v))


def kv_dev(seed, kind, layer, out, t0=0, stream=0):
    """Fill a CUDA int16/uint16-viewed tensor ``out`` of shape [B][H][nt][d]
    (last dim contiguous; any strides for the others) with fp16 K/V bits."""
    B, H, nt, d = out.shape
    s = out.stride()
    if s[3] != 1:
        raise ValueError("last dim must be contiguous")
    rc = _lib_dev().synth_kv_dev(seed, kind, layer, B, H, d, t0, nt, out.data_ptr(),
                                 s[0], s[1], s[2], stream)
    if rc:
        raise RuntimeError("synth_kv_dev launch failed")


def q_dev(seed, step, layer, out, stream=0):
    """Fill a CUDA tensor ``out`` [B][Hq][d] (contiguous) with fp16 query bits."""
    B, Hq, d = out.shape
    if not out.is_contiguous():
        raise ValueError("query tensor must be contiguous")
    rc = _lib_dev().synth_q_dev(seed, step, layer, B, Hq, d, out.data_ptr(), Hq * d, stream)
    if rc:
        raise RuntimeError("synth_q_dev launch failed")
