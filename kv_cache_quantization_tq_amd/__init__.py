"""Python binding of the ``libtq.so`` C ABI (``include/tq.h``).

Argument marshalling only: every step of encode, append and decode runs in the
library's gfx950 kernels.  PyTorch provides device memory and streams.  There
is no fallback: if the library is missing or no GPU is present the calls raise.
"""
import ctypes
import os

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "libtq.so")

TQ_OK = 0
STATUS = {0: "TQ_OK", 1: "TQ_ERR_ARG", 2: "TQ_ERR_UNSUPPORTED", 3: "TQ_ERR_CAPACITY",
          4: "TQ_ERR_WORKSPACE", 5: "TQ_ERR_DEVICE"}

# Every function include/tq.h declares (checked by the tests).
EXPORTS = (
    "tq_status_str", "tq_codebook_compute", "tq_codebook_init", "tq_codebook_read",
    "tq_codebook_head_dim", "tq_codebook_bits", "tq_codebook_free", "tq_encode",
    "tq_cache_layer_bytes", "tq_append", "tq_decode_workspace_bytes", "tq_decode_attn",
    "tq_decode_attn_sparse", "tq_decode_attn_noalloc", "tq_prefill_attn", "tq_qjl_encode",
    "tq_qjl_scores",
)


class TQError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")
        self.code = code


class KVCacheStruct(ctypes.Structure):
    """Mirror of ``tq_kv_cache``."""
    _fields_ = [
        ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
        ("k_norms", ctypes.c_void_p), ("v_norms", ctypes.c_void_p),
        ("batch", ctypes.c_int), ("kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
        ("bits_k", ctypes.c_int), ("bits_v", ctypes.c_int), ("capacity", ctypes.c_int),
        ("layer_stride_k_codes", ctypes.c_int64), ("layer_stride_v_codes", ctypes.c_int64),
        ("layer_stride_k_norms", ctypes.c_int64), ("layer_stride_v_norms", ctypes.c_int64),
        ("block_table", ctypes.c_void_p),
        ("page_tokens", ctypes.c_int), ("max_pages", ctypes.c_int), ("num_pages", ctypes.c_int),
    ]


_lib = None


def lib():
    """The loaded ``libtq.so`` (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        P = ctypes.POINTER
        L.tq_status_str.argtypes = [i32]
        L.tq_status_str.restype = ctypes.c_char_p
        L.tq_codebook_compute.argtypes = [i32, i32, vp, vp]
        L.tq_codebook_init.argtypes = [i32, i32, P(vp)]
        L.tq_codebook_read.argtypes = [vp, vp, vp]
        L.tq_codebook_head_dim.argtypes = [vp]
        L.tq_codebook_bits.argtypes = [vp]
        L.tq_codebook_free.argtypes = [vp]
        L.tq_codebook_free.restype = None
        L.tq_encode.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp]
        L.tq_cache_layer_bytes.argtypes = [P(KVCacheStruct), P(i64), P(i64), P(i64), P(i64)]
        L.tq_append.argtypes = [P(KVCacheStruct), vp, vp, vp, vp, vp, i32, vp, ctypes.c_int32,
                                i32, vp]
        L.tq_decode_workspace_bytes.argtypes = [P(KVCacheStruct), i32, i32, i32]
        L.tq_decode_workspace_bytes.restype = sz
        L.tq_decode_attn.argtypes = [P(KVCacheStruct), vp, vp, vp, vp, i32, vp, i32, i32, vp,
                                     vp, sz, vp]
        L.tq_decode_attn_sparse.argtypes = [P(KVCacheStruct), vp, vp, vp, vp, i32, vp, i32, i32,
                                            ctypes.c_float, vp, vp, vp, vp, sz, vp]
        L.tq_decode_attn_noalloc.argtypes = [P(KVCacheStruct), vp, vp, vp, vp, i32, vp, i32, i32,
                                             vp, vp]
        L.tq_prefill_attn.argtypes = [P(KVCacheStruct), vp, vp, vp, vp, i32, i32, vp, i32, vp, vp]
        L.tq_qjl_encode.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp, vp, vp]
        L.tq_qjl_scores.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, vp, i64, vp, vp]
        for f in ("tq_codebook_compute", "tq_codebook_init", "tq_codebook_read", "tq_encode",
                  "tq_cache_layer_bytes", "tq_append", "tq_decode_attn", "tq_decode_attn_sparse",
                  "tq_decode_attn_noalloc", "tq_prefill_attn", "tq_qjl_encode", "tq_qjl_scores"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _check(fn, code):
    if code != TQ_OK:
        raise TQError(fn, code)


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def codebook_compute(head_dim, bits):
    """Host Lloyd-Max levels and thresholds (float32 lists) of N(0, 1/d)."""
    L = 1 << bits
    c = (ctypes.c_float * L)()
    t = (ctypes.c_float * (L - 1))()
    _check("tq_codebook_compute", lib().tq_codebook_compute(head_dim, bits, c, t))
    return list(c), list(t)


class Codebook:
    """Device codebook handle for (head_dim, bits) on the current device."""

    def __init__(self, head_dim, bits):
        h = ctypes.c_void_p()
        _check("tq_codebook_init", lib().tq_codebook_init(head_dim, bits, ctypes.byref(h)))
        self.handle = h
        self.head_dim = head_dim
        self.bits = bits

    def read(self):
        L = 1 << self.bits
        c = (ctypes.c_float * L)()
        t = (ctypes.c_float * (L - 1))()
        _check("tq_codebook_read", lib().tq_codebook_read(self.handle, c, t))
        return list(c), list(t)

    def close(self):
        if getattr(self, "handle", None):
            lib().tq_codebook_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def encode(cb, x, sign_bits, codes, norms, stream=None):
    """tq_encode: x fp16 [n][stride] (CUDA), sign_bits uint8 [d/8], codes uint8
    [n][d*bits/8], norms int16/float16 [n]."""
    n = x.shape[0]
    _check("tq_encode", lib().tq_encode(cb.handle, _ptr(x), n, x.stride(0), _ptr(sign_bits),
                                        _ptr(codes), _ptr(norms), _stream(stream)))


class KVCache:
    """Compressed cache of n_layers layers in torch CUDA tensors.

    k_codes [L][B][H][cap][d*bk/8], v_codes [L][B][H][cap/32][32*d*bv/8],
    k_norms / v_norms [L][B][H][cap] (fp16 bits as int16)."""

    def __init__(self, n_layers, batch, kv_heads, head_dim, bits_k, bits_v, capacity,
                 device="cuda"):
        import torch
        if capacity % 32:
            raise ValueError("capacity must be a multiple of 32")
        self.n_layers, self.batch, self.kv_heads = n_layers, batch, kv_heads
        self.head_dim, self.bits_k, self.bits_v, self.capacity = head_dim, bits_k, bits_v, capacity
        d = head_dim
        self.k_codes = torch.zeros((n_layers, batch, kv_heads, capacity, d * bits_k // 8),
                                   dtype=torch.uint8, device=device)
        self.v_codes = torch.zeros((n_layers, batch, kv_heads, capacity // 32, 32 * d * bits_v // 8),
                                   dtype=torch.uint8, device=device)
        self.k_norms = torch.zeros((n_layers, batch, kv_heads, capacity), dtype=torch.int16,
                                   device=device)
        self.v_norms = torch.zeros_like(self.k_norms)

    def struct(self, layer=0):
        s = KVCacheStruct()
        s.k_codes = self.k_codes[layer].data_ptr()
        s.v_codes = self.v_codes[layer].data_ptr()
        s.k_norms = self.k_norms[layer].data_ptr()
        s.v_norms = self.v_norms[layer].data_ptr()
        s.batch, s.kv_heads, s.head_dim = self.batch, self.kv_heads, self.head_dim
        s.bits_k, s.bits_v, s.capacity = self.bits_k, self.bits_v, self.capacity
        s.layer_stride_k_codes = self.k_codes.stride(0)
        s.layer_stride_v_codes = self.v_codes.stride(0)
        s.layer_stride_k_norms = self.k_norms.stride(0) * 2
        s.layer_stride_v_norms = self.v_norms.stride(0) * 2
        return s

    def packed_bytes(self, lengths=None):
        """Bytes of codes + norms for the given per-sequence lengths (all layers)."""
        d = self.head_dim
        per_tok = d * (self.bits_k + self.bits_v) // 8 + 4
        if lengths is None:
            lengths = [self.capacity] * self.batch
        return self.n_layers * self.kv_heads * per_tok * sum(lengths)


class PagedKVCache:
    """Paged compressed cache of n_layers layers: per layer a pool of
    num_pages pages of page_tokens tokens, shared by the batch's sequences
    through block_table (int32 [batch][max_pages], the same for every layer).

    k_codes [L][num_pages][H][P][d*bk/8], v_codes [L][num_pages][H][P/32][32*d*bv/8],
    k_norms / v_norms [L][num_pages][H][P] (fp16 bits as int16)."""

    def __init__(self, n_layers, batch, kv_heads, head_dim, bits_k, bits_v, page_tokens,
                 max_pages, num_pages, block_table, device="cuda"):
        import torch
        self.n_layers, self.batch, self.kv_heads = n_layers, batch, kv_heads
        self.head_dim, self.bits_k, self.bits_v = head_dim, bits_k, bits_v
        self.page_tokens, self.max_pages, self.num_pages = page_tokens, max_pages, num_pages
        self.capacity = page_tokens * max_pages
        self.block_table = torch.as_tensor(block_table, dtype=torch.int32, device=device).contiguous()
        assert tuple(self.block_table.shape) == (batch, max_pages)
        d, P = head_dim, page_tokens
        self.k_codes = torch.zeros((n_layers, num_pages, kv_heads, P, d * bits_k // 8),
                                   dtype=torch.uint8, device=device)
        self.v_codes = torch.zeros((n_layers, num_pages, kv_heads, P // 32, 32 * d * bits_v // 8),
                                   dtype=torch.uint8, device=device)
        self.k_norms = torch.zeros((n_layers, num_pages, kv_heads, P), dtype=torch.int16,
                                   device=device)
        self.v_norms = torch.zeros_like(self.k_norms)

    def struct(self, layer=0):
        s = KVCacheStruct()
        s.k_codes = self.k_codes[layer].data_ptr()
        s.v_codes = self.v_codes[layer].data_ptr()
        s.k_norms = self.k_norms[layer].data_ptr()
        s.v_norms = self.v_norms[layer].data_ptr()
        s.batch, s.kv_heads, s.head_dim = self.batch, self.kv_heads, self.head_dim
        s.bits_k, s.bits_v, s.capacity = self.bits_k, self.bits_v, self.capacity
        s.layer_stride_k_codes = self.k_codes.stride(0)
        s.layer_stride_v_codes = self.v_codes.stride(0)
        s.layer_stride_k_norms = self.k_norms.stride(0) * 2
        s.layer_stride_v_norms = self.v_norms.stride(0) * 2
        s.block_table = self.block_table.data_ptr()
        s.page_tokens, s.max_pages, s.num_pages = self.page_tokens, self.max_pages, self.num_pages
        return s

    def gather(self, layer, b, h):
        """The (layer, sequence b, head h) stream in contiguous layout: key rows
        [capacity][d*bk/8], value tiles [capacity/32][...], norms [capacity]
        (torch tensors, for comparisons)."""
        import torch
        pages = self.block_table[b].long()
        kc = self.k_codes[layer][pages, h].reshape(self.capacity, -1)
        vc = self.v_codes[layer][pages, h].reshape(self.capacity // 32, -1)
        kn = self.k_norms[layer][pages, h].reshape(self.capacity)
        vn = self.v_norms[layer][pages, h].reshape(self.capacity)
        return kc, vc, kn, vn


def append(cache, cbk, cbv, sign_bits, k_new, v_new, pos, host_max_pos=-1, layer0=0,
           n_layers=None, stream=None):
    """tq_append over layers layer0 .. layer0 + n_layers - 1.
    k_new, v_new: fp16 [n_layers][B][H][t_new][d]; pos: int32 [B] (CUDA);
    sign_bits: uint8 [n_layers][d/8] (the same layers)."""
    n_layers = n_layers if n_layers is not None else k_new.shape[0]
    t_new = k_new.shape[3]
    s = cache.struct(layer0)
    _check("tq_append", lib().tq_append(ctypes.byref(s), cbk.handle, cbv.handle, _ptr(sign_bits),
                                        _ptr(k_new), _ptr(v_new), t_new, _ptr(pos),
                                        int(host_max_pos), n_layers, _stream(stream)))


def decode_workspace_bytes(cache, q_heads, max_len, n_layers=None, layer0=0):
    n_layers = n_layers if n_layers is not None else cache.n_layers
    s = cache.struct(layer0)
    return lib().tq_decode_workspace_bytes(ctypes.byref(s), q_heads, max_len, n_layers)


def decode(cache, cbk, cbv, sign_bits, q, seq_lens, max_len, out, ws=None, layer0=0,
           n_layers=None, stream=None):
    """tq_decode_attn: q fp16 [n_layers][B][Hq][d], seq_lens int32 [B] (CUDA),
    out fp32 [n_layers][B][Hq][d], ws uint8 workspace (or None if not needed)."""
    n_layers = n_layers if n_layers is not None else q.shape[0]
    q_heads = q.shape[2]
    s = cache.struct(layer0)
    ws_bytes = ws.numel() if ws is not None else 0
    _check("tq_decode_attn", lib().tq_decode_attn(
        ctypes.byref(s), cbk.handle, cbv.handle, _ptr(sign_bits), _ptr(q), q_heads,
        _ptr(seq_lens), max_len, n_layers, _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def decode_noalloc(cache, cbk, cbv, sign_bits, q, seq_lens, max_len, out, layer0=0,
                   n_layers=None, stream=None):
    """tq_decode_attn_noalloc: decode() with the library's own workspace (no
    allocation; calls on one GPU must not overlap)."""
    n_layers = n_layers if n_layers is not None else q.shape[0]
    q_heads = q.shape[2]
    s = cache.struct(layer0)
    _check("tq_decode_attn_noalloc", lib().tq_decode_attn_noalloc(
        ctypes.byref(s), cbk.handle, cbv.handle, _ptr(sign_bits), _ptr(q), q_heads,
        _ptr(seq_lens), max_len, n_layers, _ptr(out), _stream(stream)))


def skip_words(max_len):
    """Words per (layer, sequence, KV head) of a Sparse V skip bitmap."""
    return (max_len + 1023) // 1024


def decode_sparse(cache, cbk, cbv, sign_bits, q, seq_lens, max_len, out, eps, ws=None,
                  skip_counts=None, skip_tiles=None, layer0=0, n_layers=None, stream=None):
    """tq_decode_attn_sparse: decode with the Sparse V gate at threshold eps;
    skip_counts (optional) uint32/int32 [n_layers][B][Hkv] receives added
    per-unit counts of skipped tiles, skip_tiles (optional) int32
    [n_layers][B][Hkv][skip_words(max_len)] the OR of one bit per skipped
    tile.  Other arguments as decode()."""
    n_layers = n_layers if n_layers is not None else q.shape[0]
    q_heads = q.shape[2]
    s = cache.struct(layer0)
    ws_bytes = ws.numel() if ws is not None else 0
    _check("tq_decode_attn_sparse", lib().tq_decode_attn_sparse(
        ctypes.byref(s), cbk.handle, cbv.handle, _ptr(sign_bits), _ptr(q), q_heads,
        _ptr(seq_lens), max_len, n_layers, float(eps), _ptr(skip_counts), _ptr(skip_tiles),
        _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def prefill(cache, cbk, cbv, sign_bits, q, pos, out, layer0=0, n_layers=None, stream=None):
    """tq_prefill_attn: q fp16 [n_layers][B][Hq][t_new][d], pos int32 [B]
    (CUDA), out fp32 [n_layers][B][Hq][t_new][d]."""
    n_layers = n_layers if n_layers is not None else q.shape[0]
    q_heads, t_new = q.shape[2], q.shape[3]
    s = cache.struct(layer0)
    _check("tq_prefill_attn", lib().tq_prefill_attn(
        ctypes.byref(s), cbk.handle, cbv.handle, _ptr(sign_bits), _ptr(q), q_heads, t_new,
        _ptr(pos), n_layers, _ptr(out), _stream(stream)))


def qjl_encode(cb, x, sign_bits, S, codes, signs, gamma, stream=None):
    """tq_qjl_encode: x fp16 [n][>= d] (CUDA), S fp16 [d][d], codes [n][d*bits/8]
    (tq_encode rows); writes signs uint8 [n][d/8] and gamma fp16 [n]."""
    _check("tq_qjl_encode", lib().tq_qjl_encode(
        cb.handle, _ptr(x), x.shape[0], x.stride(0), _ptr(sign_bits), _ptr(S), _ptr(codes),
        _ptr(signs), _ptr(gamma), _stream(stream)))


def qjl_scores(cb, q, sign_bits, S, codes, norms, signs, gamma, out, stream=None):
    """tq_qjl_scores: q fp16 [n_q][d]; out fp32 [n_q][n_keys]."""
    _check("tq_qjl_scores", lib().tq_qjl_scores(
        cb.handle, _ptr(q), q.shape[0], _ptr(sign_bits), _ptr(S), _ptr(codes), _ptr(norms),
        _ptr(signs), _ptr(gamma), codes.shape[0], _ptr(out), _stream(stream)))


def workspace(cache, q_heads, max_len, n_layers=None, layer0=0, device="cuda"):
    """A zero-filled torch workspace for tq_decode_attn (None if none is needed)."""
    import torch
    nb = decode_workspace_bytes(cache, q_heads, max_len, n_layers, layer0)
    if nb == 0:
        return None
    return torch.zeros(nb, dtype=torch.uint8, device=device)
