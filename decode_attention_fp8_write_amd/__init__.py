"""Python binding of libpda.so — FP8 (OCP e4m3) paged decode attention for
MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in include/pda.h. PyTorch provides device memory and the
current stream; the functions take torch tensors and pass raw device
pointers. There is no CPU fallback: if the library or a GPU is missing the
calls raise.

Names follow the C ABI: kv_write_fp8, kv_write_bf16, validate_page_tags,
kv_write_check, paged_decode_attn_workspace_bytes, paged_decode_attn.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpda.so")

(PDA_OK, PDA_ERR_INVALID_ARG, PDA_ERR_UNSUPPORTED, PDA_ERR_LAUNCH, PDA_ERR_WORKSPACE,
 PDA_ERR_POOL_EXHAUSTED, PDA_ERR_SCRATCH) = range(7)
KV_BF16, KV_FP8_E4M3 = 0, 1
SCALE_NONE, SCALE_PER_HEAD, SCALE_PER_TOKEN = 0, 1, 2

EXPORTS = ("kv_write_fp8", "kv_write_bf16", "kv_transcode_bf16_to_fp8", "validate_page_tags",
           "kv_write_check",
           "paged_decode_attn_workspace_bytes", "paged_decode_attn",
           "paged_decode_attn_noalloc", "paged_decode_attn_noalloc_scratch_bytes",
           "pda_status_string", "pda_pool_create", "pda_pool_destroy", "pda_pool_alloc",
           "pda_pool_free", "pda_pool_tags", "pda_pool_num_free",
           "pda_hbm_read_probe", "pda_hbm_read_probe_sink_words", "int4_gemv_bf16")


class PdaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class AttnShape(ctypes.Structure):
    """Mirror of pda_attn_shape."""
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim_qk", ctypes.c_int32),
                ("head_dim_v", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("scale_mode", ctypes.c_int32),
                ("v_in_k", ctypes.c_int32), ("split_tokens", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


_lib = None


def load(path: str | None = None):
    """Load libpda.so (built in-tree by build.py). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libpda.so not built at {p}: run "
                           "`python -m decode_attention_fp8_write_amd.build`")
    lib = ctypes.CDLL(p)
    V, I32, I64P = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p
    lib.kv_write_fp8.argtypes = [V, V, I64P, I32, I32, I32, I32, I32, I32, I32, V, V,
                                 V, V, V, V]
    lib.kv_write_fp8.restype = ctypes.c_int
    lib.kv_write_bf16.argtypes = [V, V, I64P, I32, I32, I32, I32, I32, I32, V, V, V]
    lib.kv_write_bf16.restype = ctypes.c_int
    lib.kv_transcode_bf16_to_fp8.argtypes = [V, V, V, V, V, I32, I32, I32, I32, I32, I32,
                                             I32, I32, V, V, V, V, V, V]
    lib.kv_transcode_bf16_to_fp8.restype = ctypes.c_int
    lib.validate_page_tags.argtypes = [V, I32, V, V, I32, V, I32, I32, V, V]
    lib.validate_page_tags.restype = ctypes.c_int
    lib.kv_write_check.argtypes = [V, V, I64P, I32, I32, I32, I32, I32, I32, I32, I32, V, V, V,
                                   V, V, V, V, V, I32, V, I32, V, V]
    lib.kv_write_check.restype = ctypes.c_int
    lib.paged_decode_attn_workspace_bytes.argtypes = [ctypes.POINTER(AttnShape), I32]
    lib.paged_decode_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.paged_decode_attn.argtypes = [ctypes.POINTER(AttnShape), V, V, V, V, V, V, V, I32,
                                      V, V, ctypes.c_size_t, V, V]
    lib.paged_decode_attn.restype = ctypes.c_int
    lib.paged_decode_attn_noalloc.argtypes = [ctypes.POINTER(AttnShape), V, V, V, V, V, V, V,
                                              I32, V, V, V]
    lib.paged_decode_attn_noalloc.restype = ctypes.c_int
    lib.paged_decode_attn_noalloc_scratch_bytes.argtypes = []
    lib.paged_decode_attn_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.pda_status_string.argtypes = [ctypes.c_int]
    lib.pda_status_string.restype = ctypes.c_char_p
    lib.pda_pool_create.argtypes = [I32, V, ctypes.c_uint32, I32, ctypes.POINTER(ctypes.c_void_p)]
    lib.pda_pool_create.restype = ctypes.c_int
    lib.pda_pool_destroy.argtypes = [V]
    lib.pda_pool_destroy.restype = None
    lib.pda_pool_alloc.argtypes = [V, I32, V, V]
    lib.pda_pool_alloc.restype = ctypes.c_int
    lib.pda_pool_free.argtypes = [V, V, I32]
    lib.pda_pool_free.restype = ctypes.c_int
    lib.pda_pool_tags.argtypes = [V]
    lib.pda_pool_tags.restype = ctypes.POINTER(ctypes.c_uint32)
    lib.pda_pool_num_free.argtypes = [V]
    lib.pda_pool_num_free.restype = I32
    lib.pda_hbm_read_probe_sink_words.argtypes = []
    lib.pda_hbm_read_probe_sink_words.restype = ctypes.c_size_t
    lib.pda_hbm_read_probe.argtypes = [V, ctypes.c_size_t, I32, V, V]
    lib.pda_hbm_read_probe.restype = ctypes.c_int
    lib.int4_gemv_bf16.argtypes = [V, V, V, I32, I32, I32, I32, V, V]
    lib.int4_gemv_bf16.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().pda_status_string(status).decode()


def _check(fn: str, status: int):
    if status != PDA_OK:
        raise PdaError(fn, status, status_string(status))


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t, *, elem=None, name="tensor"):
    """Device pointer of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if elem is not None and t.element_size() != elem:
        raise ValueError(f"{name} must have {elem}-byte elements")
    return ctypes.c_void_p(t.data_ptr())


def kv_write_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, *, page_size, num_pages,
                 scale_mode=SCALE_PER_HEAD, k_scale=None, v_scale=None, token_scale=None,
                 stream=None):
    """Quantise bf16 K/V rows [T, Hkv, D] to e4m3 and scatter them by slot.
    Caches are uint8 tensors in the format of include/pda.h."""
    T, hkv, dk = k_new.shape
    dv = v_new.shape[2] if v_new is not None else 0
    st = load().kv_write_fp8(
        _ptr(k_new, elem=2, name="k_new"), _ptr(v_new, elem=2, name="v_new"),
        _ptr(slot_mapping, elem=8, name="slot_mapping"), T, hkv, dk, dv, page_size, num_pages,
        scale_mode, _ptr(k_scale, elem=4, name="k_scale"), _ptr(v_scale, elem=4, name="v_scale"),
        _ptr(token_scale, elem=4, name="token_scale"), _ptr(k_cache, elem=1, name="k_cache"),
        _ptr(v_cache, elem=1, name="v_cache"), _stream(stream))
    _check("kv_write_fp8", st)


def kv_write_bf16(k_new, v_new, slot_mapping, k_cache, v_cache, *, page_size, num_pages,
                  stream=None):
    T, hkv, dk = k_new.shape
    dv = v_new.shape[2] if v_new is not None else 0
    st = load().kv_write_bf16(
        _ptr(k_new, elem=2, name="k_new"), _ptr(v_new, elem=2, name="v_new"),
        _ptr(slot_mapping, elem=8, name="slot_mapping"), T, hkv, dk, dv, page_size, num_pages,
        _ptr(k_cache, elem=2, name="k_cache"), _ptr(v_cache, elem=2, name="v_cache"),
        _stream(stream))
    _check("kv_write_bf16", st)


def kv_transcode_bf16_to_fp8(k_src, v_src, src_pages, dst_pages, valid, k_dst, v_dst, *,
                             num_kv_heads, head_dim_k, head_dim_v, page_size, src_num_pages,
                             dst_num_pages, scale_mode=SCALE_PER_HEAD, k_scale=None,
                             v_scale=None, token_scale=None, stream=None):
    """Re-encode slots [0, valid[i]) of BF16 page src_pages[i] into FP8 page
    dst_pages[i] (int32 device arrays of one length; caches as in
    include/pda.h: uint16 sources, uint8 destinations)."""
    n = src_pages.numel()
    if dst_pages.numel() != n or valid.numel() != n:
        raise ValueError("src_pages, dst_pages and valid must have one length")
    st = load().kv_transcode_bf16_to_fp8(
        _ptr(k_src, elem=2, name="k_src"), _ptr(v_src, elem=2, name="v_src"),
        _ptr(src_pages, elem=4, name="src_pages"), _ptr(dst_pages, elem=4, name="dst_pages"),
        _ptr(valid, elem=4, name="valid"), n, num_kv_heads, head_dim_k, head_dim_v, page_size,
        src_num_pages, dst_num_pages, scale_mode, _ptr(k_scale, elem=4, name="k_scale"),
        _ptr(v_scale, elem=4, name="v_scale"), _ptr(token_scale, elem=4, name="token_scale"),
        _ptr(k_dst, elem=1, name="k_dst"), _ptr(v_dst, elem=1, name="v_dst"), _stream(stream))
    _check("kv_transcode_bf16_to_fp8", st)


def validate_page_tags(page_tags, block_table, expected_tags, seq_lens, verdict, *,
                       page_size, stream=None):
    B, max_blocks = block_table.shape
    st = load().validate_page_tags(
        _ptr(page_tags, elem=4, name="page_tags"), page_tags.shape[0],
        _ptr(block_table, elem=4, name="block_table"),
        _ptr(expected_tags, elem=4, name="expected_tags"), max_blocks,
        _ptr(seq_lens, elem=4, name="seq_lens"), B, page_size,
        _ptr(verdict, elem=4, name="verdict"), _stream(stream))
    _check("validate_page_tags", st)


def kv_write_check(k_new, v_new, slot_mapping, k_cache, v_cache, page_tags, block_table,
                   expected_tags, seq_lens, verdict, *, page_size, num_pages, kv_dtype,
                   scale_mode, k_scale=None, v_scale=None, token_scale=None, stream=None):
    """kv_write_fp8 (kv_dtype KV_FP8_E4M3) or kv_write_bf16 (KV_BF16,
    scale_mode SCALE_NONE) and validate_page_tags in one launch; arguments
    as those calls take them."""
    T, hkv, dk = k_new.shape
    dv = v_new.shape[2] if v_new is not None else 0
    B, max_blocks = block_table.shape
    elem = 1 if kv_dtype == KV_FP8_E4M3 else 2
    st = load().kv_write_check(
        _ptr(k_new, elem=2, name="k_new"), _ptr(v_new, elem=2, name="v_new"),
        _ptr(slot_mapping, elem=8, name="slot_mapping"), T, hkv, dk, dv, page_size, num_pages,
        kv_dtype, scale_mode, _ptr(k_scale, elem=4, name="k_scale"),
        _ptr(v_scale, elem=4, name="v_scale"), _ptr(token_scale, elem=4, name="token_scale"),
        _ptr(k_cache, elem=elem, name="k_cache"), _ptr(v_cache, elem=elem, name="v_cache"),
        _ptr(page_tags, elem=4, name="page_tags"), _ptr(block_table, elem=4, name="block_table"),
        _ptr(expected_tags, elem=4, name="expected_tags"), max_blocks,
        _ptr(seq_lens, elem=4, name="seq_lens"), B, _ptr(verdict, elem=4, name="verdict"),
        _stream(stream))
    _check("kv_write_check", st)


def make_shape(*, num_seqs, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size,
               num_pages, max_blocks_per_seq, kv_dtype, scale_mode, v_in_k=False,
               split_tokens=0, sm_scale) -> AttnShape:
    return AttnShape(num_seqs, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size,
                     num_pages, max_blocks_per_seq, kv_dtype, scale_mode, int(v_in_k),
                     split_tokens, sm_scale)


def paged_decode_attn_workspace_bytes(shape: AttnShape, max_seq_len: int) -> int:
    return int(load().paged_decode_attn_workspace_bytes(ctypes.byref(shape), max_seq_len))


def paged_decode_attn(shape: AttnShape, q, k_cache, v_cache, k_scale, v_scale, block_table,
                      seq_lens, max_seq_len, verdict, workspace, out, stream=None):
    """out[B, Hq, Dv] fp32 <- attention over the paged cache. verdict None =
    no-op tracker. workspace: uint8 GPU tensor of at least
    paged_decode_attn_workspace_bytes(shape, max_seq_len) bytes."""
    elem = 1 if shape.kv_dtype == KV_FP8_E4M3 else 2
    st = load().paged_decode_attn(
        ctypes.byref(shape), _ptr(q, elem=2, name="q"), _ptr(k_cache, elem=elem, name="k_cache"),
        _ptr(v_cache, elem=elem, name="v_cache"), _ptr(k_scale, elem=4, name="k_scale"),
        _ptr(v_scale, elem=4, name="v_scale"), _ptr(block_table, elem=4, name="block_table"),
        _ptr(seq_lens, elem=4, name="seq_lens"), int(max_seq_len),
        _ptr(verdict, elem=4, name="verdict"), _ptr(workspace, name="workspace"),
        workspace.numel() * workspace.element_size(), _ptr(out, elem=4, name="out"),
        _stream(stream))
    _check("paged_decode_attn", st)


def paged_decode_attn_noalloc(shape: AttnShape, q, k_cache, v_cache, k_scale, v_scale,
                              block_table, seq_lens, max_seq_len, verdict, out, stream=None):
    """paged_decode_attn without a workspace: the library's fixed per-device
    scratch holds the partials (calls on one device must not overlap)."""
    elem = 1 if shape.kv_dtype == KV_FP8_E4M3 else 2
    st = load().paged_decode_attn_noalloc(
        ctypes.byref(shape), _ptr(q, elem=2, name="q"), _ptr(k_cache, elem=elem, name="k_cache"),
        _ptr(v_cache, elem=elem, name="v_cache"), _ptr(k_scale, elem=4, name="k_scale"),
        _ptr(v_scale, elem=4, name="v_scale"), _ptr(block_table, elem=4, name="block_table"),
        _ptr(seq_lens, elem=4, name="seq_lens"), int(max_seq_len),
        _ptr(verdict, elem=4, name="verdict"), _ptr(out, elem=4, name="out"), _stream(stream))
    _check("paged_decode_attn_noalloc", st)


def paged_decode_attn_noalloc_scratch_bytes() -> int:
    return int(load().paged_decode_attn_noalloc_scratch_bytes())


class PagePool:
    """The host page pool and tag tracker of libpda.so (pda_pool_*), over
    numpy arrays. alloc raises PdaError(PDA_ERR_POOL_EXHAUSTED) when fewer
    pages are free than asked for; free raises on ids out of range, not in
    use or repeated; in both cases nothing changes."""

    def __init__(self, num_pages: int, initial_order=None, tag_start: int = 0,
                 track_tags: bool = True):
        import numpy as np
        self._np = np
        lib = load()
        order = None
        if initial_order is not None:
            order = np.ascontiguousarray(initial_order, dtype=np.int32)
            if order.size != num_pages:
                raise ValueError("initial_order must hold num_pages ids")
        h = ctypes.c_void_p()
        st = lib.pda_pool_create(num_pages, None if order is None else order.ctypes.data,
                                 tag_start & 0xFFFFFFFF, 1 if track_tags else 0,
                                 ctypes.byref(h))
        _check("pda_pool_create", st)
        self._h = h
        self.num_pages = num_pages

    def close(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:   # the library may be gone at interpreter exit
            _lib.pda_pool_destroy(h)
        self._h = None

    def __del__(self):
        self.close()

    @property
    def num_free(self) -> int:
        return int(load().pda_pool_num_free(self._h))

    def alloc(self, n: int):
        np = self._np
        pages = np.empty(n, np.int32)
        tags = np.empty(n, np.uint32)
        st = load().pda_pool_alloc(self._h, n, pages.ctypes.data, tags.ctypes.data)
        _check("pda_pool_alloc", st)
        return pages, tags

    def free(self, pages) -> None:
        np = self._np
        p = np.ascontiguousarray(pages, dtype=np.int32)
        _check("pda_pool_free", load().pda_pool_free(self._h, p.ctypes.data, p.size))

    def tags(self):
        """Copy of the current per-page tags (uint32 [num_pages])."""
        np = self._np
        ptr = load().pda_pool_tags(self._h)
        return np.ctypeslib.as_array(ptr, shape=(self.num_pages,)).copy()


def hbm_read_probe(buf, chunk_bytes: int, sink, stream=None):
    """Read every byte of the CUDA tensor `buf` once (include/pda_probe.h):
    chunk_bytes 0 streams, else scrambled chunks of that size. sink: int32
    tensor of at least hbm_read_probe_sink_words() elements."""
    if sink.numel() < load().pda_hbm_read_probe_sink_words():
        raise ValueError("sink too small")
    nbytes = buf.numel() * buf.element_size()
    _check("pda_hbm_read_probe", load().pda_hbm_read_probe(
        _ptr(buf, name="buf"), nbytes, chunk_bytes, _ptr(sink, elem=4, name="sink"),
        _stream(stream)))


def hbm_read_probe_sink_words() -> int:
    return int(load().pda_hbm_read_probe_sink_words())


def int4_gemv_bf16(x, w, scale, y, *, group=128, stream=None):
    """y[m][n] = x[m][k] . dequant(w)^T (include/pda_int4.h). x: bf16 (or
    int16 bits) [m, k]; w: int32/uint32 [n, k/8] of packed two's-complement
    4-bit codes; scale: bf16 (or int16 bits) [n, k/group]; y: float32 [m, n]."""
    m, k = x.shape
    n = w.shape[0]
    if w.shape != (n, k // 8) or scale.shape != (n, k // group) or y.shape != (m, n):
        raise ValueError("int4_gemv_bf16: shapes do not match")
    _check("int4_gemv_bf16", load().int4_gemv_bf16(
        _ptr(x, elem=2, name="x"), _ptr(w, elem=4, name="w"), _ptr(scale, elem=2, name="scale"),
        m, n, k, group, _ptr(y, elem=4, name="y"), _stream(stream)))
