"""CPU oracle for the FP8 paged decode-attention path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU product
path (``decode_attention_fp8_write_amd``) never imports it and shares no code
with it: the arithmetic lives in ``oracle.c`` (plain C, fp64, built with
``-ffp-contract=off`` and no fast-math) and this module only marshals numpy
arrays into it.

What each function computes, and which passage of the pages it follows, is
stated in ``oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build() -> str:
    """Compile liboracle.so with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
           "-pthread", "-Wall", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = f64
    lib.oracle_e4m3_encode.argtypes = [f32]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode_brute.argtypes = [f32]
    lib.oracle_e4m3_encode_brute.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode_closed.argtypes = [f32]
    lib.oracle_e4m3_encode_closed.restype = ctypes.c_uint8
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = f32
    lib.oracle_kv_write_fp8.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32,
                                        i32, P, P, P, P, P]
    lib.oracle_kv_write_fp8.restype = ctypes.c_int
    lib.oracle_kv_write_bf16.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32,
                                         P, P]
    lib.oracle_kv_write_bf16.restype = ctypes.c_int
    lib.oracle_kv_transcode_bf16_to_fp8.argtypes = [P, P, P, P, P, i32, i32, i32, i32,
                                                    i32, i32, i32, i32, P, P, P, P, P]
    lib.oracle_kv_transcode_bf16_to_fp8.restype = ctypes.c_int
    lib.oracle_validate_page_tags.argtypes = [P, i32, P, P, i32, P, i32, i32, P]
    lib.oracle_validate_page_tags.restype = None
    lib.oracle_paged_decode_attn.argtypes = [
        i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, f64,
        P, P, P, P, P, P, P, P, P, P, i32, i32]
    lib.oracle_paged_decode_attn.restype = None
    lib.oracle_int4_gemv.argtypes = [P, P, P, i32, i32, i32, i32, P, i32, P, P]
    lib.oracle_int4_gemv.restype = ctypes.c_int
    _ = i64
    _lib = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _arr(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, f"expected {dtype}, got {a.dtype}"
    return a


# --- codec ------------------------------------------------------------------

def e4m3_decode(code: int) -> float:
    return _load().oracle_e4m3_decode(int(code))


def e4m3_encode(x: float) -> int:
    return _load().oracle_e4m3_encode(float(x))


def e4m3_encode_brute(x: float) -> int:
    return _load().oracle_e4m3_encode_brute(float(x))


def e4m3_encode_closed(x: float) -> int:
    return _load().oracle_e4m3_encode_closed(float(x))


def e4m3_decode_all() -> np.ndarray:
    """fp64 value of every code 0..255 (NaN for 0x7F, 0xFF)."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def bf16_to_f32(bits: int) -> float:
    return _load().oracle_bf16_to_f32(int(bits))


# --- kv write ---------------------------------------------------------------

def kv_write_fp8(k_new, v_new, slot_mapping, page_size, num_pages, scale_mode,
                 k_scale, v_scale, token_scale, k_cache, v_cache):
    """In-place quantise + scatter into numpy caches (uint8). k_new/v_new are
    uint16 bf16 bit patterns [T, Hkv, D]; v_new None for latent caches."""
    k_new = _arr(k_new, np.uint16)
    v_new = _arr(v_new, np.uint16)
    slots = _arr(slot_mapping, np.int64)
    T, hkv, dk = k_new.shape
    dv = v_new.shape[2] if v_new is not None else 0
    for c in (k_cache, v_cache, token_scale):
        if c is not None:
            assert c.flags["C_CONTIGUOUS"]
    rc = _load().oracle_kv_write_fp8(
        _ptr(k_new), _ptr(v_new), _ptr(slots), T, hkv, dk, dv, page_size,
        num_pages, scale_mode, _ptr(_arr(k_scale, np.float32)),
        _ptr(_arr(v_scale, np.float32)), _ptr(token_scale), _ptr(k_cache),
        _ptr(v_cache))
    if rc != 0:
        raise ValueError("oracle_kv_write_fp8 rejected its arguments")


def kv_write_bf16(k_new, v_new, slot_mapping, page_size, num_pages, k_cache,
                  v_cache):
    k_new = _arr(k_new, np.uint16)
    v_new = _arr(v_new, np.uint16)
    slots = _arr(slot_mapping, np.int64)
    T, hkv, dk = k_new.shape
    dv = v_new.shape[2] if v_new is not None else 0
    rc = _load().oracle_kv_write_bf16(
        _ptr(k_new), _ptr(v_new), _ptr(slots), T, hkv, dk, dv, page_size,
        num_pages, _ptr(k_cache), _ptr(v_cache))
    if rc != 0:
        raise ValueError("oracle_kv_write_bf16 rejected its arguments")


def kv_transcode_bf16_to_fp8(k_src, v_src, src_pages, dst_pages, valid, num_kv_heads,
                             head_dim_k, head_dim_v, page_size, src_num_pages,
                             dst_num_pages, scale_mode, k_scale, v_scale, token_scale,
                             k_dst, v_dst):
    """In place: re-encode slots [0, valid[i]) of BF16 page src_pages[i] into
    FP8 page dst_pages[i] (uint16 / uint8 numpy caches, flat)."""
    k_src = _arr(k_src, np.uint16)
    v_src = _arr(v_src, np.uint16)
    sp = _arr(np.asarray(src_pages, np.int32), np.int32)
    dp = _arr(np.asarray(dst_pages, np.int32), np.int32)
    vl = _arr(np.asarray(valid, np.int32), np.int32)
    for c in (k_dst, v_dst, token_scale):
        if c is not None:
            assert c.flags["C_CONTIGUOUS"]
    rc = _load().oracle_kv_transcode_bf16_to_fp8(
        _ptr(k_src), _ptr(v_src), _ptr(sp), _ptr(dp), _ptr(vl), len(sp), num_kv_heads,
        head_dim_k, head_dim_v, page_size, src_num_pages, dst_num_pages, scale_mode,
        _ptr(_arr(k_scale, np.float32)), _ptr(_arr(v_scale, np.float32)), _ptr(token_scale),
        _ptr(k_dst), _ptr(v_dst))
    if rc != 0:
        raise ValueError("oracle_kv_transcode_bf16_to_fp8 rejected its arguments")


# --- validation ---------------------------------------------------------------

def validate_page_tags(page_tags, block_table, expected_tags, seq_lens,
                       page_size) -> np.ndarray:
    page_tags = _arr(page_tags, np.uint32)
    block_table = _arr(block_table, np.int32)
    expected_tags = _arr(expected_tags, np.uint32)
    seq_lens = _arr(seq_lens, np.int32)
    B, max_blocks = block_table.shape
    verdict = np.empty(B, dtype=np.int32)
    _load().oracle_validate_page_tags(
        _ptr(page_tags), page_tags.shape[0], _ptr(block_table),
        _ptr(expected_tags), max_blocks, _ptr(seq_lens), B, page_size,
        _ptr(verdict))
    return verdict


# --- attention ----------------------------------------------------------------

def paged_decode_attn(q, k_cache, v_cache, k_scale, v_scale, block_table,
                      seq_lens, *, num_kv_heads, head_dim_v, page_size,
                      num_pages, kv_dtype, scale_mode, v_in_k, sm_scale,
                      verdict=None, rows=None, out=None, num_threads=None):
    """fp32 [B, Hq, Dv]. q: uint16 bf16 bits [B, Hq, Dk]. kv_dtype 0 = BF16
    caches (uint16), 1 = FP8 (uint8). rows: optional int array [n, 2] of
    (seq, q_head) to compute; other rows of `out` are left as they were
    (NaN when `out` is not given)."""
    q = _arr(q, np.uint16)
    B, hq, dk = q.shape
    block_table = _arr(block_table, np.int32)
    seq_lens = _arr(seq_lens, np.int32)
    verdict = _arr(verdict, np.int32)
    if kv_dtype == 0:
        k_cache = _arr(k_cache, np.uint16)
        v_cache = _arr(v_cache, np.uint16)
    else:
        k_cache = _arr(k_cache, np.uint8)
        v_cache = _arr(v_cache, np.uint8)
    if out is None:
        out = np.full((B, hq, head_dim_v), np.nan, dtype=np.float32)
    rows_arr = None
    n_rows = 0
    if rows is not None:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        n_rows = rows_arr.shape[0]
    if num_threads is None:
        num_threads = os.cpu_count() or 1
    _load().oracle_paged_decode_attn(
        B, hq, num_kv_heads, dk, head_dim_v, page_size, num_pages,
        block_table.shape[1], kv_dtype, scale_mode, int(v_in_k),
        float(sm_scale), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(_arr(k_scale, np.float32)), _ptr(_arr(v_scale, np.float32)),
        _ptr(block_table), _ptr(seq_lens), _ptr(verdict), _ptr(out),
        _ptr(rows_arr), n_rows, int(num_threads))
    return out


# --- INT4 weight-only GEMV ---------------------------------------------------

def int4_gemv(x, w, scale, group=128, cols=None):
    """y[m][n] = x @ dequant(w)^T in fp64, and sum |x * W| per output.
    x: uint16 bf16 bits [m][k]; w: uint32 [n][k/8] (code j of a word is
    element 8*word + j, two's complement in bits 4j..4j+3); scale: uint16
    bf16 bits [n][k/group]. cols: optional output columns to compute (the
    others are NaN)."""
    x = _arr(x, np.uint16)
    w = _arr(w, np.uint32)
    scale = _arr(scale, np.uint16)
    m, k = x.shape
    n = w.shape[0]
    assert w.shape == (n, k // 8) and scale.shape == (n, k // group)
    y = np.full((m, n), np.nan)
    ya = np.full((m, n), np.nan)
    c = None if cols is None else np.ascontiguousarray(np.asarray(cols, np.int32))
    rc = _load().oracle_int4_gemv(_ptr(x), _ptr(w), _ptr(scale), m, n, k, group, _ptr(c),
                                  0 if c is None else c.size, _ptr(y), _ptr(ya))
    if rc != 0:
        raise ValueError("oracle_int4_gemv: invalid arguments")
    return y, ya
