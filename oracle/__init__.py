"""CPU oracle for the indexer path: paged MQA logits and per-row top-k.

TEST INFRASTRUCTURE ONLY. The library's product path never imports this
package; only the test suite, the smoke check and the CPU-baseline leg of the
benchmark do. The arithmetic lives in ``oracle.c`` (plain loops, double
precision, its own FP8/E2M1/E8M0 decoders); this module only builds it with
gcc and marshals numpy arrays into it.

Definitions followed are stated in the header of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_SANITIZE=1 builds and loads a copy instrumented with AddressSanitizer
# and UndefinedBehaviorSanitizer (every report fatal); the process must then
# preload gcc's libasan and libubsan (the interpreter itself is not built with
# them).
_SANITIZE = os.environ.get("ORACLE_SANITIZE", "") not in ("", "0")
_LIB = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")

FP8 = 1
MXFP4 = 2

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP over rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        if _SANITIZE:
            cmd[1:1] = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-fno-omit-frame-pointer", "-g"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        lib.orc_threads.restype = ctypes.c_int
        lib.orc_threads.argtypes = []
        lib.orc_dec_fp8_e4m3.restype = ctypes.c_double
        lib.orc_dec_fp8_e4m3.argtypes = [ctypes.c_uint8]
        lib.orc_dec_e2m1.restype = ctypes.c_double
        lib.orc_dec_e2m1.argtypes = [ctypes.c_uint8]
        lib.orc_dec_e8m0.restype = ctypes.c_double
        lib.orc_dec_e8m0.argtypes = [ctypes.c_uint8]
        lib.orc_decode_logits.restype = i32
        lib.orc_decode_logits.argtypes = [
            i32, P, P, P, i32, i32, P, i64, i64, P, i64, i64, i32, i64,
            P, i64, P, i32, i32, P, i64, i64, P, P]
        lib.orc_prefill_logits.restype = i32
        lib.orc_prefill_logits.argtypes = [
            i32, P, P, P, i32, i32, P, i64, i64, P, i64, i64, i32, i64,
            P, P, i64, P, i64, i64, P, P]
        lib.orc_topk_f64.restype = i32
        lib.orc_topk_f64.argtypes = [P, i64, i32, P]
        lib.orc_topk_f32.restype = i32
        lib.orc_topk_f32.argtypes = [P, i64, i32, P]
        lib.orc_topk_rows_f32.restype = i32
        lib.orc_topk_rows_f32.argtypes = [P, i64, P, i64, i32, P]
        lib.orc_enc_fp8_e4m3.restype = ctypes.c_uint8
        lib.orc_enc_fp8_e4m3.argtypes = [ctypes.c_float]
        lib.orc_quant_fp8_row.restype = None
        lib.orc_quant_fp8_row.argtypes = [P, i32, P, P]
        lib.orc_quant_mxfp4_row.restype = None
        lib.orc_quant_mxfp4_row.argtypes = [P, i32, P, P]
        lib.orc_kv_write.restype = i32
        lib.orc_kv_write.argtypes = [i32, P, i64, i64, i32, P, i32, i64, P, i64, i64, P, i64, i64]
        lib.orc_quantize_query.restype = i32
        lib.orc_quantize_query.argtypes = [i32, P, i64, i64, i32, i32, P, ctypes.c_float, i32,
                                           P, P, P]
        lib.orc_sparse_mla.restype = i32
        lib.orc_sparse_mla.argtypes = [P, i64, i32, i32, P, i64, i64, i32, i64, P, i64, i32, P,
                                       i64, P, ctypes.c_double, P, P]
        lib.orc_varlen_windows.restype = i32
        lib.orc_varlen_windows.argtypes = [P, P, i32, i64, P]
        lib.orc_varlen_logits.restype = i32
        lib.orc_varlen_logits.argtypes = [i32, P, P, P, i32, i32, P, i64, i64, P, i64, i64, i32,
                                          i64, P, i64, P, P, i32, i64, P, i64, i64, P, P]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u8(a):
    return None if a is None else np.ascontiguousarray(a).view(np.uint8)


def threads() -> int:
    """OpenMP threads the oracle's row loops use."""
    return _load().orc_threads()


def dec_fp8(code: int) -> float:
    return _load().orc_dec_fp8_e4m3(code)


def dec_e2m1(nibble: int) -> float:
    return _load().orc_dec_e2m1(nibble)


def dec_e8m0(code: int) -> float:
    return _load().orc_dec_e8m0(code)


class Cache:
    """Host view of a paged K cache: byte pool + strides (all in bytes)."""

    def __init__(self, dtype, data, page_stride, row_stride, scale,
                 scale_page_stride, scale_row_stride, page_size, num_pages):
        self.dtype = dtype
        self.data = _u8(data)
        self.page_stride = int(page_stride)
        self.row_stride = int(row_stride)
        self.scale = _u8(scale)
        self.scale_page_stride = int(scale_page_stride)
        self.scale_row_stride = int(scale_row_stride)
        self.page_size = int(page_size)
        self.num_pages = int(num_pages)


def decode_logits(dtype, q, q_scale, w, H, D, cache: Cache, block_tables, lens,
                  next_n, rows, W):
    """Double-precision logits of the listed decode rows.

    Returns (logits [len(rows), W] float64 with -inf past each row's visible
    length, E [len(rows)] int64)."""
    lib = _load()
    q = _u8(q)
    qs = _u8(q_scale)
    w = np.ascontiguousarray(w, dtype=np.float32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((len(rows), W), dtype=np.float64)
    E = np.empty(len(rows), dtype=np.int64)
    rc = lib.orc_decode_logits(
        dtype, _ptr(q), _ptr(qs), _ptr(w), H, D, _ptr(cache.data),
        cache.page_stride, cache.row_stride, _ptr(cache.scale),
        cache.scale_page_stride, cache.scale_row_stride, cache.page_size,
        cache.num_pages, _ptr(bt), bt.shape[1], _ptr(lens), len(lens), next_n,
        _ptr(rows), len(rows), W, _ptr(out), _ptr(E))
    if rc != 0:
        raise ValueError("oracle decode_logits failed with code %d" % rc)
    return out, E


def prefill_logits(dtype, q, q_scale, w, H, D, cache: Cache, block_table,
                   visible_end, rows, W):
    """Double-precision logits of the listed prefill rows (one sequence)."""
    lib = _load()
    q = _u8(q)
    qs = _u8(q_scale)
    w = np.ascontiguousarray(w, dtype=np.float32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32).reshape(-1)
    ve = np.ascontiguousarray(visible_end, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((len(rows), W), dtype=np.float64)
    E = np.empty(len(rows), dtype=np.int64)
    rc = lib.orc_prefill_logits(
        dtype, _ptr(q), _ptr(qs), _ptr(w), H, D, _ptr(cache.data),
        cache.page_stride, cache.row_stride, _ptr(cache.scale),
        cache.scale_page_stride, cache.scale_row_stride, cache.page_size,
        cache.num_pages, _ptr(bt), _ptr(ve), len(ve), _ptr(rows), len(rows), W,
        _ptr(out), _ptr(E))
    if rc != 0:
        raise ValueError("oracle prefill_logits failed with code %d" % rc)
    return out, E


def topk(values, E, k):
    """Top-k token indices of one row (largest first, ties to lower index),
    padded with -1. float32 input is ordered as float32, float64 as float64."""
    lib = _load()
    out = np.empty(k, dtype=np.int32)
    if values.dtype == np.float32:
        v = np.ascontiguousarray(values)
        rc = lib.orc_topk_f32(_ptr(v), int(E), k, _ptr(out))
    else:
        v = np.ascontiguousarray(values, dtype=np.float64)
        rc = lib.orc_topk_f64(_ptr(v), int(E), k, _ptr(out))
    if rc != 0:
        raise ValueError("oracle topk failed with code %d" % rc)
    return out


def topk_rows_f32(logits, E, k):
    """Top-k of many float32 rows (row stride = logits.shape[1])."""
    lib = _load()
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    E = np.ascontiguousarray(E, dtype=np.int64)
    out = np.empty((lg.shape[0], k), dtype=np.int32)
    rc = lib.orc_topk_rows_f32(_ptr(lg), lg.shape[1], _ptr(E), lg.shape[0], k, _ptr(out))
    if rc != 0:
        raise ValueError("oracle topk_rows failed with code %d" % rc)
    return out


def enc_fp8(y: float) -> int:
    """Nearest E4M3FN code to the single-precision value y (ties to even)."""
    return int(_load().orc_enc_fp8_e4m3(float(y)))


def quant_fp8_row(x):
    """One row to (FP8 codes uint8 [D], fp32 scale) by the oracle's encoder."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(x.shape[0], dtype=np.uint8)
    scale = np.empty(1, dtype=np.float32)
    _load().orc_quant_fp8_row(_ptr(x), x.shape[0], _ptr(codes), _ptr(scale))
    return codes, float(scale[0])


def quant_mxfp4_row(x):
    """One row to (packed E2M1 uint8 [D/2], E8M0 scales uint8 [D/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    D = x.shape[0]
    packed = np.empty(D // 2, dtype=np.uint8)
    scales = np.empty(D // 32, dtype=np.uint8)
    _load().orc_quant_mxfp4_row(_ptr(x), D, _ptr(packed), _ptr(scales))
    return packed, scales


def kv_write(dtype, k, slot_mapping, cache: Cache):
    """Quantizes the rows of k (float32 [N, D]) into the cache image in place
    (cache.data / cache.scale are modified); rows with a negative slot or a
    page past the pool are skipped."""
    k = np.ascontiguousarray(k, dtype=np.float32)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    N, D = k.shape
    rc = _load().orc_kv_write(dtype, _ptr(k), D, N, D, _ptr(sm), cache.page_size,
                              cache.num_pages, _ptr(cache.data), cache.page_stride,
                              cache.row_stride, _ptr(cache.scale), cache.scale_page_stride,
                              cache.scale_row_stride)
    if rc != 0:
        raise ValueError("oracle kv_write failed with code %d" % rc)


def quantize_query(dtype, x, w, c=1.0, fold=True):
    """Query rows x (float32 [R, H, D]) and weights w (float32 [R, H]) to
    (q codes, q scales, weights): FP8 -> (uint8 [R,H,D], float32 [R] or None
    when folded, float32 [R,H]); MXFP4 -> (uint8 [R,H,D/2], uint8 [R,H,D/32],
    float32 [R,H])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    R, H, D = x.shape
    w_out = np.empty((R, H), dtype=np.float32)
    if dtype == FP8:
        q = np.empty((R, H, D), dtype=np.uint8)
        qs = None if fold else np.empty(R, dtype=np.float32)
    else:
        q = np.empty((R, H, D // 2), dtype=np.uint8)
        qs = np.empty((R, H, D // 32), dtype=np.uint8)
    rc = _load().orc_quantize_query(dtype, _ptr(x), H * D, R, H, D, _ptr(w), float(c),
                                    1 if (fold and dtype == FP8) else 0, _ptr(q), _ptr(qs),
                                    _ptr(w_out))
    if rc != 0:
        raise ValueError("oracle quantize_query failed with code %d" % rc)
    return q, qs, w_out


def varlen_windows(lens, row_offsets, R):
    """Visible ends (int64 [R]) of the packed rows of a ragged decode step."""
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    off = np.ascontiguousarray(row_offsets, dtype=np.int32)
    E = np.empty(R, dtype=np.int64)
    rc = _load().orc_varlen_windows(_ptr(lens), _ptr(off), len(lens), R, _ptr(E))
    if rc != 0:
        raise ValueError("oracle varlen_windows failed with code %d" % rc)
    return E


def varlen_logits(dtype, q, q_scale, w, H, D, cache: Cache, block_tables, lens, row_offsets,
                  R, rows, W):
    """Double-precision logits of the listed packed rows of a ragged decode
    step; returns (logits [len(rows), W], E [len(rows)])."""
    lib = _load()
    q = _u8(q)
    qs = _u8(q_scale)
    w = np.ascontiguousarray(w, dtype=np.float32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    off = np.ascontiguousarray(row_offsets, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((len(rows), W), dtype=np.float64)
    E = np.empty(len(rows), dtype=np.int64)
    rc = lib.orc_varlen_logits(
        dtype, _ptr(q), _ptr(qs), _ptr(w), H, D, _ptr(cache.data), cache.page_stride,
        cache.row_stride, _ptr(cache.scale), cache.scale_page_stride, cache.scale_row_stride,
        cache.page_size, cache.num_pages, _ptr(bt), bt.shape[1], _ptr(lens), _ptr(off),
        len(lens), R, _ptr(rows), len(rows), W, _ptr(out), _ptr(E))
    if rc != 0:
        raise ValueError("oracle varlen_logits failed with code %d" % rc)
    return out, E


def sparse_mla(q, cache_data, page_stride, row_stride, page_size, num_pages, block_tables,
               next_n, indices, topk_lens, scale):
    """Sparse attention of bf16 query rows q (uint16 bits [R, H, D]) over the
    selected latent rows of a bf16 paged cache (uint8 bytes). Returns
    (out float64 [R, H, D], lse float64 [R, H])."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    R, H, D = q.shape
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    lens = np.ascontiguousarray(topk_lens, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    data = np.ascontiguousarray(cache_data).view(np.uint8)
    out = np.empty((R, H, D), dtype=np.float64)
    lse = np.empty((R, H), dtype=np.float64)
    rc = _load().orc_sparse_mla(_ptr(q), R, H, D, _ptr(data), page_stride, row_stride, page_size,
                                num_pages, _ptr(bt), bt.shape[1], next_n, _ptr(idx),
                                idx.shape[1], _ptr(lens), float(scale), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle sparse_mla failed with code %d" % rc)
    return out, lse
