"""CPU oracle for GGUF block-quantized matmul with q8_1 activations -- TEST INFRASTRUCTURE.

Only tests/, the smoke check and bench.py's cpu_baseline leg may import this package.  The
product library (block_quantized_matmul_quantize_amd) never imports, links or falls back to it.

Thin ctypes marshalling over qmm_oracle.c; every step of the arithmetic lives in that C file,
which states the readings of the pages it follows.  numpy arrays in, numpy arrays out.
"""
import ctypes
import os

import numpy as np

from . import build as _build

Q4_0 = 2
Q8_0 = 8
Q3_K = 11
Q4_K = 12
Q5_K = 13
Q6_K = 14
IQ4_XS = 23

BLOCK_VALUES = {Q4_0: 32, Q8_0: 32, Q3_K: 256, Q4_K: 256, Q5_K: 256, Q6_K: 256, IQ4_XS: 256}
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34, Q3_K: 110, Q4_K: 144, Q5_K: 176, Q6_K: 210, IQ4_XS: 136}
Q8_1_BYTES = 36

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        L = ctypes.CDLL(path)
        i64, i32, u16 = ctypes.c_int64, ctypes.c_int, ctypes.c_uint16
        vp = ctypes.c_void_p
        L.oracle_half_to_double.argtypes = [u16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_float_to_half.argtypes = [ctypes.c_float]
        L.oracle_float_to_half.restype = u16
        L.oracle_quantize_q8_1.argtypes = [vp, i64, i64, vp]
        L.oracle_quantize_q8_1.restype = None
        L.oracle_row_bytes.argtypes = [i32, i64]
        L.oracle_row_bytes.restype = i64
        L.oracle_subdots_per_row.argtypes = [i32, i64]
        L.oracle_subdots_per_row.restype = i64
        L.oracle_dequantize.argtypes = [i32, vp, i64, i64, vp]
        L.oracle_dequantize.restype = i32
        L.oracle_dequantize_q8_1.argtypes = [vp, i64, i64, vp, vp, vp]
        L.oracle_dequantize_q8_1.restype = None
        L.oracle_matmul_q8_1.argtypes = [i32, vp, i64, i64, vp, i64, vp]
        L.oracle_matmul_q8_1.restype = i32
        L.oracle_matmul_q8_1_at.argtypes = [i32, vp, i64, i64, vp, i64, vp, vp, i64, vp]
        L.oracle_matmul_q8_1_at.restype = i32
        L.oracle_subdots.argtypes = [i32, vp, i64, i64, vp, i64, vp]
        L.oracle_subdots.restype = i32
        L.oracle_subdots_q6_K_folded.argtypes = [vp, i64, i64, vp, i64, vp]
        L.oracle_subdots_q6_K_folded.restype = i32
        L.oracle_subdots_q3_K_folded.argtypes = [vp, i64, i64, vp, i64, vp]
        L.oracle_subdots_q3_K_folded.restype = i32
        L.oracle_matmul.argtypes = [i32, vp, i64, i64, vp, i64, vp]
        L.oracle_matmul.restype = i32
        L.oracle_matmul_id.argtypes = [i32, vp, i64, i64, i64, vp, i64, vp, i64, i64, vp, vp]
        L.oracle_matmul_id.restype = i32
        L.oracle_matmul_glu.argtypes = [i32, vp, vp, i64, i64, vp, i64, vp]
        L.oracle_matmul_glu.restype = i32
        L.oracle_matmul_id_glu.argtypes = [i32, vp, vp, i64, i64, i64, vp, vp, i64, i64, vp, vp]
        L.oracle_matmul_id_glu.restype = i32
        L.oracle_f16act_encode.argtypes = [vp, i64, i64, vp, vp, vp]
        L.oracle_f16act_encode.restype = i32
        L.oracle_matmul_f16act.argtypes = [i32, vp, i64, i64, vp, i64, vp]
        L.oracle_matmul_f16act.restype = i32
        L.oracle_panel_bytes.argtypes = [i32, i64, i64]
        L.oracle_panel_bytes.restype = i64
        L.oracle_panel_offset.argtypes = [i32, i32, i32]
        L.oracle_panel_offset.restype = i64
        L.oracle_repack_panels.argtypes = [i32, vp, i64, i64, vp]
        L.oracle_repack_panels.restype = i32
        L.oracle_dequantize_panels.argtypes = [i32, vp, i64, i64, vp]
        L.oracle_dequantize_panels.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def row_bytes(qtype, k):
    return int(lib().oracle_row_bytes(qtype, k))


def half_to_double(bits):
    return float(lib().oracle_half_to_double(int(bits) & 0xFFFF))


def float_to_half(x):
    return int(lib().oracle_float_to_half(float(np.float32(x))))


def quantize_q8_1(x):
    """fp32 [n, k] -> uint8 [n, k/32*36] canonical q8_1 blocks."""
    x = _c(x, np.float32)
    n, k = x.shape
    assert k % 32 == 0
    y = np.zeros((n, k // 32 * Q8_1_BYTES), dtype=np.uint8)
    lib().oracle_quantize_q8_1(_ptr(x), n, k, _ptr(y))
    return y


def dequantize(qtype, w, rows, k):
    w = _c(w, np.uint8)
    out = np.zeros((rows, k), dtype=np.float64)
    rc = lib().oracle_dequantize(qtype, _ptr(w), rows, k, _ptr(out))
    if rc:
        raise ValueError("oracle_dequantize: bad arguments")
    return out


def dequantize_q8_1(xq, n, k):
    """q8_1 blocks -> (values d*q fp64 [n,k], d [n,k/32], s [n,k/32])."""
    xq = _c(xq, np.uint8)
    out = np.zeros((n, k), dtype=np.float64)
    d = np.zeros((n, k // 32), dtype=np.float64)
    s = np.zeros((n, k // 32), dtype=np.float64)
    lib().oracle_dequantize_q8_1(_ptr(xq), n, k, _ptr(out), _ptr(d), _ptr(s))
    return out, d, s


def matmul_q8_1(qtype, w, rows, k, xq, n):
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    y = np.zeros((n, rows), dtype=np.float32)
    rc = lib().oracle_matmul_q8_1(qtype, _ptr(w), rows, k, _ptr(xq), n, _ptr(y))
    if rc:
        raise ValueError("oracle_matmul_q8_1: bad arguments")
    return y


def matmul_q8_1_at(qtype, w, rows, k, xq, n, cols, rws):
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    cols = _c(cols, np.int64)
    rws = _c(rws, np.int64)
    out = np.zeros(cols.shape[0], dtype=np.float32)
    rc = lib().oracle_matmul_q8_1_at(qtype, _ptr(w), rows, k, _ptr(xq), n, _ptr(cols), _ptr(rws),
                                     cols.shape[0], _ptr(out))
    if rc:
        raise ValueError("oracle_matmul_q8_1_at: bad arguments")
    return out


def subdots(qtype, w, rows, k, xq, n):
    """Integer sub-block dots, int32 [n, rows, k/32] (Q6_K: [n, rows, k/16])."""
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    per = int(lib().oracle_subdots_per_row(qtype, k))
    D = np.zeros((n, rows, per), dtype=np.int32)
    rc = lib().oracle_subdots(qtype, _ptr(w), rows, k, _ptr(xq), n, _ptr(D))
    if rc:
        raise ValueError("oracle_subdots: bad arguments")
    return D


def subdots_q6_K_folded(w, rows, k, xq, n):
    """Q6_K: sc0*D0 + sc1*D1 per 32-value block, int32 [n, rows, k/32]."""
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    F = np.zeros((n, rows, k // 32), dtype=np.int32)
    rc = lib().oracle_subdots_q6_K_folded(_ptr(w), rows, k, _ptr(xq), n, _ptr(F))
    if rc:
        raise ValueError("oracle_subdots_q6_K_folded: bad arguments")
    return F


def subdots_q3_K_folded(w, rows, k, xq, n):
    """Q3_K: sc0*D0 + sc1*D1 per 32-value block (sc = 6-bit scale - 32), int32 [n, rows, k/32]."""
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    F = np.zeros((n, rows, k // 32), dtype=np.int32)
    rc = lib().oracle_subdots_q3_K_folded(_ptr(w), rows, k, _ptr(xq), n, _ptr(F))
    if rc:
        raise ValueError("oracle_subdots_q3_K_folded: bad arguments")
    return F


def matmul(qtype, w, rows, k, x):
    w = _c(w, np.uint8)
    x = _c(x, np.float32)
    n = x.shape[0]
    y = np.zeros((n, rows), dtype=np.float32)
    rc = lib().oracle_matmul(qtype, _ptr(w), rows, k, _ptr(x), n, _ptr(y))
    if rc:
        raise ValueError("oracle_matmul: bad arguments")
    return y


def matmul_id(qtype, w, n_exp, rows, k, x, x_per_tok, ids, fill=np.nan):
    """Expert-indexed product; returns (y [n_tok, top_k, rows], n_invalid).  Rows of y whose id is
    out of range keep `fill`."""
    w = _c(w, np.uint8)
    x = _c(x, np.float32)
    ids = _c(ids, np.int32)
    n_tok, top_k = ids.shape
    y = np.full((n_tok, top_k, rows), fill, dtype=np.float32)
    bad = ctypes.c_int64(0)
    rc = lib().oracle_matmul_id(qtype, _ptr(w), n_exp, rows, k, _ptr(x), x_per_tok, _ptr(ids), n_tok,
                                top_k, _ptr(y), ctypes.byref(bad))
    if rc:
        raise ValueError("oracle_matmul_id: bad arguments")
    return y, int(bad.value)


def matmul_glu(qtype, w_gate, w_up, rows, k, x):
    """silu(W_gate x) * (W_up x) -> y [n, rows] (fp32)."""
    w_gate = _c(w_gate, np.uint8)
    w_up = _c(w_up, np.uint8)
    x = _c(x, np.float32)
    n = x.shape[0]
    y = np.zeros((n, rows), dtype=np.float32)
    rc = lib().oracle_matmul_glu(qtype, _ptr(w_gate), _ptr(w_up), rows, k, _ptr(x), n, _ptr(y))
    if rc:
        raise ValueError("oracle_matmul_glu: bad arguments")
    return y


def matmul_id_glu(qtype, w_gate, w_up, n_exp, rows, k, x, ids, fill=np.nan):
    """Expert form of matmul_glu (one activation row per token); returns (y [n_tok, top_k, rows],
    n_invalid).  Rows of y whose id is out of range keep `fill`."""
    w_gate = _c(w_gate, np.uint8)
    w_up = _c(w_up, np.uint8)
    x = _c(x, np.float32)
    ids = _c(ids, np.int32)
    n_tok, top_k = ids.shape
    y = np.full((n_tok, top_k, rows), fill, dtype=np.float32)
    bad = ctypes.c_int64(0)
    rc = lib().oracle_matmul_id_glu(qtype, _ptr(w_gate), _ptr(w_up), n_exp, rows, k, _ptr(x), _ptr(ids), n_tok,
                                    top_k, _ptr(y), ctypes.byref(bad))
    if rc:
        raise ValueError("oracle_matmul_id_glu: bad arguments")
    return y, int(bad.value)


def f16act_encode(x):
    """fp16-activation mode encoder: x fp32 [n, k] -> (fp16 bit patterns uint16 [n, k], prescale
    exponents e int32 [n, k/32], exact block sums of the fp16 values fp64 [n, k/32])."""
    x = _c(x, np.float32)
    n, k = x.shape
    y = np.zeros((n, k), dtype=np.uint16)
    e = np.zeros((n, k // 32), dtype=np.int32)
    s = np.zeros((n, k // 32), dtype=np.float64)
    if lib().oracle_f16act_encode(_ptr(x), n, k, _ptr(y), _ptr(e), _ptr(s)):
        raise ValueError("oracle_f16act_encode: bad arguments")
    return y, e, s


def matmul_f16act(qtype, w, rows, k, x):
    """fp16-activation mode product W . x -> y [n, rows] (fp32)."""
    w = _c(w, np.uint8)
    x = _c(x, np.float32)
    n = x.shape[0]
    y = np.zeros((n, rows), dtype=np.float32)
    if lib().oracle_matmul_f16act(qtype, _ptr(w), rows, k, _ptr(x), n, _ptr(y)):
        raise ValueError("oracle_matmul_f16act: bad arguments")
    return y


def panel_bytes(qtype, rows, k):
    """Bytes of the panel layout of a [rows, k] matrix (-1: type or shape not supported)."""
    return int(lib().oracle_panel_bytes(qtype, rows, k))


def panel_offset(qtype, i, o):
    """Offset inside a panel of byte o of row i's 256-value step (-1: out of range)."""
    return int(lib().oracle_panel_offset(qtype, i, o))


def repack_panels(qtype, w, rows, k):
    """Original blocks [rows, row_bytes] -> panel layout (uint8, flat)."""
    w = _c(w, np.uint8)
    nb = panel_bytes(qtype, rows, k)
    if nb < 0:
        raise ValueError("repack_panels: type or shape not supported")
    out = np.zeros(nb, dtype=np.uint8)
    if lib().oracle_repack_panels(qtype, _ptr(w), rows, k, _ptr(out)):
        raise ValueError("oracle_repack_panels: bad arguments")
    return out


def dequantize_panels(qtype, wp, rows, k):
    """Panel layout -> fp64 values [rows, k]."""
    wp = _c(wp, np.uint8)
    out = np.zeros((rows, k), dtype=np.float64)
    if lib().oracle_dequantize_panels(qtype, _ptr(wp), rows, k, _ptr(out)):
        raise ValueError("oracle_dequantize_panels: bad arguments")
    return out
