"""Python binding of libqmm: GGUF block-quantized (Q4_K / Q5_K / Q6_K / Q8_0 / Q4_0 / Q3_K / IQ4_XS) x q8_1
matmul on MI355X.

Thin ctypes marshalling over the C ABI declared in include/qmm.h; every computation runs in the
library's HIP kernels.  Function names follow the C entry points without the ``qmm_`` prefix.
Tensors are torch tensors on a ROCm device; calls are enqueued on torch's current stream.
There is no CPU fallback: if libqmm.so is missing, importing this package raises.
"""
import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "qmm.h")

Q4_0 = 2
Q8_0 = 8
Q4_K = 12
Q5_K = 13
Q6_K = 14
Q3_K = 11
IQ4_XS = 23
BLOCK_VALUES = {Q4_0: 32, Q8_0: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256, Q3_K: 256, IQ4_XS: 256}
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34, Q4_K: 144, Q5_K: 176, Q6_K: 210, Q3_K: 110, IQ4_XS: 136}
Q8_1_BYTES = 36

OVR_PATH, OVR_STREAMK, OVR_TILE_J, OVR_MV_STEPS, OVR_MV_KERNEL, OVR_FUSE_COLS = 1, 2, 3, 4, 5, 6
PATH_AUTO, PATH_MATVEC, PATH_TILED = 0, 1, 2

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m block_quantized_matmul_quantize_amd.build`")

# torch ships its own HIP runtime with the same soname as the system one; loading torch first
# makes libqmm bind to that already-loaded runtime, so one HIP runtime owns the device.
import torch  # noqa: E402,F401

_L = ctypes.CDLL(LIB_PATH)
_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t


class Plan(ctypes.Structure):
    _fields_ = [("regime", ctypes.c_int32), ("tile_i", ctypes.c_int32), ("tile_j", ctypes.c_int32),
                ("ntiles", ctypes.c_int64), ("efficiency_pct", ctypes.c_int32), ("stream_k", ctypes.c_int32),
                ("k_iters", ctypes.c_int64), ("units", ctypes.c_int64), ("fixup", ctypes.c_int32),
                ("ws_bytes", ctypes.c_uint64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


def _sig(name, res, *args):
    fn = getattr(_L, name)
    fn.restype = res
    fn.argtypes = list(args)
    return fn


_sig("qmm_last_error", ctypes.c_char_p)
_sig("qmm_version", ctypes.c_char_p)
_sig("qmm_quantize_q8_1", _i32, _vp, _i64, _i64, _vp, _vp)
_sig("qmm_matmul_workspace", _sz, _i32, _i64, _i64, _i64)
_sig("qmm_encode_f16act", _i32, _vp, _i64, _i64, _vp, _vp, _vp, _vp)
_sig("qmm_matmul_f16act_workspace", _sz, _i64, _i64)
_sig("qmm_matmul_f16act", _i32, _i32, _vp, _i64, _i64, _vp, _i64, _vp, _vp, _sz, _vp)
_sig("qmm_matmul", _i32, _i32, _vp, _i64, _i64, _vp, _i64, _vp, _vp, _sz, _vp)
_sig("qmm_matmul_noalloc", _i32, _i32, _vp, _i64, _i64, _vp, _i64, _vp, _vp)
_sig("qmm_repack_bytes", ctypes.c_uint64, _i32, _i64, _i64)
_sig("qmm_repack", _i32, _i32, _vp, _i64, _i64, _vp, ctypes.c_uint64, _vp)
_sig("qmm_matmul_packed_workspace", _sz, _i32, _i64, _i64, _i64)
_sig("qmm_matmul_packed", _i32, _i32, _vp, _i64, _i64, _vp, _i64, _vp, _vp, _sz, _vp)
_sig("qmm_matmul_q8_1_workspace", _sz, _i32, _i64, _i64, _i64)
_sig("qmm_matmul_q8_1", _i32, _i32, _vp, _i64, _i64, _vp, _i64, _vp, _vp, _sz, _vp)
_sig("qmm_matmul_id_workspace", _sz, _i32, _i64, _i64, _i64, _i64, _i64, _i64)
_sig("qmm_matmul_id", _i32, _i32, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _vp, _sz, _vp)
_sig("qmm_matmul_id_invalid_count", _i32, _vp, ctypes.POINTER(_i64), _vp)
_sig("qmm_matmul_glu_workspace", _sz, _i32, _i64, _i64, _i64)
_sig("qmm_matmul_glu", _i32, _i32, _vp, _vp, _i64, _i64, _vp, _i64, _vp, _vp, _sz, _vp)
_sig("qmm_matmul_id_glu_workspace", _sz, _i32, _i64, _i64, _i64, _i64, _i64)
_sig("qmm_matmul_id_glu", _i32, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _vp, _sz, _vp)
_sig("qmm_matmul_id_grouping_layout", _i32, _i32, _i64, _i64, _i64, _i64, _i64, ctypes.POINTER(_i64))
_sig("qmm_debug_subdots_workspace", _sz, _i32, _i64, _i64, _i64, _i32)
_sig("qmm_debug_subdots", _i32, _i32, _vp, _i64, _i64, _vp, _i64, _i32, _vp, _vp, _sz, _vp)
_sig("qmm_set_override", _i32, _i32, _i32)
_sig("qmm_plan_dense", _i32, _i32, _i64, _i64, _i64, ctypes.c_int32, ctypes.POINTER(Plan))
_sig("qmm_tile_efficiency", ctypes.c_int32, _i64, ctypes.c_int32)
_sig("qmm_select_tile_j", ctypes.c_int32, _i64)
_sig("qmm_streamk_unit_start", _i64, _i64, _i64, _i64, _i64)
_sig("qmm_matvec_kernel", _i32, _i32, _vp, _i64, _i64, _vp, _i64, _i32, ctypes.POINTER(_i32))


class QmmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"qmm status {status}: {msg}")
        self.status = status


def _check(st):
    if st != 0:
        raise QmmError(st, _L.qmm_last_error().decode())


def lib():
    return _L


def header_symbols():
    """Entry points declared in include/qmm.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(qmm_[a-z0-9_]+)\s*\(", text)))


def version():
    return _L.qmm_version().decode()


# --------------------------------------------------------------------------------------------
# Host-side planner (no GPU needed)
# --------------------------------------------------------------------------------------------
def set_override(key, value):
    _check(_L.qmm_set_override(key, value))


def plan_dense(qtype, rows, k, n, nsm=256):
    p = Plan()
    _check(_L.qmm_plan_dense(qtype, rows, k, n, nsm, ctypes.byref(p)))
    return p.as_dict()


def tile_efficiency(ntiles, nsm):
    return int(_L.qmm_tile_efficiency(ntiles, nsm))


def select_tile_j(ncols):
    return int(_L.qmm_select_tile_j(ncols))


def streamk_unit_start(u, units, ntiles, k_iters):
    return int(_L.qmm_streamk_unit_start(u, units, ntiles, k_iters))


MV_KERNEL_NAMES = {1: "mmvq_kernel", 2: "mmvq_stream_kernel", 3: "mmvq_dot4_kernel"}


def matvec_kernel(qtype, w_ptr, rows, k, x_ptr, n, x_fp32=True):
    """(kernel id, fused) a dense call would launch: 0 tiled path, 1 register-streamed, 2
    LDS-staged MFMA, 3 dot4; fused = the kernel quantizes the fp32 activations itself.  Takes
    raw addresses (ints) or tensors; only their alignment matters."""
    w_ptr = w_ptr.data_ptr() if hasattr(w_ptr, "data_ptr") else int(w_ptr)
    x_ptr = x_ptr.data_ptr() if hasattr(x_ptr, "data_ptr") else int(x_ptr)
    out = _i32(0)
    _check(_L.qmm_matvec_kernel(qtype, w_ptr, rows, k, x_ptr, n, 1 if x_fp32 else 0, ctypes.byref(out)))
    return out.value & 15, bool(out.value & 16)


def matmul_workspace(qtype, rows, k, n):
    return int(_L.qmm_matmul_workspace(qtype, rows, k, n))


def matmul_q8_1_workspace(qtype, rows, k, n):
    return int(_L.qmm_matmul_q8_1_workspace(qtype, rows, k, n))


def matmul_id_workspace(qtype, n_exp, rows, k, n_tok, top_k, x_per_tok):
    return int(_L.qmm_matmul_id_workspace(qtype, n_exp, rows, k, n_tok, top_k, x_per_tok))


def matmul_glu_workspace(qtype, rows, k, n):
    return int(_L.qmm_matmul_glu_workspace(qtype, rows, k, n))


def matmul_id_glu_workspace(qtype, n_exp, rows, k, n_tok, top_k):
    return int(_L.qmm_matmul_id_glu_workspace(qtype, n_exp, rows, k, n_tok, top_k))


# --------------------------------------------------------------------------------------------
# Device entry points (torch tensors)
# --------------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _need(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _on_device(**tensors):
    """Last check before a pointer crosses the C ABI: every tensor lives in device memory."""
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


def weight_bytes(qtype, rows, k):
    """Bytes of a [rows][k] weight matrix of GGUF blocks (ValueError for an unknown type or a k
    that is not a multiple of the block size)."""
    if qtype not in BLOCK_VALUES:
        raise ValueError(f"unsupported weight type {qtype}")
    if k <= 0 or k % BLOCK_VALUES[qtype]:
        raise ValueError(f"k={k} is not a positive multiple of the block size {BLOCK_VALUES[qtype]}")
    return rows * (k // BLOCK_VALUES[qtype]) * BLOCK_BYTES[qtype]


def _need_size(t, nbytes, name):
    """The C ABI receives bare pointers, so a tensor smaller than the shape it stands for would be
    read or written past its end on the device: refuse it here."""
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, the call needs {nbytes}")


def _need_weights(t, qtype, rows, k, name, n_mat=1):
    """Size check of a weight tensor; an unknown type or a k the type cannot take is left to the
    library, which reports it as QMM_ERR_TYPE / QMM_ERR_SHAPE (QmmError)."""
    if qtype in BLOCK_VALUES and k > 0 and k % BLOCK_VALUES[qtype] == 0 and rows > 0:
        _need_size(t, n_mat * weight_bytes(qtype, rows, k), name)


def _workspace(nbytes, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def quantize_q8_1(x, out=None):
    """fp32 [n, k] -> uint8 [n, k/32*36] q8_1 blocks."""
    torch = _torch()
    px = _need(x, torch.float32, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [n, k]")
    n, k = x.shape
    if out is None:
        out = torch.empty((n, (k // 32) * Q8_1_BYTES), dtype=torch.uint8, device=x.device)
    py = _need(out, torch.uint8, "out")
    _need_size(out, n * (k // 32) * Q8_1_BYTES, "out")
    _on_device(x=x, out=out)
    _check(_L.qmm_quantize_q8_1(px, n, k, py, _stream()))
    return out


def matmul(w, qtype, rows, k, x, out=None, ws=None):
    """Y[n, rows] = W[rows, k] . X[n, k]^T with X quantized to q8_1 on the way."""
    torch = _torch()
    pw = _need(w, torch.uint8, "w")
    px = _need(x, torch.float32, "x")
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [n, {k}]")
    n = x.shape[0]
    _need_weights(w, qtype, rows, k, "w")
    if out is None:
        out = torch.empty((n, rows), dtype=torch.float32, device=x.device)
    py = _need(out, torch.float32, "out")
    _need_size(out, n * rows * 4, "out")
    nbytes = matmul_workspace(qtype, rows, k, n)
    if ws is None:
        ws = _workspace(nbytes, x.device)
    _on_device(w=w, x=x, out=out, ws=ws)
    _check(_L.qmm_matmul(qtype, pw, rows, k, px, n, py, ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream()))
    return out


def repack_bytes(qtype, rows, k):
    """Bytes of the panel layout of a [rows, k] matrix (0: type or shape not supported)."""
    return int(_L.qmm_repack_bytes(qtype, rows, k))


def repack(w, qtype, rows, k, out=None):
    """One-time repack of original blocks w into the panel layout (uint8 tensor on w's device)."""
    torch = _torch()
    pw = _need(w, torch.uint8, "w")
    _need_weights(w, qtype, rows, k, "w")
    nb = repack_bytes(qtype, rows, k)
    if out is None:
        out = torch.empty(max(nb, 16), dtype=torch.uint8, device=w.device)
    pp = _need(out, torch.uint8, "out")
    _on_device(w=w, out=out)
    _check(_L.qmm_repack(qtype, pw, rows, k, pp, out.numel(), _stream()))
    return out


def matmul_packed_workspace(qtype, rows, k, n):
    return int(_L.qmm_matmul_packed_workspace(qtype, rows, k, n))


def matmul_packed(wp, qtype, rows, k, x, out=None, ws=None):
    """matmul with the weights in the panel layout (from repack)."""
    torch = _torch()
    pw = _need(wp, torch.uint8, "wp")
    px = _need(x, torch.float32, "x")
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [n, {k}]")
    n = x.shape[0]
    need = repack_bytes(qtype, rows, k)
    if need:
        _need_size(wp, need, "wp")
    if out is None:
        out = torch.empty((n, rows), dtype=torch.float32, device=x.device)
    py = _need(out, torch.float32, "out")
    _need_size(out, n * rows * 4, "out")
    nbytes = matmul_packed_workspace(qtype, rows, k, n)
    if ws is None:
        ws = _workspace(nbytes, x.device)
    _on_device(wp=wp, x=x, out=out, ws=ws)
    _check(_L.qmm_matmul_packed(qtype, pw, rows, k, px, n, py, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                _stream()))
    return out


def matmul_noalloc(w, qtype, rows, k, x, out=None):
    """matmul without a workspace argument: the library's own per-GPU scratch buffer holds it (the
    call allocates nothing itself, apart from `out` when it is not given)."""
    torch = _torch()
    pw = _need(w, torch.uint8, "w")
    px = _need(x, torch.float32, "x")
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [n, {k}]")
    n = x.shape[0]
    _need_weights(w, qtype, rows, k, "w")
    if out is None:
        out = torch.empty((n, rows), dtype=torch.float32, device=x.device)
    py = _need(out, torch.float32, "out")
    _need_size(out, n * rows * 4, "out")
    _on_device(w=w, x=x, out=out)
    _check(_L.qmm_matmul_noalloc(qtype, pw, rows, k, px, n, py, _stream()))
    return out


def encode_f16act(x):
    """fp16-activation mode encoder: fp32 [n, k] -> (fp16 bit patterns int16 [n, k], prescale
    exponents int32 [n, k/32], fp32 block sums [n, k/32])."""
    torch = _torch()
    px = _need(x, torch.float32, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [n, k]")
    n, k = x.shape
    y16 = torch.empty((n, k), dtype=torch.int16, device=x.device)
    e = torch.empty((n, k // 32), dtype=torch.int32, device=x.device)
    s = torch.empty((n, k // 32), dtype=torch.float32, device=x.device)
    _on_device(x=x)
    _check(_L.qmm_encode_f16act(px, n, k, ctypes.c_void_p(y16.data_ptr()), ctypes.c_void_p(e.data_ptr()),
                                ctypes.c_void_p(s.data_ptr()), _stream()))
    return y16, e, s


def matmul_f16act_workspace(k, n):
    return _L.qmm_matmul_f16act_workspace(k, n)


def matmul_f16act(w, qtype, rows, k, x, out=None, ws=None):
    """Y[n, rows] = W[rows, k] . X[n, k]^T in the fp16-activation mode (n <= 8)."""
    torch = _torch()
    pw = _need(w, torch.uint8, "w")
    px = _need(x, torch.float32, "x")
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [n, {k}]")
    n = x.shape[0]
    _need_weights(w, qtype, rows, k, "w")
    if out is None:
        out = torch.empty((n, rows), dtype=torch.float32, device=x.device)
    py = _need(out, torch.float32, "out")
    _need_size(out, n * rows * 4, "out")
    if ws is None:
        ws = _workspace(matmul_f16act_workspace(k, n), x.device)
    _on_device(w=w, x=x, out=out, ws=ws)
    _check(_L.qmm_matmul_f16act(qtype, pw, rows, k, px, n, py, ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream()))
    return out


def matmul_q8_1(w, qtype, rows, k, xq, n, out=None, ws=None):
    """Same product from q8_1 activations (uint8 [n, k/32*36])."""
    torch = _torch()
    pw = _need(w, torch.uint8, "w")
    px = _need(xq, torch.uint8, "xq")
    if xq.numel() != n * (k // 32) * Q8_1_BYTES:
        raise ValueError("xq has the wrong number of bytes")
    _need_weights(w, qtype, rows, k, "w")
    if out is None:
        out = torch.empty((n, rows), dtype=torch.float32, device=xq.device)
    py = _need(out, torch.float32, "out")
    _need_size(out, n * rows * 4, "out")
    nbytes = matmul_q8_1_workspace(qtype, rows, k, n)
    if ws is None:
        ws = _workspace(nbytes, xq.device)
    _on_device(w=w, xq=xq, out=out, ws=ws)
    _check(_L.qmm_matmul_q8_1(qtype, pw, rows, k, px, n, py, ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream()))
    return out


def matmul_id(w, qtype, n_exp, rows, k, x, ids, x_per_tok=1, out=None, ws=None):
    """Expert-indexed product.  x: fp32 [n_tok*x_per_tok, k]; ids: int32 [n_tok, top_k];
    returns y fp32 [n_tok, top_k, rows] (rows with an invalid id are left as they were in `out`)."""
    torch = _torch()
    pw = _need(w, torch.uint8, "w")
    px = _need(x, torch.float32, "x")
    pi = _need(ids, torch.int32, "ids")
    if ids.dim() != 2:
        raise ValueError("ids must be 2-D [n_tok, top_k]")
    n_tok, top_k = ids.shape
    if x.shape != (n_tok * x_per_tok, k):
        raise ValueError(f"x must be [{n_tok * x_per_tok}, {k}]")
    _need_weights(w, qtype, rows, k, "w", n_exp)
    if out is None:
        out = torch.zeros((n_tok, top_k, rows), dtype=torch.float32, device=x.device)
    py = _need(out, torch.float32, "out")
    _need_size(out, n_tok * top_k * rows * 4, "out")
    nbytes = matmul_id_workspace(qtype, n_exp, rows, k, n_tok, top_k, x_per_tok)
    if ws is None:
        ws = _workspace(nbytes, x.device)
    _on_device(w=w, x=x, ids=ids, out=out, ws=ws)
    _check(_L.qmm_matmul_id(qtype, pw, n_exp, rows, k, px, x_per_tok, pi, n_tok, top_k, py,
                            ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream()))
    return out, ws


def matmul_glu(w_gate, w_up, qtype, rows, k, x, out=None, ws=None):
    """Y[n, rows] = silu(W_gate . X^T) * (W_up . X^T), both products of X quantized to q8_1 once."""
    torch = _torch()
    pg = _need(w_gate, torch.uint8, "w_gate")
    pu = _need(w_up, torch.uint8, "w_up")
    if w_gate.numel() != w_up.numel():
        raise ValueError("w_gate and w_up must have the same size")
    _need_weights(w_gate, qtype, rows, k, "w_gate")
    px = _need(x, torch.float32, "x")
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [n, {k}]")
    n = x.shape[0]
    if out is None:
        out = torch.empty((n, rows), dtype=torch.float32, device=x.device)
    py = _need(out, torch.float32, "out")
    _need_size(out, n * rows * 4, "out")
    if ws is None:
        ws = _workspace(matmul_glu_workspace(qtype, rows, k, n), x.device)
    _on_device(w_gate=w_gate, w_up=w_up, x=x, out=out, ws=ws)
    _check(_L.qmm_matmul_glu(qtype, pg, pu, rows, k, px, n, py, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                             _stream()))
    return out


def matmul_id_glu(w_gate, w_up, qtype, n_exp, rows, k, x, ids, out=None, ws=None):
    """Expert form of matmul_glu.  x: fp32 [n_tok, k]; ids: int32 [n_tok, top_k]; returns
    (y fp32 [n_tok, top_k, rows], ws) -- rows with an invalid id keep their value in `out`."""
    torch = _torch()
    pg = _need(w_gate, torch.uint8, "w_gate")
    pu = _need(w_up, torch.uint8, "w_up")
    if w_gate.numel() != w_up.numel():
        raise ValueError("w_gate and w_up must have the same size")
    _need_weights(w_gate, qtype, rows, k, "w_gate", n_exp)
    px = _need(x, torch.float32, "x")
    pi = _need(ids, torch.int32, "ids")
    if ids.dim() != 2:
        raise ValueError("ids must be 2-D [n_tok, top_k]")
    n_tok, top_k = ids.shape
    if x.shape != (n_tok, k):
        raise ValueError(f"x must be [{n_tok}, {k}]")
    if out is None:
        out = torch.zeros((n_tok, top_k, rows), dtype=torch.float32, device=x.device)
    py = _need(out, torch.float32, "out")
    _need_size(out, n_tok * top_k * rows * 4, "out")
    if ws is None:
        ws = _workspace(matmul_id_glu_workspace(qtype, n_exp, rows, k, n_tok, top_k), x.device)
    _on_device(w_gate=w_gate, w_up=w_up, x=x, ids=ids, out=out, ws=ws)
    _check(_L.qmm_matmul_id_glu(qtype, pg, pu, n_exp, rows, k, px, pi, n_tok, top_k, py,
                                ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream()))
    return out, ws


def matmul_id_invalid_count(ws):
    v = _i64(0)
    _check(_L.qmm_matmul_id_invalid_count(ctypes.c_void_p(ws.data_ptr()), ctypes.byref(v), _stream()))
    return int(v.value)


def matmul_id_layout(qtype, n_exp, k, n_tok, top_k, x_per_tok=1):
    """Host logic only: workspace byte offsets of the expert grouping (sorted, bounds, tile_start,
    small), the column-tile width and the small-expert limit a matmul_id of this shape uses."""
    out = (_i64 * 6)()
    _check(_L.qmm_matmul_id_grouping_layout(qtype, n_exp, k, n_tok, top_k, x_per_tok, out))
    return tuple(int(v) for v in out)


def matmul_id_grouping(ws, qtype, n_exp, k, n_tok, top_k, x_per_tok=1):
    """Expert grouping the last matmul_id with workspace `ws` built (synchronizes the stream):
    dict of int32 CPU tensors sorted, bounds, tile_start, small, plus tile_j and small_max."""
    torch = _torch()
    out = matmul_id_layout(qtype, n_exp, k, n_tok, top_k, x_per_tok)
    torch.cuda.current_stream().synchronize()
    pairs = n_tok * top_k
    raw = ws.view(torch.uint8)

    def take(off, count):
        return raw[off:off + 4 * count].view(torch.int32).cpu()

    return {"sorted": take(out[0], pairs), "bounds": take(out[1], n_exp + 1), "tile_start": take(out[2], n_exp + 1),
            "small": take(out[3], n_exp), "tile_j": int(out[4]), "small_max": int(out[5])}


def debug_subdots_workspace(qtype, rows, k, n, path):
    return int(_L.qmm_debug_subdots_workspace(qtype, rows, k, n, path))


def debug_subdots(w, qtype, rows, k, xq, n, path):
    """Integer sub-block dots from the chosen production kernel in its production plan: int32
    [n, rows, per]."""
    torch = _torch()
    pw = _need(w, torch.uint8, "w")
    px = _need(xq, torch.uint8, "xq")
    _need_weights(w, qtype, rows, k, "w")
    _need_size(xq, n * (k // 32) * Q8_1_BYTES, "xq")
    per = k // 16 if (qtype in (Q6_K, Q3_K) and path == PATH_MATVEC) else k // 32
    out = torch.zeros((n, rows, per), dtype=torch.int32, device=xq.device)
    ws = _workspace(debug_subdots_workspace(qtype, rows, k, n, path), xq.device)
    _on_device(w=w, xq=xq, out=out, ws=ws)
    _check(_L.qmm_debug_subdots(qtype, pw, rows, k, px, n, path, ctypes.c_void_p(out.data_ptr()),
                                ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream()))
    return out
