"""MI355X-native W4A4 + INT8-outlier hybrid linear layer (QUIK / Atom style).

Python binding over the C ABI in ``include/w4a4.h`` (``libw4a4.so``, built
with ``python -m mixed_precision_integer_amd.build``). This module only
marshals arguments: every step of the layer runs in the HIP kernels. PyTorch
provides device memory and the current stream.

Names follow the C ABI: ``quant_reorder_act``, ``pack_int4_weights``,
``w4a4_outlier_gemm`` (+ ``w4a4_outlier_gemm_i32``, the accumulator export)
and ``quant_gemm`` map to ``w4a4_quant_reorder_act``,
``w4a4_pack_int4_weights``, ``w4a4_outlier_gemm`` (+ ``_i32``) and
``w4a4_quant_gemm``; ``rmsnorm_quant_reorder_act`` and ``rmsnorm_quant_gemm``
(the producer fused with the preceding RMSNorm) map to
``w4a4_rmsnorm_quant_reorder_act`` and ``w4a4_rmsnorm_quant_gemm``.

There is no fallback: if the library is missing or no GPU is present the
calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a4.so")
_lib = None

STATUS = {0: "W4A4_OK", 1: "W4A4_ERR_INVALID_ARG", 2: "W4A4_ERR_UNSUPPORTED",
          3: "W4A4_ERR_ALIGNMENT", 4: "W4A4_ERR_HIP", 5: "W4A4_ERR_WORKSPACE"}

EXPORTED = ("w4a4_status_string", "w4a4_num_groups", "w4a4_pitch4_bytes", "w4a4_pitch8_bytes",
            "w4a4_make_perm", "w4a4_quant_reorder_act", "w4a4_pack_int4_weights",
            "w4a4_outlier_gemm_workspace_bytes", "w4a4_outlier_gemm_kernel_name", "w4a4_outlier_gemm",
            "w4a4_outlier_gemm_i32",
            "w4a4_quant_gemm_workspace_bytes", "w4a4_quant_gemm_kernel_name", "w4a4_quant_gemm",
            "w4a4_rmsnorm_quant_reorder_act", "w4a4_rmsnorm_quant_gemm",
            "w4a4_select_outliers_workspace_bytes", "w4a4_select_outliers",
            "w4a4_w4a8_gemm", "w4a4_w4a8_gemm_i32", "w4a4_kv_quant", "w4a4_kv_dequant",
            "w4a4_u6_bytes", "w4a4_repack_u6", "w4a4_quant_reorder_act_u6",
            "w4a4_rmsnorm_quant_reorder_act_u6", "w4a4_outlier_gemm_fp6_kernel_name",
            "w4a4_outlier_gemm_fp6", "w4a4_outlier_gemm_fp6_i32", "w4a4_quant_gemm_fp6_workspace_bytes",
            "w4a4_quant_gemm_fp6", "w4a4_quant_gemm_static_max_bytes", "w4a4_quant_gemm_static")


class W4A4Error(RuntimeError):
    def __init__(self, status: int, call: str):
        super().__init__(f"{call} failed: {STATUS.get(status, status)}")
        self.status = status


def lib():
    """Load libw4a4.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mixed_precision_integer_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    L.w4a4_status_string.argtypes = [ctypes.c_int]
    L.w4a4_status_string.restype = ctypes.c_char_p
    L.w4a4_num_groups.argtypes = [i32, i32]
    L.w4a4_num_groups.restype = i32
    L.w4a4_pitch4_bytes.argtypes = [i32]
    L.w4a4_pitch4_bytes.restype = i64
    L.w4a4_pitch8_bytes.argtypes = [i32]
    L.w4a4_pitch8_bytes.restype = i64
    L.w4a4_make_perm.argtypes = [i32, vp, i32, vp]
    L.w4a4_make_perm.restype = ctypes.c_int
    for name in ("w4a4_quant_reorder_act", "w4a4_pack_int4_weights"):
        f = getattr(L, name)
        f.argtypes = [vp, i64, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        f.restype = ctypes.c_int
    for name in ("w4a4_outlier_gemm_workspace_bytes", "w4a4_quant_gemm_workspace_bytes"):
        f = getattr(L, name)
        f.argtypes = [i32, i32, i32, i32, i32]
        f.restype = sz
    for name in ("w4a4_outlier_gemm_kernel_name", "w4a4_quant_gemm_kernel_name"):
        f = getattr(L, name)
        f.argtypes = [i32, i32, i32, i32, i32]
        f.restype = ctypes.c_char_p
    L.w4a4_outlier_gemm.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                    vp, i64, vp, sz, vp]
    L.w4a4_outlier_gemm.restype = ctypes.c_int
    L.w4a4_outlier_gemm_i32.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                        vp, i64, vp, sz, vp, vp, vp]
    L.w4a4_outlier_gemm_i32.restype = ctypes.c_int
    L.w4a4_quant_gemm.argtypes = [vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i64,
                                  vp, sz, vp]
    L.w4a4_quant_gemm.restype = ctypes.c_int
    f32 = ctypes.c_float
    L.w4a4_rmsnorm_quant_reorder_act.argtypes = [vp, i64, vp, f32, vp, i32, i32, i32, i32, vp, vp,
                                                 vp, vp, vp, vp]
    L.w4a4_rmsnorm_quant_reorder_act.restype = ctypes.c_int
    L.w4a4_rmsnorm_quant_gemm.argtypes = [vp, i64, vp, f32, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                          i32, vp, i64, vp, sz, vp]
    L.w4a4_rmsnorm_quant_gemm.restype = ctypes.c_int
    L.w4a4_select_outliers_workspace_bytes.argtypes = [i32, i32]
    L.w4a4_select_outliers_workspace_bytes.restype = sz
    L.w4a4_select_outliers.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.w4a4_select_outliers.restype = ctypes.c_int
    L.w4a4_w4a8_gemm.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, i64, vp]
    L.w4a4_w4a8_gemm.restype = ctypes.c_int
    L.w4a4_w4a8_gemm_i32.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp]
    L.w4a4_w4a8_gemm_i32.restype = ctypes.c_int
    L.w4a4_kv_quant.argtypes = [vp, i64, i32, i32, i32, i32, vp, i64, vp, vp, vp]
    L.w4a4_kv_quant.restype = ctypes.c_int
    L.w4a4_kv_dequant.argtypes = [vp, vp, i64, vp, i32, i32, i32, i32, vp, i64, vp]
    L.w4a4_kv_dequant.restype = ctypes.c_int
    L.w4a4_quant_gemm_static_max_bytes.argtypes = []
    L.w4a4_quant_gemm_static_max_bytes.restype = sz
    L.w4a4_quant_gemm_static.argtypes = [vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i64, vp]
    L.w4a4_quant_gemm_static.restype = ctypes.c_int
    L.w4a4_u6_bytes.argtypes = [i32, i32]
    L.w4a4_u6_bytes.restype = i64
    L.w4a4_repack_u6.argtypes = [vp, i32, i32, vp, vp]
    L.w4a4_repack_u6.restype = ctypes.c_int
    L.w4a4_quant_reorder_act_u6.argtypes = [vp, i64, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp]
    L.w4a4_quant_reorder_act_u6.restype = ctypes.c_int
    L.w4a4_rmsnorm_quant_reorder_act_u6.argtypes = [vp, i64, vp, f32, vp, i32, i32, i32, i32, vp, vp,
                                                    vp, vp, vp, vp]
    L.w4a4_rmsnorm_quant_reorder_act_u6.restype = ctypes.c_int
    L.w4a4_outlier_gemm_fp6_kernel_name.argtypes = [i32, i32, i32, i32, i32]
    L.w4a4_outlier_gemm_fp6_kernel_name.restype = ctypes.c_char_p
    L.w4a4_outlier_gemm_fp6.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i64, vp]
    L.w4a4_outlier_gemm_fp6.restype = ctypes.c_int
    L.w4a4_outlier_gemm_fp6_i32.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i64,
                                            vp, vp, vp]
    L.w4a4_outlier_gemm_fp6_i32.restype = ctypes.c_int
    L.w4a4_quant_gemm_fp6_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.w4a4_quant_gemm_fp6_workspace_bytes.restype = sz
    L.w4a4_quant_gemm_fp6.argtypes = [vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i64, vp, sz, vp]
    L.w4a4_quant_gemm_fp6.restype = ctypes.c_int
    _lib = L
    return L


def _ok(status: int, call: str):
    if status != 0:
        raise W4A4Error(status, call)


# ---------------------------------------------------------------------------
# host helpers
# ---------------------------------------------------------------------------
def num_groups(K_n: int, group: int) -> int:
    return int(lib().w4a4_num_groups(K_n, group))


def pitch4_bytes(K_n: int) -> int:
    return int(lib().w4a4_pitch4_bytes(K_n))


def pitch8_bytes(n_out: int) -> int:
    return int(lib().w4a4_pitch8_bytes(n_out))


def make_perm(K: int, outlier_idx) -> np.ndarray:
    """Host int32 permutation: non-outliers ascending, then outliers ascending."""
    o = np.ascontiguousarray(np.asarray(outlier_idx, dtype=np.int32).reshape(-1))
    perm = np.zeros(max(K, 1), np.int32)
    _ok(lib().w4a4_make_perm(K, o.ctypes.data if o.size else None, o.size, perm.ctypes.data),
        "w4a4_make_perm")
    return perm[:K]


# ---------------------------------------------------------------------------
# device calls
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return _torch().cuda.current_stream().cuda_stream


def _check(t, dtype, name, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    if t.numel() and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dim")


class QuantizedOperand(NamedTuple):
    """Quantized rows in the ABI layout (activations or weights)."""
    q4: object      # uint8 [rows, pitch4]
    q8: object      # int8 [rows, pitch8] (None when n_out == 0)
    s4: object      # fp32 [rows, G]
    s8: object      # fp32 [rows]
    K: int
    n_out: int
    group: int


def _quant_args(src, perm, op: QuantizedOperand):
    rows, K = src.shape
    return (src.data_ptr(), src.stride(0) if rows else K, _ptr(perm), rows, K, op.n_out,
            op.group, _nz(op.q4), _nz(op.q8), _nz(op.s4), _nz(op.s8), _stream())


def _quant_rows(fn, name, src, perm, n_out, group):
    torch = _torch()
    _check(src, torch.float16, name, 2)
    if perm is not None:                      # None: the identity order
        _check(perm, torch.int32, "perm", 1)
    op = alloc_operand(src.shape[0], src.shape[1], n_out, group, src.device)
    _ok(fn(*_quant_args(src, perm, op)), name)
    return op


def alloc_operand(rows: int, K: int, n_out: int, group: int, device) -> QuantizedOperand:
    """Empty device buffers in the ABI layout for `rows` quantized rows."""
    torch = _torch()
    K_n = K - n_out
    G = num_groups(K_n, group)
    if G < 0:
        raise ValueError("group must divide K - n_out")
    return QuantizedOperand(
        torch.empty((rows, pitch4_bytes(K_n)), dtype=torch.uint8, device=device),
        torch.empty((rows, pitch8_bytes(n_out)), dtype=torch.int8, device=device) if n_out else None,
        torch.empty((rows, G), dtype=torch.float32, device=device),
        torch.empty((rows,), dtype=torch.float32, device=device), K, n_out, group)


def quant_reorder_act(X, perm, n_out: int, group: int) -> QuantizedOperand:
    """Runtime activation producer: reorder + INT4/INT8 quantize every token row."""
    return _quant_rows(lib().w4a4_quant_reorder_act, "w4a4_quant_reorder_act", X, perm, n_out,
                       group)


def _norm_args(X, gamma, eps):
    torch = _torch()
    _check(gamma, torch.float16, "gamma", 1)
    if gamma.shape[0] != X.shape[1] or (gamma.numel() and gamma.stride(0) != 1):
        raise ValueError("gamma must be a contiguous [K] vector")
    return gamma.data_ptr(), float(eps)


def rmsnorm_quant_reorder_act(X, gamma, eps: float, perm, n_out: int, group: int,
                              want_rstd: bool = False):
    """Producer fused with the preceding RMSNorm: normalize every token row
    (weight gamma [K] fp16, original channel order), then reorder and quantize
    it as quant_reorder_act does. Returns the operand, or (operand, rstd fp32
    [M]) with want_rstd."""
    torch = _torch()
    _check(X, torch.float16, "X", 2)
    _check(perm, torch.int32, "perm", 1)
    g, e = _norm_args(X, gamma, eps)
    M, K = X.shape
    op = alloc_operand(M, K, n_out, group, X.device)
    rstd = torch.empty((M,), dtype=torch.float32, device=X.device) if want_rstd else None
    _ok(lib().w4a4_rmsnorm_quant_reorder_act(X.data_ptr(), X.stride(0) if M else K, g, e,
                                             perm.data_ptr(), M, K, n_out, group, _nz(op.q4),
                                             _nz(op.q8), _nz(op.s4), _nz(op.s8), _nz(rstd),
                                             _stream()), "w4a4_rmsnorm_quant_reorder_act")
    return (op, rstd) if want_rstd else op


def pack_int4_weights(W, perm, n_out: int, group: int) -> QuantizedOperand:
    """Offline weight preparation with the same quantizer (rows = output channels)."""
    return _quant_rows(lib().w4a4_pack_int4_weights, "w4a4_pack_int4_weights", W, perm, n_out,
                       group)


def _gemm_ptrs(a: QuantizedOperand, w: QuantizedOperand):
    if (a.K, a.n_out, a.group) != (w.K, w.n_out, w.group):
        raise ValueError("activation and weight quantization parameters differ")
    return a.q4, a.q8, a.s4, a.s8, w.q4, w.q8, w.s4, w.s8


def _nz(t):
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _gemm_args(a: QuantizedOperand, w: QuantizedOperand, out, ws):
    M, N = a.s8.shape[0], w.s8.shape[0]
    return (*[_nz(t) for t in _gemm_ptrs(a, w)], M, N, a.K, a.n_out, a.group, out.data_ptr(),
            out.stride(0) if M else N, _ptr(ws), 0 if ws is None else ws.numel(), _stream())


def outlier_gemm_workspace_bytes(M: int, N: int, K: int, n_out: int, group: int) -> int:
    return int(lib().w4a4_outlier_gemm_workspace_bytes(M, N, K, n_out, group))


def outlier_gemm_kernel_name(M: int, N: int, K: int, n_out: int, group: int):
    """Kernel the GEMM launches for this shape (as named in a kernel trace), or None."""
    r = lib().w4a4_outlier_gemm_kernel_name(M, N, K, n_out, group)
    return None if r is None else r.decode()


def quant_gemm_kernel_name(M: int, N: int, K: int, n_out: int, group: int):
    """Kernel that computes the fused layer call's product for this shape:
    "decode_fused_kernel" when the quantizer runs inside it, else the GEMM's."""
    r = lib().w4a4_quant_gemm_kernel_name(M, N, K, n_out, group)
    return None if r is None else r.decode()


def w4a4_outlier_gemm(a: QuantizedOperand, w: QuantizedOperand, out=None):
    """Y[M, N] fp16 = INT4 GEMM + INT8 outlier GEMM + fp32 scale epilogue."""
    torch = _torch()
    M, N = a.s8.shape[0], w.s8.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=a.s8.device)
    _check(out, torch.float16, "out", 2)
    ws_bytes = outlier_gemm_workspace_bytes(M, N, a.K, a.n_out, a.group)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=out.device) if ws_bytes else None
    _ok(lib().w4a4_outlier_gemm(*_gemm_args(a, w, out, ws)), "w4a4_outlier_gemm")
    return out


def w4a4_outlier_gemm_i32(a: QuantizedOperand, w: QuantizedOperand, out=None):
    """The GEMM with its accumulator export: the same kernel and main loop as
    w4a4_outlier_gemm. Returns (acc4 int32 [G, M, N], acc8 int32 [M, N], Y fp16
    [M, N])."""
    torch = _torch()
    M, N = a.s8.shape[0], w.s8.shape[0]
    G = num_groups(a.K - a.n_out, a.group)
    dev = a.s8.device
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
    _check(out, torch.float16, "out", 2)
    acc4 = torch.empty((G, M, N), dtype=torch.int32, device=dev)
    acc8 = torch.empty((M, N), dtype=torch.int32, device=dev)
    ws_bytes = outlier_gemm_workspace_bytes(M, N, a.K, a.n_out, a.group)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    _ok(lib().w4a4_outlier_gemm_i32(*_gemm_args(a, w, out, ws)[:-1], _nz(acc4),
                                    _nz(acc8) if a.n_out else None, _stream()), "w4a4_outlier_gemm_i32")
    if not a.n_out:
        acc8.zero_()
    return acc4, acc8, out


def quant_gemm_workspace_bytes(M: int, N: int, K: int, n_out: int, group: int) -> int:
    return int(lib().w4a4_quant_gemm_workspace_bytes(M, N, K, n_out, group))


def quant_gemm(X, perm, w: QuantizedOperand, out=None, workspace=None):
    """The fused layer: activation producer + mixed-precision GEMM on one stream."""
    torch = _torch()
    _check(X, torch.float16, "X", 2)
    _check(perm, torch.int32, "perm", 1)
    M, K = X.shape
    N = w.s8.shape[0]
    if K != w.K:
        raise ValueError("X and weights disagree on K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _check(out, torch.float16, "out", 2)
    need = quant_gemm_workspace_bytes(M, N, K, w.n_out, w.group)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=X.device)
    _check(workspace, torch.uint8, "workspace", 1)
    _ok(lib().w4a4_quant_gemm(X.data_ptr(), X.stride(0) if M else K, perm.data_ptr(), _nz(w.q4),
                              _nz(w.q8), _nz(w.s4), _nz(w.s8), M, N, K, w.n_out, w.group,
                              out.data_ptr(), out.stride(0) if M else N, workspace.data_ptr(),
                              workspace.numel(), _stream()), "w4a4_quant_gemm")
    return out


def quant_gemm_static(X, perm, w: QuantizedOperand, out=None):
    """The fused layer with the library's static per-GPU workspace (no device
    allocation by the call; calls that overlap on one GPU race)."""
    torch = _torch()
    _check(X, torch.float16, "X", 2)
    _check(perm, torch.int32, "perm", 1)
    M, K = X.shape
    N = w.s8.shape[0]
    if K != w.K:
        raise ValueError("X and weights disagree on K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _check(out, torch.float16, "out", 2)
    _ok(lib().w4a4_quant_gemm_static(X.data_ptr(), X.stride(0) if M else K, perm.data_ptr(), _nz(w.q4),
                                     _nz(w.q8), _nz(w.s4), _nz(w.s8), M, N, K, w.n_out, w.group,
                                     out.data_ptr(), out.stride(0) if M else N, _stream()),
        "w4a4_quant_gemm_static")
    return out


def rmsnorm_quant_gemm(X, gamma, eps: float, perm, w: QuantizedOperand, out=None, workspace=None):
    """The fused layer behind an RMSNorm: norm + producer, then the GEMM."""
    torch = _torch()
    _check(X, torch.float16, "X", 2)
    _check(perm, torch.int32, "perm", 1)
    g, e = _norm_args(X, gamma, eps)
    M, K = X.shape
    N = w.s8.shape[0]
    if K != w.K:
        raise ValueError("X and weights disagree on K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _check(out, torch.float16, "out", 2)
    need = quant_gemm_workspace_bytes(M, N, K, w.n_out, w.group)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=X.device)
    _check(workspace, torch.uint8, "workspace", 1)
    _ok(lib().w4a4_rmsnorm_quant_gemm(X.data_ptr(), X.stride(0) if M else K, g, e, perm.data_ptr(),
                                      _nz(w.q4), _nz(w.q8), _nz(w.s4), _nz(w.s8), M, N, K,
                                      w.n_out, w.group, out.data_ptr(),
                                      out.stride(0) if M else N, workspace.data_ptr(),
                                      workspace.numel(), _stream()), "w4a4_rmsnorm_quant_gemm")
    return out


def select_outliers_workspace_bytes(rows: int, K: int) -> int:
    return int(lib().w4a4_select_outliers_workspace_bytes(rows, K))


def select_outliers(Xcal, n_out: int, workspace=None, want_absmax: bool = False):
    """Offline outlier-channel selection on the GPU: the n_out channels of the
    calibration batch Xcal [rows, K] (fp16) with the largest absmax, ties to
    the lower index. Returns (outlier_idx int32 [n_out] ascending, perm int32
    [K]), plus the fp16 scores [K] with want_absmax."""
    torch = _torch()
    _check(Xcal, torch.float16, "Xcal", 2)
    rows, K = Xcal.shape
    dev = Xcal.device
    need = select_outliers_workspace_bytes(rows, K)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(workspace, torch.uint8, "workspace", 1)
    idx = torch.empty((n_out,), dtype=torch.int32, device=dev)
    perm = torch.empty((K,), dtype=torch.int32, device=dev)
    amax = torch.empty((K,), dtype=torch.float16, device=dev) if want_absmax else None
    _ok(lib().w4a4_select_outliers(Xcal.data_ptr() if rows else None, Xcal.stride(0) if rows else K,
                                   rows, K, n_out, _nz(idx), perm.data_ptr(), _ptr(amax),
                                   workspace.data_ptr(), workspace.numel(), _stream()),
        "w4a4_select_outliers")
    return (idx, perm, amax) if want_absmax else (idx, perm)


# ---------------------------------------------------------------------------
# FP6 prefill path: INT4 codes q held as the FP6 E2M3 values q / 8 ("u6" operands)
# ---------------------------------------------------------------------------
def u6_bytes(rows: int, K_n: int) -> int:
    return int(lib().w4a4_u6_bytes(rows, K_n))


def repack_u6(q4, K_n: int):
    """Packed INT4 nibbles [rows, pitch4] -> the u6 operand of the FP6 GEMM
    (uint8 [u6_bytes]: 32-row x 64-channel blocks of 1536 bytes)."""
    torch = _torch()
    _check(q4, torch.uint8, "q4", 2)
    rows = q4.shape[0]
    out = torch.empty(max(u6_bytes(rows, K_n), 1), dtype=torch.uint8, device=q4.device)
    _ok(lib().w4a4_repack_u6(_nz(q4), rows, K_n, out.data_ptr(), _stream()), "w4a4_repack_u6")
    return out


class Fp6Operand(NamedTuple):
    """An operand of the FP6 GEMM: the INT4 head as u6 bytes, the INT8 tail
    and the scales as in QuantizedOperand."""
    u6: object
    q8: object
    s4: object
    s8: object
    K: int
    n_out: int
    group: int


def to_fp6(op: QuantizedOperand) -> Fp6Operand:
    """Repack a quantized operand's INT4 head for the FP6 GEMM."""
    return Fp6Operand(repack_u6(op.q4, op.K - op.n_out), op.q8, op.s4, op.s8, op.K, op.n_out, op.group)


def quant_reorder_act_u6(X, perm, n_out: int, group: int = 0, out: Fp6Operand = None) -> Fp6Operand:
    """Runtime activation producer of the FP6 path: reorder + quantize every
    token row, the INT4 head written straight into a u6 operand (into `out`'s
    buffers when given)."""
    torch = _torch()
    _check(X, torch.float16, "X", 2)
    _check(perm, torch.int32, "perm", 1)
    M, K = X.shape
    a = out if out is not None else alloc_fp6_operand(M, K, n_out, group, X.device)
    if a.u6.numel() < u6_bytes(M, K - n_out) or a.s8.shape[0] < M:
        raise ValueError("out is too small")
    _ok(lib().w4a4_quant_reorder_act_u6(X.data_ptr(), X.stride(0) if M else K, perm.data_ptr(), M, K, n_out,
                                        group, a.u6.data_ptr(), _nz(a.q8), a.s4.data_ptr(), a.s8.data_ptr(),
                                        _stream()),
        "w4a4_quant_reorder_act_u6")
    return a


def rmsnorm_quant_reorder_act_u6(X, gamma, eps: float, perm, n_out: int, group: int,
                                 want_rstd: bool = False):
    """The FP6 path's producer fused with the preceding RMSNorm: the codes,
    scales and rstd of rmsnorm_quant_reorder_act, the INT4 head written as a
    u6 operand. Returns the operand, or (operand, rstd fp32 [M])."""
    torch = _torch()
    _check(X, torch.float16, "X", 2)
    _check(perm, torch.int32, "perm", 1)
    g, e = _norm_args(X, gamma, eps)
    M, K = X.shape
    a = alloc_fp6_operand(M, K, n_out, group, X.device)
    rstd = torch.empty((M,), dtype=torch.float32, device=X.device) if want_rstd else None
    _ok(lib().w4a4_rmsnorm_quant_reorder_act_u6(X.data_ptr(), X.stride(0) if M else K, g, e, perm.data_ptr(),
                                                M, K, n_out, group, a.u6.data_ptr(), _nz(a.q8),
                                                a.s4.data_ptr(), a.s8.data_ptr(), _nz(rstd), _stream()),
        "w4a4_rmsnorm_quant_reorder_act_u6")
    return (a, rstd) if want_rstd else a


def alloc_fp6_operand(rows: int, K: int, n_out: int, group: int, device) -> Fp6Operand:
    """Empty device buffers of an FP6-path operand of `rows` rows."""
    torch = _torch()
    K_n = K - n_out
    G = num_groups(K_n, group)
    if G < 0:
        raise ValueError("group must divide K - n_out")
    return Fp6Operand(
        torch.empty(max(u6_bytes(rows, K_n), 1), dtype=torch.uint8, device=device),
        torch.empty((rows, pitch8_bytes(n_out)), dtype=torch.int8, device=device) if n_out else None,
        torch.empty((rows, G), dtype=torch.float32, device=device),
        torch.empty((rows,), dtype=torch.float32, device=device), K, n_out, group)


def pack_weights_fp6(W, perm, n_out: int, group: int) -> Fp6Operand:
    """Offline weight preparation for the FP6 prefill path."""
    return to_fp6(pack_int4_weights(W, perm, n_out, group))


def outlier_gemm_fp6_kernel_name(M: int, N: int, K: int, n_out: int, group: int):
    r = lib().w4a4_outlier_gemm_fp6_kernel_name(M, N, K, n_out, group)
    return None if r is None else r.decode()


def _fp6_args(a: Fp6Operand, w: Fp6Operand, out):
    if (a.K, a.n_out, a.group) != (w.K, w.n_out, w.group):
        raise ValueError("activation and weight quantization parameters differ")
    M, N = a.s8.shape[0], w.s8.shape[0]
    return (_nz(a.u6), _nz(a.q8), _nz(a.s4), _nz(a.s8), _nz(w.u6), _nz(w.q8), _nz(w.s4), _nz(w.s8), M, N, a.K,
            a.n_out, a.group, out.data_ptr(), out.stride(0) if M else N)


def outlier_gemm_fp6(a: Fp6Operand, w: Fp6Operand, out=None):
    """Y[M, N] fp16 from FP6-held INT4 operands (the same integer sums as
    w4a4_outlier_gemm)."""
    torch = _torch()
    M, N = a.s8.shape[0], w.s8.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=a.s8.device)
    _check(out, torch.float16, "out", 2)
    _ok(lib().w4a4_outlier_gemm_fp6(*_fp6_args(a, w, out), _stream()), "w4a4_outlier_gemm_fp6")
    return out


def outlier_gemm_fp6_i32(a: Fp6Operand, w: Fp6Operand, out=None):
    """The FP6 GEMM with its accumulator export: (acc4 int32 [G, M, N], acc8
    int32 [M, N], Y)."""
    torch = _torch()
    M, N = a.s8.shape[0], w.s8.shape[0]
    G = num_groups(a.K - a.n_out, a.group)
    dev = a.s8.device
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
    acc4 = torch.zeros((G, M, N), dtype=torch.int32, device=dev)
    acc8 = torch.zeros((M, N), dtype=torch.int32, device=dev)
    _ok(lib().w4a4_outlier_gemm_fp6_i32(*_fp6_args(a, w, out), _nz(acc4), _nz(acc8) if a.n_out else None,
                                        _stream()), "w4a4_outlier_gemm_fp6_i32")
    return acc4, acc8, out


def quant_gemm_fp6_workspace_bytes(M: int, N: int, K: int, n_out: int, group: int) -> int:
    return int(lib().w4a4_quant_gemm_fp6_workspace_bytes(M, N, K, n_out, group))


def quant_gemm_fp6(X, perm, w: Fp6Operand, out=None, workspace=None):
    """The fused prefill layer on the FP6 path: producer, repack of the
    activation codes, FP6 GEMM, on one stream."""
    torch = _torch()
    _check(X, torch.float16, "X", 2)
    _check(perm, torch.int32, "perm", 1)
    M, K = X.shape
    N = w.s8.shape[0]
    if K != w.K:
        raise ValueError("X and weights disagree on K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _check(out, torch.float16, "out", 2)
    need = quant_gemm_fp6_workspace_bytes(M, N, K, w.n_out, w.group)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=X.device)
    _check(workspace, torch.uint8, "workspace", 1)
    _ok(lib().w4a4_quant_gemm_fp6(X.data_ptr(), X.stride(0) if M else K, perm.data_ptr(), _nz(w.u6), _nz(w.q8),
                                  _nz(w.s4), _nz(w.s8), M, N, K, w.n_out, w.group, out.data_ptr(),
                                  out.stride(0) if M else N, workspace.data_ptr(), workspace.numel(), _stream()),
        "w4a4_quant_gemm_fp6")
    return out


class W4A8Operand(NamedTuple):
    """W4A8 operand: INT8 activation rows (q [rows, K], s [rows]) or INT4
    weight rows (q [rows, K / 2] packed, s [rows, G])."""
    q: object
    s: object
    K: int
    group: int


def quant_act_int8(X) -> W4A8Operand:
    """W4A8 activations: per-token INT8 over all K channels in the original
    order (the producer with a null permutation and n_out = K)."""
    op = _quant_rows(lib().w4a4_quant_reorder_act, "w4a4_quant_reorder_act", X, None, X.shape[1], 0)
    return W4A8Operand(op.q8, op.s8, X.shape[1], 0)


def pack_int4_weights_w4a8(W, group: int) -> W4A8Operand:
    """W4A8 weights: INT4 per output channel (group 0) or per `group`
    channels, original order (no outliers)."""
    op = _quant_rows(lib().w4a4_pack_int4_weights, "w4a4_pack_int4_weights", W, None, 0, group)
    return W4A8Operand(op.q4, op.s4, W.shape[1], group)


def w4a8_gemm(a: W4A8Operand, w: W4A8Operand, out=None):
    """Y [M, N] fp16 = sa8[m] * sum_t sw4[n, t] * (INT8 x INT4 group sums)."""
    torch = _torch()
    if a.K != w.K:
        raise ValueError("activations and weights disagree on K")
    M, N = a.s.shape[0], w.s.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=a.s.device)
    _check(out, torch.float16, "out", 2)
    _ok(lib().w4a4_w4a8_gemm(_nz(a.q), _nz(a.s), _nz(w.q), _nz(w.s), M, N, a.K, w.group,
                             out.data_ptr(), out.stride(0) if M else N, _stream()), "w4a4_w4a8_gemm")
    return out


def w4a8_gemm_i32(a: W4A8Operand, w: W4A8Operand):
    """Accumulator export of the W4A8 main loop: int32 [G, M, N]."""
    torch = _torch()
    M, N = a.s.shape[0], w.s.shape[0]
    G = num_groups(a.K, w.group)
    acc = torch.zeros((G, M, N), dtype=torch.int32, device=a.s.device)
    _ok(lib().w4a4_w4a8_gemm_i32(_nz(a.q), _nz(w.q), M, N, a.K, w.group, _nz(acc), _stream()),
        "w4a4_w4a8_gemm_i32")
    return acc


class KVCache:
    """A slot-mapped low-bit KV cache for one tensor (keys or values):
    codes uint8 [num_slots, H, D * bits / 8] and scales fp32 [num_slots, H]."""

    def __init__(self, num_slots: int, H: int, D: int, bits: int, device):
        torch = _torch()
        self.num_slots, self.H, self.D, self.bits = num_slots, H, D, bits
        self.q = torch.zeros((num_slots, H, D * bits // 8), dtype=torch.uint8, device=device)
        self.s = torch.zeros((num_slots, H), dtype=torch.float32, device=device)

    def store(self, X, slots=None):
        """Quantize X [T, H * D] (fp16) into the slots (int32 [T], or None for 0..T-1)."""
        torch = _torch()
        _check(X, torch.float16, "X", 2)
        if slots is not None:
            _check(slots, torch.int32, "slots", 1)
        T = X.shape[0]
        _ok(lib().w4a4_kv_quant(X.data_ptr() if T else None, X.stride(0) if T else self.H * self.D, T,
                                self.H, self.D, self.bits, _ptr(slots), self.num_slots, self.q.data_ptr(),
                                self.s.data_ptr(), _stream()), "w4a4_kv_quant")

    def load(self, slots=None, T=None, out=None):
        """fp16 [T, H * D] of the given slots (None: slots 0..T-1)."""
        torch = _torch()
        if slots is not None:
            _check(slots, torch.int32, "slots", 1)
            T = slots.shape[0]
        if out is None:
            out = torch.empty((T, self.H * self.D), dtype=torch.float16, device=self.q.device)
        _check(out, torch.float16, "out", 2)
        _ok(lib().w4a4_kv_dequant(self.q.data_ptr(), self.s.data_ptr(), self.num_slots, _ptr(slots), T,
                                  self.H, self.D, self.bits, out.data_ptr() if T else None,
                                  out.stride(0) if T else self.H * self.D, _stream()), "w4a4_kv_dequant")
        return out


def fp6_path_fills_chip(M: int, N: int, K: int, n_out: int, group: int, cus: int = 256) -> bool:
    """Whether the FP6 GEMM takes this shape with at least one workgroup per
    CU (its 256 x 256 or 128 x 128 tiles over more than 128 rows, or the FP6
    decode kernel's 32-column stripes): the shapes where it beats the i8 path."""
    name = outlier_gemm_fp6_kernel_name(M, N, K, n_out, group)
    if name is None:
        return False
    if name.startswith("gemm_fp6_decode_kernel"):
        return -(-N // 32) >= cus
    tile = 256 if group == 0 else 128
    return M > 128 and -(-M // tile) * -(-N // tile) >= cus


class W4A4Linear:
    """A linear layer y = x W^T with W held as packed INT4 + INT8 outlier
    columns; with norm_weight (fp16 [K]) the layer first applies the RMSNorm
    in front of it, fused into its producer. With fp6=True the layer also
    keeps the weights as a u6 operand (1.5 times the nibble bytes) and runs
    the FP6 GEMM for the batch sizes where it fills the chip
    (fp6_path_fills_chip); other batches keep the i8 path."""

    def __init__(self, weight, outlier_idx, group: int = 0, norm_weight=None, eps: float = 1e-6,
                 fp6: bool = False):
        torch = _torch()
        K = weight.shape[1]
        self.outlier_idx = np.asarray(outlier_idx, np.int32)
        self.perm = torch.from_numpy(make_perm(K, self.outlier_idx)).to(weight.device)
        self.n_out = int(self.outlier_idx.size)
        self.group = group
        self.weight = pack_int4_weights(weight, self.perm, self.n_out, group)
        self.weight_fp6 = to_fp6(self.weight) if fp6 else None
        self.norm_weight, self.eps = norm_weight, eps
        self._ws = None

    def __call__(self, X, out=None):
        M, N = X.shape[0], self.weight.s8.shape[0]
        if self.weight_fp6 is not None and fp6_path_fills_chip(M, N, self.weight.K, self.n_out, self.group):
            if self.norm_weight is None:
                return quant_gemm_fp6(X, self.perm, self.weight_fp6, out=out)
            a = rmsnorm_quant_reorder_act_u6(X, self.norm_weight, self.eps, self.perm, self.n_out, self.group)
            return outlier_gemm_fp6(a, self.weight_fp6, out=out)
        need = quant_gemm_workspace_bytes(X.shape[0], self.weight.s8.shape[0], self.weight.K,
                                          self.n_out, self.group)
        if self._ws is None or self._ws.numel() < need:
            self._ws = _torch().zeros(max(need, 1), dtype=_torch().uint8, device=X.device)
        if self.norm_weight is not None:
            return rmsnorm_quant_gemm(X, self.norm_weight, self.eps, self.perm, self.weight, out=out,
                                      workspace=self._ws)
        return quant_gemm(X, self.perm, self.weight, out=out, workspace=self._ws)


class LayerPlan:
    """Arguments of one layer call, marshalled once.

    ``fused()`` is ``w4a4_quant_gemm``; ``produce()`` and ``gemm()`` are its two
    halves (``w4a4_quant_reorder_act`` into a pre-allocated operand, then
    ``w4a4_outlier_gemm``), which launch the same kernels. With ``norm=(gamma,
    eps)`` the producer is the RMSNorm-fused one (``w4a4_rmsnorm_quant_*``).
    Each call is one ctypes call on the stream that was current when the plan
    was made.
    """

    def __init__(self, X, perm, w: QuantizedOperand, out=None, norm=None):
        torch = _torch()
        _check(X, torch.float16, "X", 2)
        _check(perm, torch.int32, "perm", 1)
        M, K = X.shape
        N = w.s8.shape[0]
        self.out = out if out is not None else torch.empty((M, N), dtype=torch.float16,
                                                           device=X.device)
        self.a = alloc_operand(M, K, w.n_out, w.group, X.device)
        need = quant_gemm_workspace_bytes(M, N, K, w.n_out, w.group)
        self.ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=X.device)
        gws = outlier_gemm_workspace_bytes(M, N, K, w.n_out, w.group)
        self.gws = torch.zeros(gws, dtype=torch.uint8, device=X.device) if gws else None
        self._keep = (X, perm, w, norm)
        L = lib()
        self._g = L.w4a4_outlier_gemm
        self._ga = _gemm_args(self.a, w, self.out, self.gws)
        qa = _quant_args(X, perm, self.a)
        fa = (perm.data_ptr(), _nz(w.q4), _nz(w.q8), _nz(w.s4), _nz(w.s8), M, N, K, w.n_out,
              w.group, self.out.data_ptr(), self.out.stride(0) if M else N, self.ws.data_ptr(),
              self.ws.numel(), _stream())
        xa = (X.data_ptr(), X.stride(0) if M else K)
        if norm is None:
            self._qname, self._fname = "w4a4_quant_reorder_act", "w4a4_quant_gemm"
            self._q, self._f = L.w4a4_quant_reorder_act, L.w4a4_quant_gemm
            self._qa, self._fa = qa, (*xa, *fa)
        else:
            g, e = _norm_args(X, *norm)
            self._qname, self._fname = "w4a4_rmsnorm_quant_reorder_act", "w4a4_rmsnorm_quant_gemm"
            self._q, self._f = L.w4a4_rmsnorm_quant_reorder_act, L.w4a4_rmsnorm_quant_gemm
            self._qa = (*xa, g, e, *qa[2:11], None, qa[11])
            self._fa = (*xa, g, e, *fa)

    def produce(self):
        st = self._q(*self._qa)
        if st:
            raise W4A4Error(st, self._qname)

    def gemm(self):
        st = self._g(*self._ga)
        if st:
            raise W4A4Error(st, "w4a4_outlier_gemm")

    def fused(self):
        st = self._f(*self._fa)
        if st:
            raise W4A4Error(st, self._fname)
        return self.out


class Fp6LayerPlan:
    """Arguments of one FP6-path layer call, marshalled once (the FP6
    counterpart of LayerPlan): ``produce()`` runs w4a4_quant_reorder_act_u6
    (w4a4_rmsnorm_quant_reorder_act_u6 with norm = (gamma, eps)) into
    pre-allocated operands, ``gemm()`` runs w4a4_outlier_gemm_fp6,
    ``fused()`` is w4a4_quant_gemm_fp6 (the same launches; no norm)."""

    def __init__(self, X, perm, w: Fp6Operand, out=None, norm=None):
        torch = _torch()
        _check(X, torch.float16, "X", 2)
        _check(perm, torch.int32, "perm", 1)
        M, K = X.shape
        N = w.s8.shape[0]
        self.out = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=X.device)
        self.a = alloc_fp6_operand(M, K, w.n_out, w.group, X.device)
        need = quant_gemm_fp6_workspace_bytes(M, N, K, w.n_out, w.group)
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=X.device)
        self._keep = (X, perm, w)
        L = lib()
        st = _stream()
        if norm is None:
            self._q, self._qn = L.w4a4_quant_reorder_act_u6, "w4a4_quant_reorder_act_u6"
            self._qa = (X.data_ptr(), X.stride(0) if M else K, perm.data_ptr(), M, K, w.n_out, w.group,
                        self.a.u6.data_ptr(), _nz(self.a.q8), _nz(self.a.s4), _nz(self.a.s8), st)
        else:
            g, e = _norm_args(X, *norm)
            self._keep = (X, perm, w, norm[0])
            self._q, self._qn = L.w4a4_rmsnorm_quant_reorder_act_u6, "w4a4_rmsnorm_quant_reorder_act_u6"
            self._qa = (X.data_ptr(), X.stride(0) if M else K, g, e, perm.data_ptr(), M, K, w.n_out, w.group,
                        self.a.u6.data_ptr(), _nz(self.a.q8), _nz(self.a.s4), _nz(self.a.s8), None, st)
        self._g, self._ga = L.w4a4_outlier_gemm_fp6, (*_fp6_args(self.a, w, self.out), st)
        self._f = L.w4a4_quant_gemm_fp6
        self._fa = (X.data_ptr(), X.stride(0) if M else K, perm.data_ptr(), _nz(w.u6), _nz(w.q8), _nz(w.s4),
                    _nz(w.s8), M, N, K, w.n_out, w.group, self.out.data_ptr(), self.out.stride(0) if M else N,
                    self.ws.data_ptr(), self.ws.numel(), st)

    def produce(self):
        st = self._q(*self._qa)
        if st:
            raise W4A4Error(st, self._qn)

    def gemm(self):
        st = self._g(*self._ga)
        if st:
            raise W4A4Error(st, "w4a4_outlier_gemm_fp6")

    def fused(self):
        st = self._f(*self._fa)
        if st:
            raise W4A4Error(st, "w4a4_quant_gemm_fp6")
        return self.out

