"""ctypes binding of libawq_mi355x.so (the C ABI in include/awq.h).

Argument marshalling only: every step of the forward runs in the library's
HIP kernels.  PyTorch provides device memory and the current stream.  There is
no CPU fallback: without the built library, or with tensors that are not on a
HIP device, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_NAME = "libawq_mi355x.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

AWQ_SUCCESS = 0
AWQ_ERROR_INVALID_VALUE = 1
AWQ_ERROR_SHAPE = 2
AWQ_ERROR_MISALIGNED = 3
AWQ_ERROR_WORKSPACE = 4
AWQ_ERROR_HIP = 5

AWQ_PATH_DECODE = 1
AWQ_PATH_PREFILL = 2
AWQ_PATH_GENERIC = 3
PATH_NAMES = {AWQ_PATH_DECODE: "decode", AWQ_PATH_PREFILL: "prefill",
              AWQ_PATH_GENERIC: "generic"}

# Every symbol include/awq.h declares, with (restype, argtypes).
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
SIGNATURES = {
    "awq_abi_version": (ctypes.c_int, []),
    "awq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "awq_gemm_workspace_size": (ctypes.c_size_t, [_i64, _i64, _i64, _i64]),
    "awq_gemm_plan": (ctypes.c_int, [_i64, _i64, _i64, _i64, _vp, _vp, _vp,
                                     ctypes.POINTER(ctypes.c_int),
                                     ctypes.POINTER(ctypes.c_size_t)]),
    "awq_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                _vp, ctypes.c_size_t, _vp]),
    "awq_dequant": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "awq_dense_gemv": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "awq_dequant_gidx": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "awq_gemm_gidx": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                     _i64, _vp]),
    "awq_gidx_order": (ctypes.c_int, [_vp, _i64, _i64, _vp, ctypes.POINTER(ctypes.c_int64)]),
    "awq_permute_rows": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _vp]),
    "awq_gemm_act_order_workspace_size": (ctypes.c_size_t, [_i64, _i64, _i64, _i64]),
    "awq_gemm_act_order": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                          _i64, _vp, ctypes.c_size_t, _vp]),
}

_lib = None
_lib_lock = threading.Lock()


class AwqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {status_string(status)}")


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lib_lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError(
                        f"{LIB_PATH} is not built; run bit_weight_quantized_awq_amd.build.build() "
                        "(or __graft_entry__.build()) first")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def abi_version() -> int:
    return lib().awq_abi_version()


def status_string(status: int) -> str:
    return lib().awq_status_string(int(status)).decode()


def gemm_workspace_size(M: int, K: int, N: int, group_size: int) -> int:
    return int(lib().awq_gemm_workspace_size(M, K, N, group_size))


def gemm_plan(M: int, K: int, N: int, group_size: int, x_ptr: int = 0,
              scales_ptr: int = 0, qweight_ptr: int = 0) -> tuple[int, int]:
    """(path, workspace bytes) that awq_gemm would use; pointers are only
    inspected for alignment (0 counts as aligned)."""
    path = ctypes.c_int(0)
    ws = ctypes.c_size_t(0)
    st = lib().awq_gemm_plan(M, K, N, group_size, x_ptr or None, qweight_ptr or None,
                             scales_ptr or None, ctypes.byref(path), ctypes.byref(ws))
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_gemm_plan")
    return path.value, ws.value


def gidx_order(g_idx, num_groups: int):
    """Host-only awq_gidx_order: (perm, group_size) for a row-to-group map
    given as a sequence or numpy array of K integers.  perm is an int32 numpy
    array (perm[j] = row placed j-th, rows stably sorted by group);
    group_size is K / num_groups when every group holds that many rows,
    else 0."""
    import numpy as np
    g = np.ascontiguousarray(np.asarray(g_idx), dtype=np.int32)
    if g.ndim != 1:
        raise ValueError("g_idx must be 1-D")
    K = g.shape[0]
    perm = np.empty(K, dtype=np.int32)
    gs = ctypes.c_int64(0)
    st = lib().awq_gidx_order(g.ctypes.data if K else None, K, num_groups,
                              perm.ctypes.data if K else None, ctypes.byref(gs))
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_gidx_order")
    return perm, gs.value


def act_order_workspace_size(M: int, K: int, N: int, group_size: int) -> int:
    return lib().awq_gemm_act_order_workspace_size(M, K, N, group_size)


# --------------------------------------------------------------------- torch
def _torch():
    import torch
    return torch


_workspaces: dict = {}
_ws_lock = threading.Lock()


def _workspace(device, stream_ptr: int, nbytes: int):
    """A zero-filled workspace per (device, stream), grown on demand.  The
    kernels leave it zeroed where it must start at zero, so one buffer serves
    every later call on that stream."""
    torch = _torch()
    if nbytes == 0:
        return None
    key = (device.index, stream_ptr)
    with _ws_lock:
        buf = _workspaces.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            _workspaces[key] = buf
        return buf


def _check_device(name, t, device):
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device (no CPU fallback)")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_group_shapes(K, N, group_size, qzeros, scales):
    # The library validates sizes; the tensors' own shapes must agree with
    # them or it would read past their ends.
    g = K if group_size == -1 else group_size
    if g > 0 and K % g == 0:
        G = K // g
        if tuple(qzeros.shape) != (G, N // 8) or tuple(scales.shape) != (G, N):
            raise ValueError(f"qzeros {tuple(qzeros.shape)} / scales {tuple(scales.shape)} do "
                             f"not match {G} groups of {N} columns")


def gemm(x, qweight, qzeros, scales, bias=None, group_size: int = 128, out=None,
         workspace=None):
    """y = x . dequant(qweight, qzeros, scales) + bias through awq_gemm.

    x: float16 (*, K); qweight int32 (K, N/8); qzeros int32 (G, N/8);
    scales float16 (G, N); bias float16 (N) or None.  Returns float16 (*, N)
    on x's device, enqueued on the current stream."""
    torch = _torch()
    device = qweight.device
    for name, t in (("x", x), ("qweight", qweight), ("qzeros", qzeros), ("scales", scales)):
        _check_device(name, t, device)
    if bias is not None:
        _check_device("bias", bias, device)
    if x.dtype != torch.float16 or scales.dtype != torch.float16:
        raise TypeError("x and scales must be float16")
    if qweight.dtype != torch.int32 or qzeros.dtype != torch.int32:
        raise TypeError("qweight and qzeros must be int32")
    if bias is not None and bias.dtype != torch.float16:
        raise TypeError("bias must be float16")
    K = qweight.shape[0]
    N = qweight.shape[1] * 8
    if x.shape[-1] != K:
        raise ValueError(f"x has {x.shape[-1]} features, qweight has {K}")
    lead = x.shape[:-1]
    x2 = x.reshape(-1, K)
    if not x2.is_contiguous():
        x2 = x2.contiguous()
    M = x2.shape[0]
    _check_group_shapes(K, N, group_size, qzeros, scales)
    qweight, qzeros, scales = qweight.contiguous(), qzeros.contiguous(), scales.contiguous()
    if bias is not None:
        if tuple(bias.shape) != (N,):
            raise ValueError(f"bias shape {tuple(bias.shape)} != ({N},)")
        bias = bias.contiguous()
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=device)
    if out is not None:
        _check_device("out", out, device)
        if out.shape != (M, N) or out.dtype != torch.float16 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float16 (M, N) tensor")
    stream = torch.cuda.current_stream(device).cuda_stream
    if M > 0:
        _, need = gemm_plan(M, K, N, group_size, x2.data_ptr(), scales.data_ptr(),
                            qweight.data_ptr())
    else:
        need = 0
    if workspace is None:
        ws = _workspace(device, stream, need)
    else:
        ws = workspace
    ws_ptr = ws.data_ptr() if ws is not None else None
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = lib().awq_gemm(x2.data_ptr() if M else None, qweight.data_ptr(), qzeros.data_ptr(),
                        scales.data_ptr(), bias.data_ptr() if bias is not None else None,
                        y.data_ptr() if M else None, M, K, N, group_size, ws_ptr, ws_bytes,
                        stream)
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_gemm")
    return y.reshape(*lead, N)


def dense_gemv(x, w, bias=None, out=None):
    """Unquantised baseline through awq_dense_gemv: F.linear(x, w, bias) for
    float16 x (*, K) with at most 4 rows and w (N, K).  Returns float16
    (*, N) on x's device, enqueued on the current stream."""
    torch = _torch()
    device = w.device
    _check_device("x", x, device)
    if bias is not None:
        _check_device("bias", bias, device)
    for name, t in (("x", x), ("w", w), ("bias", bias)):
        if t is not None and t.dtype != torch.float16:
            raise TypeError(f"{name} must be float16")
    N, K = w.shape
    if x.shape[-1] != K:
        raise ValueError(f"x has {x.shape[-1]} features, w has {K}")
    lead = x.shape[:-1]
    x2 = x.reshape(-1, K).contiguous()
    w = w.contiguous()
    if bias is not None:
        if tuple(bias.shape) != (N,):
            raise ValueError(f"bias shape {tuple(bias.shape)} != ({N},)")
        bias = bias.contiguous()
    M = x2.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=device)
    if out is not None:
        _check_device("out", out, device)
        if out.shape != (M, N) or out.dtype != torch.float16 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float16 (M, N) tensor")
    stream = torch.cuda.current_stream(device).cuda_stream
    st = lib().awq_dense_gemv(x2.data_ptr() if M else None, w.data_ptr(),
                              bias.data_ptr() if bias is not None else None,
                              y.data_ptr() if M else None, M, K, N, stream)
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_dense_gemv")
    return y.reshape(*lead, N)


def dequant(qweight, qzeros, scales, group_size: int = 128, out=None):
    """float16 (K, N) dequantised weight through awq_dequant (bit-exact)."""
    torch = _torch()
    device = qweight.device
    for name, t in (("qweight", qweight), ("qzeros", qzeros), ("scales", scales)):
        _check_device(name, t, device)
    if qweight.dtype != torch.int32 or qzeros.dtype != torch.int32:
        raise TypeError("qweight and qzeros must be int32")
    if scales.dtype != torch.float16:
        raise TypeError("scales must be float16")
    K = qweight.shape[0]
    N = qweight.shape[1] * 8
    _check_group_shapes(K, N, group_size, qzeros, scales)
    qweight, qzeros, scales = qweight.contiguous(), qzeros.contiguous(), scales.contiguous()
    if out is not None:
        _check_device("out", out, device)
        if out.shape != (K, N) or out.dtype != torch.float16 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float16 (K, N) tensor")
    w = out if out is not None else torch.empty((K, N), dtype=torch.float16, device=device)
    stream = torch.cuda.current_stream(device).cuda_stream
    st = lib().awq_dequant(qweight.data_ptr(), qzeros.data_ptr(), scales.data_ptr(),
                           w.data_ptr(), K, N, group_size, stream)
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_dequant")
    return w


def _check_map(g_idx, K, device):
    torch = _torch()
    _check_device("g_idx", g_idx, device)
    if g_idx.dtype != torch.int32 or tuple(g_idx.shape) != (K,):
        raise ValueError(f"g_idx must be int32 of shape ({K},)")
    return g_idx.contiguous()


def _check_map_groups(N, qzeros, scales):
    G = scales.shape[0]
    if scales.dim() != 2 or tuple(scales.shape) != (G, N) or tuple(qzeros.shape) != (G, N // 8):
        raise ValueError(f"qzeros {tuple(qzeros.shape)} / scales {tuple(scales.shape)} must be "
                         f"(G, {N // 8}) / (G, {N})")
    return G


def dequant_gidx(qweight, qzeros, scales, g_idx, out=None):
    """float16 (K, N) weight dequantised under a row-to-group map through
    awq_dequant_gidx (bit-exact); g_idx int32 (K,) on the device, G = rows
    of scales."""
    torch = _torch()
    device = qweight.device
    for name, t in (("qweight", qweight), ("qzeros", qzeros), ("scales", scales)):
        _check_device(name, t, device)
    if qweight.dtype != torch.int32 or qzeros.dtype != torch.int32:
        raise TypeError("qweight and qzeros must be int32")
    if scales.dtype != torch.float16:
        raise TypeError("scales must be float16")
    K = qweight.shape[0]
    N = qweight.shape[1] * 8
    G = _check_map_groups(N, qzeros, scales)
    g_idx = _check_map(g_idx, K, device)
    qweight, qzeros, scales = qweight.contiguous(), qzeros.contiguous(), scales.contiguous()
    if out is not None:
        _check_device("out", out, device)
        if out.shape != (K, N) or out.dtype != torch.float16 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float16 (K, N) tensor")
    w = out if out is not None else torch.empty((K, N), dtype=torch.float16, device=device)
    stream = torch.cuda.current_stream(device).cuda_stream
    st = lib().awq_dequant_gidx(qweight.data_ptr(), qzeros.data_ptr(), scales.data_ptr(),
                                g_idx.data_ptr(), w.data_ptr(), K, N, G, stream)
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_dequant_gidx")
    return w


def _prep_x(x, K):
    lead = x.shape[:-1]
    x2 = x.reshape(-1, K)
    if not x2.is_contiguous():
        x2 = x2.contiguous()
    return lead, x2


def _prep_out(out, M, N, device):
    torch = _torch()
    if out is None:
        return torch.empty((M, N), dtype=torch.float16, device=device)
    _check_device("out", out, device)
    if out.shape != (M, N) or out.dtype != torch.float16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float16 (M, N) tensor")
    return out


def gemm_gidx(x, qweight, qzeros, scales, g_idx, bias=None, out=None):
    """y = x . W + bias under any row-to-group map, through awq_gemm_gidx
    (the general kernel).  Returns float16 (*, N)."""
    torch = _torch()
    device = qweight.device
    for name, t in (("x", x), ("qweight", qweight), ("qzeros", qzeros), ("scales", scales)):
        _check_device(name, t, device)
    if x.dtype != torch.float16 or scales.dtype != torch.float16:
        raise TypeError("x and scales must be float16")
    if qweight.dtype != torch.int32 or qzeros.dtype != torch.int32:
        raise TypeError("qweight and qzeros must be int32")
    K = qweight.shape[0]
    N = qweight.shape[1] * 8
    if x.shape[-1] != K:
        raise ValueError(f"x has {x.shape[-1]} features, qweight has {K}")
    G = _check_map_groups(N, qzeros, scales)
    g_idx = _check_map(g_idx, K, device)
    bias = _check_bias(bias, N, device)
    lead, x2 = _prep_x(x, K)
    M = x2.shape[0]
    y = _prep_out(out, M, N, device)
    qweight, qzeros, scales = qweight.contiguous(), qzeros.contiguous(), scales.contiguous()
    stream = torch.cuda.current_stream(device).cuda_stream
    st = lib().awq_gemm_gidx(x2.data_ptr() if M else None, qweight.data_ptr(),
                             qzeros.data_ptr(), scales.data_ptr(), g_idx.data_ptr(),
                             bias.data_ptr() if bias is not None else None,
                             y.data_ptr() if M else None, M, K, N, G, stream)
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_gemm_gidx")
    return y.reshape(*lead, N)


def _check_bias(bias, N, device):
    torch = _torch()
    if bias is None:
        return None
    _check_device("bias", bias, device)
    if bias.dtype != torch.float16:
        raise TypeError("bias must be float16")
    if tuple(bias.shape) != (N,):
        raise ValueError(f"bias shape {tuple(bias.shape)} != ({N},)")
    return bias.contiguous()


def permute_rows(qweight, perm, out=None):
    """qweight[perm] for a packed int32 (K, N/8) weight through
    awq_permute_rows; perm int32 (K,) on the device."""
    torch = _torch()
    device = qweight.device
    _check_device("qweight", qweight, device)
    if qweight.dtype != torch.int32:
        raise TypeError("qweight must be int32")
    K = qweight.shape[0]
    N = qweight.shape[1] * 8
    perm = _check_map(perm, K, device)
    qweight = qweight.contiguous()
    if out is None:
        out = torch.empty_like(qweight)
    else:
        _check_device("out", out, device)
        if out.shape != qweight.shape or out.dtype != torch.int32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous int32 tensor shaped like qweight")
    stream = torch.cuda.current_stream(device).cuda_stream
    st = lib().awq_permute_rows(qweight.data_ptr(), perm.data_ptr(), out.data_ptr(), K, N, stream)
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_permute_rows")
    return out


def prepare_act_order(qweight, g_idx, num_groups: int):
    """Load-time reorder of an activation-order weight: (qweight_sorted,
    perm on the device, group_size).  g_idx may be a host sequence, a numpy
    array or a tensor; every group must hold the same number of rows (else
    ValueError: such maps take gemm_gidx)."""
    torch = _torch()
    if hasattr(g_idx, "detach"):
        g_idx = g_idx.detach().cpu().numpy()
    perm, group_size = gidx_order(g_idx, num_groups)
    if group_size == 0:
        raise ValueError("the groups of this map differ in size; use gemm_gidx")
    perm_dev = torch.from_numpy(perm).to(qweight.device)
    return permute_rows(qweight, perm_dev), perm_dev, group_size


def gemm_act_order(x, perm, qweight_sorted, qzeros, scales, bias=None, group_size: int = 128,
                   out=None, workspace=None):
    """y = x[:, perm] . W_sorted + bias through awq_gemm_act_order (equal to
    the forward of the original activation-order weight).  Returns float16
    (*, N)."""
    torch = _torch()
    device = qweight_sorted.device
    for name, t in (("x", x), ("qweight_sorted", qweight_sorted), ("qzeros", qzeros),
                    ("scales", scales)):
        _check_device(name, t, device)
    if x.dtype != torch.float16 or scales.dtype != torch.float16:
        raise TypeError("x and scales must be float16")
    if qweight_sorted.dtype != torch.int32 or qzeros.dtype != torch.int32:
        raise TypeError("qweight_sorted and qzeros must be int32")
    K = qweight_sorted.shape[0]
    N = qweight_sorted.shape[1] * 8
    if x.shape[-1] != K:
        raise ValueError(f"x has {x.shape[-1]} features, qweight has {K}")
    _check_group_shapes(K, N, group_size, qzeros, scales)
    perm = _check_map(perm, K, device)
    bias = _check_bias(bias, N, device)
    lead, x2 = _prep_x(x, K)
    M = x2.shape[0]
    y = _prep_out(out, M, N, device)
    qweight_sorted = qweight_sorted.contiguous()
    qzeros, scales = qzeros.contiguous(), scales.contiguous()
    stream = torch.cuda.current_stream(device).cuda_stream
    need = act_order_workspace_size(M, K, N, group_size) if M > 0 else 0
    ws = _workspace(device, stream, need) if workspace is None else workspace
    ws_ptr = ws.data_ptr() if ws is not None else None
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = lib().awq_gemm_act_order(x2.data_ptr() if M else None, perm.data_ptr(),
                                  qweight_sorted.data_ptr(), qzeros.data_ptr(),
                                  scales.data_ptr(), bias.data_ptr() if bias is not None else None,
                                  y.data_ptr() if M else None, M, K, N, group_size, ws_ptr,
                                  ws_bytes, stream)
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_gemm_act_order")
    return y.reshape(*lead, N)
