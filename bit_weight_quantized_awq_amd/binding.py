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
AWQ_ERROR_SCRATCH = 6
AWQ_NOALLOC_SCRATCH_BYTES = 16 << 20

AWQ_OPT_FORCE_PATH = 1
AWQ_OPT_DECODE_STEPS = 2
AWQ_OPT_DECODE_GATHER_MAX_M = 3
AWQ_OPT_PREFILL_BM = 4
AWQ_OPT_PREFILL_BN = 5
AWQ_OPT_PREFILL_SPLITS = 6
AWQ_OPT_DECODE_WAVES = 7
AWQ_OPT_PREFILL_PACKED = 8
AWQ_OPT_AUTO = -1
OPTIONS = {"force_path": AWQ_OPT_FORCE_PATH, "decode_steps": AWQ_OPT_DECODE_STEPS,
           "decode_gather_max_m": AWQ_OPT_DECODE_GATHER_MAX_M,
           "prefill_bm": AWQ_OPT_PREFILL_BM, "prefill_bn": AWQ_OPT_PREFILL_BN,
           "prefill_splits": AWQ_OPT_PREFILL_SPLITS, "decode_waves": AWQ_OPT_DECODE_WAVES,
           "prefill_packed": AWQ_OPT_PREFILL_PACKED}

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
    "awq_set_option": (ctypes.c_int, [ctypes.c_int, _i64]),
    "awq_get_option": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_int64)]),
    "awq_gemm_workspace_size": (ctypes.c_size_t, [_i64, _i64, _i64, _i64]),
    "awq_gemm_plan": (ctypes.c_int, [_i64, _i64, _i64, _i64, _vp, _vp, _vp,
                                     ctypes.POINTER(ctypes.c_int),
                                     ctypes.POINTER(ctypes.c_size_t)]),
    "awq_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                _vp, ctypes.c_size_t, _vp]),
    "awq_gemm_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                        _vp]),
    "awq_dequant": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "awq_dense_gemv": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "awq_dequant_gidx": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "awq_gemm_gidx": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                     _i64, _vp]),
    "awq_gidx_layout": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64,
                                       ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_int64)]),
    "awq_gather_rows": (ctypes.c_int, [_vp, _i64, _vp, _vp, _i64, _i64, _vp]),
    "awq_gemm_sorted_workspace_size": (ctypes.c_size_t, [_i64, _i64, _i64, _i64]),
    "awq_gemm_sorted": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
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


_ws_need: dict = {}


def _gemm_workspace_need(M: int, K: int, N: int, group_size: int) -> int:
    """awq_gemm_workspace_size, remembered per shape (it depends on the shape
    and the planner overrides only; set_option clears the memory), so a
    forward makes a single C-ABI call."""
    key = (M, K, N, group_size)
    need = _ws_need.get(key)
    if need is None:
        need = _ws_need[key] = gemm_workspace_size(M, K, N, group_size)
    return need


def _option_id(name):
    if isinstance(name, int):
        return name
    try:
        return OPTIONS[name]
    except KeyError:
        raise ValueError(f"unknown option {name!r}; known: {sorted(OPTIONS)}") from None


def _option_value(opt, value):
    if value is None:
        return AWQ_OPT_AUTO
    if opt == AWQ_OPT_FORCE_PATH and isinstance(value, str):
        names = {v: k for k, v in PATH_NAMES.items()}
        if value not in names:
            raise ValueError(f"unknown kernel family {value!r}")
        return names[value]
    return int(value)


def set_option(name, value) -> None:
    """awq_set_option: a process-wide planner override (tests and tuning).
    name is an awq_option value or one of OPTIONS' keys; value None restores
    the planner's own choice; force_path also takes a family name."""
    opt = _option_id(name)
    st = lib().awq_set_option(opt, _option_value(opt, value))
    if st != AWQ_SUCCESS:
        raise AwqError(st, f"awq_set_option({name!r}, {value!r})")
    _ws_need.clear()   # an override can change a shape's workspace need


def get_option(name) -> int:
    """awq_get_option: the current override (AWQ_OPT_AUTO when none)."""
    v = ctypes.c_int64(0)
    st = lib().awq_get_option(_option_id(name), ctypes.byref(v))
    if st != AWQ_SUCCESS:
        raise AwqError(st, f"awq_get_option({name!r})")
    return v.value


class options:
    """Context manager that sets planner overrides and restores the previous
    values on exit: ``with options(force_path="prefill", prefill_bm=64): ...``."""

    def __init__(self, **kw):
        self._kw = kw
        self._old = {}

    def __enter__(self):
        for k, v in self._kw.items():
            self._old[k] = get_option(k)
            set_option(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self._old.items():
            lib().awq_set_option(_option_id(k), v)
        _ws_need.clear()
        return False


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


def gidx_layout(g_idx, num_groups: int):
    """Host-only awq_gidx_layout: (perm, block_group, block_rows) for a
    row-to-group map given as a sequence or numpy array of K integers.
    perm (int32, rows of the sorted weight) is the input row placed j-th or
    -1 for a null row; block_group (int32) is the group of each block of
    block_rows rows."""
    import numpy as np
    g = np.ascontiguousarray(np.asarray(g_idx), dtype=np.int32)
    if g.ndim != 1 or g.shape[0] == 0:
        raise ValueError("g_idx must be a non-empty 1-D sequence")
    K = g.shape[0]
    rows, brows, blocks = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
    st = lib().awq_gidx_layout(g.ctypes.data, K, num_groups, None, 0, None, 0,
                               ctypes.byref(rows), ctypes.byref(brows), ctypes.byref(blocks))
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_gidx_layout")
    perm = np.empty(rows.value, dtype=np.int32)
    block_group = np.empty(blocks.value, dtype=np.int32)
    st = lib().awq_gidx_layout(g.ctypes.data, K, num_groups, perm.ctypes.data, perm.size,
                               block_group.ctypes.data, block_group.size, ctypes.byref(rows),
                               ctypes.byref(brows), ctypes.byref(blocks))
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_gidx_layout")
    return perm, block_group, brows.value


def sorted_workspace_size(M: int, rows: int, N: int, block_rows: int) -> int:
    return lib().awq_gemm_sorted_workspace_size(M, rows, N, block_rows)


# --------------------------------------------------------------------- torch
def _torch():
    import torch
    return torch


_workspaces: dict = {}
_retired_workspaces: list = []
_ws_lock = threading.Lock()


def _workspace(device, stream_ptr: int, nbytes: int):
    """A zero-filled workspace per (device, stream), grown on demand.  The
    kernels leave it zeroed where it must start at zero, so one buffer serves
    every later call on that stream.  A buffer replaced by a larger one is
    kept alive until the process ends: a HIP graph captured earlier may still
    hold its address, and freeing it would let the allocator hand that memory
    to other tensors the replay would then overwrite."""
    torch = _torch()
    if nbytes == 0:
        return None
    key = (device.index, stream_ptr)
    with _ws_lock:
        buf = _workspaces.get(key)
        if buf is None or buf.numel() < nbytes:
            if buf is not None:
                _retired_workspaces.append(buf)
            buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            _workspaces[key] = buf
        return buf


def _current_stream(device):
    """The raw hipStream_t of the current stream on `device`."""
    torch = _torch()
    return torch._C._cuda_getCurrentRawStream(device.index)


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
    stream = _current_stream(device)
    if workspace is None:
        ws = _workspace(device, stream, _gemm_workspace_need(M, K, N, group_size) if M else 0)
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


def gemm_noalloc(x, qweight, qzeros, scales, bias=None, group_size: int = 128, out=None):
    """gemm through awq_gemm_noalloc: no workspace, the library's fixed
    per-device scratch instead (for code that cannot allocate, e.g. under
    graph capture; pass `out` so that nothing is allocated here either).
    Calls that may overlap on one device race on that scratch."""
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
    _check_group_shapes(K, N, group_size, qzeros, scales)
    if not (qweight.is_contiguous() and qzeros.is_contiguous() and scales.is_contiguous()):
        raise ValueError("qweight, qzeros and scales must be contiguous")
    bias = _check_bias(bias, N, device)
    lead, x2 = _prep_x(x, K)
    M = x2.shape[0]
    y = _prep_out(out, M, N, device)
    st = lib().awq_gemm_noalloc(x2.data_ptr() if M else None, qweight.data_ptr(),
                                qzeros.data_ptr(), scales.data_ptr(),
                                bias.data_ptr() if bias is not None else None,
                                y.data_ptr() if M else None, M, K, N, group_size,
                                _current_stream(device))
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_gemm_noalloc")
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
    stream = _current_stream(device)
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
    stream = _current_stream(device)
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
    stream = _current_stream(device)
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
    stream = _current_stream(device)
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


def gather_rows(src, idx, out=None):
    """out[j] = src[idx[j]] (zero rows for indices out of range) through
    awq_gather_rows, for a 2-D tensor whose rows are whole 4-byte words;
    idx int32 on the device."""
    torch = _torch()
    device = src.device
    _check_device("src", src, device)
    _check_device("idx", idx, device)
    if src.dim() != 2 or idx.dim() != 1 or idx.dtype != torch.int32:
        raise ValueError("src must be 2-D and idx a 1-D int32 tensor")
    src = src.contiguous()
    idx = idx.contiguous()
    rows = idx.shape[0]
    row_bytes = src.shape[1] * src.element_size()
    if out is None:
        out = torch.empty((rows, src.shape[1]), dtype=src.dtype, device=device)
    else:
        _check_device("out", out, device)
        if out.shape != (rows, src.shape[1]) or out.dtype != src.dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous tensor of shape (len(idx), src.shape[1])")
    stream = _current_stream(device)
    st = lib().awq_gather_rows(src.data_ptr(), src.shape[0], idx.data_ptr(), out.data_ptr(),
                               rows, row_bytes, stream)
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_gather_rows")
    return out


class SortedWeight:
    """A weight under a row-to-group map, rebuilt as a grouped weight:
    qweight (rows, N/8), qzeros and scales (rows / block_rows, ...), perm
    (rows, int32 on the device: input row of each sorted row, -1 for null
    rows) and in_features (K of x)."""

    def __init__(self, qweight, qzeros, scales, perm, block_rows, in_features):
        self.qweight = qweight
        self.qzeros = qzeros
        self.scales = scales
        self.perm = perm
        self.block_rows = block_rows
        self.in_features = in_features

    @property
    def rows(self):
        return self.qweight.shape[0]


def prepare_gidx(qweight, qzeros, scales, g_idx):
    """Load-time rebuild of (qweight, qzeros, scales) under a row-to-group
    map g_idx (K integers: host sequence, numpy array or tensor) into a
    SortedWeight: awq_gidx_layout on the host, awq_gather_rows on the
    device."""
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
    if hasattr(g_idx, "detach"):
        g_idx = g_idx.detach().cpu().numpy()
    if len(g_idx) != K:
        raise ValueError(f"g_idx has {len(g_idx)} entries, qweight has {K} rows")
    perm, block_group, block_rows = gidx_layout(g_idx, G)
    perm_dev = torch.from_numpy(perm).to(device)
    bg_dev = torch.from_numpy(block_group).to(device)
    return SortedWeight(gather_rows(qweight, perm_dev), gather_rows(qzeros, bg_dev),
                        gather_rows(scales, bg_dev), perm_dev, block_rows, K)


def gemm_sorted(x, w, bias=None, out=None, workspace=None):
    """y = x[:, perm] . W_sorted + bias through awq_gemm_sorted, for a
    SortedWeight w (equal to the forward of the original weight under its
    map).  Returns float16 (*, N)."""
    torch = _torch()
    device = w.qweight.device
    _check_device("x", x, device)
    if x.dtype != torch.float16:
        raise TypeError("x must be float16")
    K_in = w.in_features
    rows = w.rows
    N = w.qweight.shape[1] * 8
    if x.shape[-1] != K_in:
        raise ValueError(f"x has {x.shape[-1]} features, the weight has {K_in}")
    bias = _check_bias(bias, N, device)
    lead, x2 = _prep_x(x, K_in)
    M = x2.shape[0]
    y = _prep_out(out, M, N, device)
    stream = _current_stream(device)
    need = sorted_workspace_size(M, rows, N, w.block_rows) if M > 0 else 0
    ws = _workspace(device, stream, need) if workspace is None else workspace
    ws_ptr = ws.data_ptr() if ws is not None else None
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = lib().awq_gemm_sorted(x2.data_ptr() if M else None, w.perm.data_ptr(),
                               w.qweight.data_ptr(), w.qzeros.data_ptr(), w.scales.data_ptr(),
                               bias.data_ptr() if bias is not None else None,
                               y.data_ptr() if M else None, M, K_in, rows, N, w.block_rows,
                               ws_ptr, ws_bytes, stream)
    if st != AWQ_SUCCESS:
        raise AwqError(st, "awq_gemm_sorted")
    return y.reshape(*lead, N)
