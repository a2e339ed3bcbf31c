"""ctypes binding of libmoe.so (include/moe.h): same names, argument marshalling only.

torch is imported first so that libmoe.so binds to the HIP runtime torch already
loaded (same soname), and torch's streams and device pointers are valid for it.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOSPC, MOE_EUNSUPPORTED, MOE_EHIP = range(5)
MOE_BF16, MOE_FP32 = 0, 1
MOE_GATEUP_INTERLEAVED = 0
MOE_GATEUP_CONCAT = 1
MOE_DEV_BAD_EXPERT, MOE_DEV_OVER_CAPACITY = 1, 2

EXPORTED_SYMBOLS = [
    "moe_build_metadata_workspace", "moe_expert_forward_workspace",
    "moe_expert_backward_workspace", "moe_build_metadata", "moe_expert_forward",
    "moe_expert_backward", "moe_status_string", "moe_time_kernel", "moe_kernel_name",
    "moe_route_workspace", "moe_route", "moe_build_metadata_noalloc",
]
MOE_NOALLOC_SCRATCH_BYTES = 4 << 20
KERNELS = ["meta_hist", "meta_scan", "meta_scatter", "up_swiglu", "down", "combine", "down_bwd",
           "wgrad_down", "up_bwd", "wgrad_up", "combine_dx", "route"]
MOE_ROUTE_SOFTMAX_TOPK, MOE_ROUTE_TOPK_SOFTMAX = 0, 1


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_status_string(status)} (status {status})")


class _CMeta(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("E", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("expert_frequency", ctypes.c_void_p), ("expert_frequency_offset", ctypes.c_void_p),
        ("x_gather_idx", ctypes.c_void_p), ("s_scatter_idx", ctypes.c_void_p),
        ("s_reverse_scatter_idx", ctypes.c_void_p),
        ("num_activated_expert_per_token_offset", ctypes.c_void_p),
        ("router_scores", ctypes.c_void_p), ("status", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """The loaded libmoe.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            raise ImportError(f"{_SO} is missing: build it with __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950); there is no fallback path")
        L = ctypes.CDLL(_SO)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.moe_build_metadata_workspace.restype = sz
        L.moe_build_metadata_workspace.argtypes = [i32, i32, i32]
        L.moe_expert_forward_workspace.restype = sz
        L.moe_expert_forward_workspace.argtypes = [vp, i32, i32, ctypes.c_int]
        L.moe_expert_backward_workspace.restype = sz
        L.moe_expert_backward_workspace.argtypes = [vp, i32, i32, ctypes.c_int]
        L.moe_build_metadata.restype = ctypes.c_int
        L.moe_build_metadata.argtypes = [vp, vp, vp, vp, sz, vp]
        L.moe_build_metadata_noalloc.restype = ctypes.c_int
        L.moe_build_metadata_noalloc.argtypes = [vp, vp, vp, vp]
        L.moe_expert_forward.restype = ctypes.c_int
        L.moe_expert_forward.argtypes = [vp, vp, vp, vp, i32, i32, ctypes.c_int, ctypes.c_int,
                                         vp, vp, vp, sz, vp]
        L.moe_expert_backward.restype = ctypes.c_int
        L.moe_expert_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, ctypes.c_int,
                                          ctypes.c_int, vp, vp, vp, vp, vp, sz, vp]
        L.moe_route_workspace.restype = sz
        L.moe_route_workspace.argtypes = [i32, i32, i32]
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [vp, ctypes.c_int, ctypes.c_int, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_time_kernel.restype = ctypes.c_int
        L.moe_time_kernel.argtypes = [ctypes.c_int, vp, i32, vp]
        L.moe_kernel_name.restype = ctypes.c_char_p
        L.moe_kernel_name.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


class Metadata:
    """Device arrays of moe_metadata (caller-owned torch tensors) and the C struct."""

    def __init__(self, N: int, K: int, E: int, capacity: int | None = None, device="cuda"):
        cap = N * K if capacity is None else int(capacity)
        self.N, self.K, self.E, self.capacity = int(N), int(K), int(E), cap
        i32 = dict(dtype=torch.int32, device=device)
        c = max(cap, 1)
        self.expert_frequency = torch.empty(E, **i32)
        self.expert_frequency_offset = torch.empty(E + 1, **i32)
        self.x_gather_idx = torch.empty(c, **i32)
        self.s_scatter_idx = torch.empty(c, **i32)
        self.s_reverse_scatter_idx = torch.empty(c, **i32)
        self.num_activated_expert_per_token_offset = torch.empty(N + 1, **i32)
        self.router_scores = torch.empty(c, dtype=torch.float32, device=device)
        self.status = torch.empty(1, **i32)
        self.device = self.status.device
        self._c = _CMeta(self.N, self.K, self.E, cap,
                         *[t.data_ptr() for t in (
                             self.expert_frequency, self.expert_frequency_offset,
                             self.x_gather_idx, self.s_scatter_idx, self.s_reverse_scatter_idx,
                             self.num_activated_expert_per_token_offset, self.router_scores,
                             self.status)])

    @property
    def ptr(self):
        return ctypes.byref(self._c)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _dev_on(meta: "Metadata", t, name: str, dtype=None, shape=None):
    """_dev, and the tensor must be on the metadata's device."""
    if isinstance(t, torch.Tensor) and t.device != meta.device:
        raise ValueError(f"{name} is on {t.device}, the metadata on {meta.device}")
    return _dev(t, name, dtype, shape)


def _on(meta: "Metadata", stream):
    """The call runs with the metadata's device current (switched only when another one
    is); an explicit stream must be on it."""
    if stream is not None and stream.device != meta.device:
        raise ValueError(f"stream is on {stream.device}, the metadata on {meta.device}")
    if torch.cuda.current_device() != meta.device.index:
        return torch.cuda.device(meta.device)
    return contextlib.nullcontext()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _workspace(workspace, need: int, device, stream):
    """(tensor, pointer, bytes). A workspace allocated here is tied to the stream the
    call runs on; the caller keeps the tensor alive until after the call."""
    if workspace is not None and workspace.device != torch.device(device):
        raise ValueError(f"workspace is on {workspace.device}, the call on {device}")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
        if stream is not None:
            workspace.record_stream(stream)
    return (workspace, ctypes.c_void_p(workspace.data_ptr()),
            workspace.numel() * workspace.element_size())


def moe_build_metadata_workspace(N: int, K: int, E: int) -> int:
    return int(lib().moe_build_metadata_workspace(N, K, E))


def moe_expert_forward_workspace(meta: Metadata, H: int, I: int, dtype: int = MOE_BF16) -> int:
    return int(lib().moe_expert_forward_workspace(meta.ptr, H, I, dtype))


def moe_expert_backward_workspace(meta: Metadata, H: int, I: int, dtype: int = MOE_BF16) -> int:
    return int(lib().moe_expert_backward_workspace(meta.ptr, H, I, dtype))


def moe_build_metadata(topk_idx, topk_weights, meta: Metadata, workspace=None, stream=None):
    N, K = meta.N, meta.K
    pi = _dev_on(meta, topk_idx, "topk_idx", torch.int32, (N, K))
    pw = _dev_on(meta, topk_weights, "topk_weights", torch.float32, (N, K))
    need = moe_build_metadata_workspace(N, K, meta.E)
    wst, ws, nb = _workspace(workspace, need, topk_idx.device, stream)
    with _on(meta, stream):
        _check(lib().moe_build_metadata(pi, pw, meta.ptr, ws, nb, _stream(stream)),
               "moe_build_metadata")
    return wst


def moe_build_metadata_noalloc(topk_idx, topk_weights, meta: Metadata, stream=None):
    """moe_build_metadata with the library's static per-GPU scratch as its workspace:
    allocates nothing (raises MoeError with MOE_ENOSPC when the build needs more than
    MOE_NOALLOC_SCRATCH_BYTES). Calls overlapping on one GPU race on that scratch."""
    N, K = meta.N, meta.K
    pi = _dev_on(meta, topk_idx, "topk_idx", torch.int32, (N, K))
    pw = _dev_on(meta, topk_weights, "topk_weights", torch.float32, (N, K))
    with _on(meta, stream):
        _check(lib().moe_build_metadata_noalloc(pi, pw, meta.ptr, _stream(stream)),
               "moe_build_metadata_noalloc")


def moe_route_workspace(N: int, K: int, E: int) -> int:
    return int(lib().moe_route_workspace(N, K, E))


def moe_route(logits, meta: Metadata, mode: int = MOE_ROUTE_SOFTMAX_TOPK, renormalize=False,
              topk_idx=None, topk_weights=None, aux_loss=None, workspace=None, stream=None,
              want_aux: bool = True):
    """Router top-K of logits [N,E] (bf16 or fp32) fused with the metadata build into
    meta. Returns (topk_idx [N,K] int32, topk_weights [N,K] fp32, aux_loss [1] fp32 or
    None); output tensors may be passed in."""
    N, K, E = meta.N, meta.K, meta.E
    dev = logits.device
    pl = _dev_on(meta, logits, "logits", logits.dtype, (N, E))
    if topk_idx is None:
        topk_idx = torch.empty(N, K, dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty(N, K, dtype=torch.float32, device=dev)
    if aux_loss is None and want_aux:
        aux_loss = torch.empty(1, dtype=torch.float32, device=dev)
    pi = _dev_on(meta, topk_idx, "topk_idx", torch.int32, (N, K))
    pw = _dev_on(meta, topk_weights, "topk_weights", torch.float32, (N, K))
    pa = None if aux_loss is None else _dev_on(meta, aux_loss, "aux_loss", torch.float32, (1,))
    need = moe_route_workspace(N, K, E)
    wst, ws, nb = _workspace(workspace, need, dev, stream)
    with _on(meta, stream):
        _check(lib().moe_route(pl, _dtype_code(logits), int(mode), int(bool(renormalize)), pi,
                               pw, pa, meta.ptr, ws, nb, _stream(stream)), "moe_route")
    return topk_idx, topk_weights, aux_loss


def moe_expert_forward(meta: Metadata, x, w_up, w_down, out, h_save=None, workspace=None,
                       stream=None, layout: int = MOE_GATEUP_INTERLEAVED):
    N, E = meta.N, meta.E
    H = x.shape[1]
    I = w_down.shape[1]
    dt = _dtype_code(x)
    px = _dev_on(meta, x, "x", x.dtype, (N, H))
    pu = _dev_on(meta, w_up, "w_up", x.dtype, (E, H, 2 * I))
    pd = _dev_on(meta, w_down, "w_down", x.dtype, (E, I, H))
    po = _dev_on(meta, out, "out", x.dtype, (N, H))
    ph = None if h_save is None else _dev_on(meta, h_save, "h_save", x.dtype, (meta.capacity, 2 * I))
    need = moe_expert_forward_workspace(meta, H, I, dt)
    wst, ws, nb = _workspace(workspace, need, x.device, stream)
    with _on(meta, stream):
        _check(lib().moe_expert_forward(meta.ptr, px, pu, pd, H, I, dt, layout, ph, po, ws, nb,
                                        _stream(stream)), "moe_expert_forward")


def moe_expert_backward(meta: Metadata, topk_idx, x, w_up, w_down, h_saved, dout, dx, dw_up,
                        dw_down, d_topk_weights, workspace=None, stream=None,
                        layout: int = MOE_GATEUP_INTERLEAVED):
    N, K, E = meta.N, meta.K, meta.E
    H = x.shape[1]
    I = w_down.shape[1]
    dt = _dtype_code(x)
    args = [
        _dev_on(meta, topk_idx, "topk_idx", torch.int32, (N, K)),
        _dev_on(meta, x, "x", x.dtype, (N, H)),
        _dev_on(meta, w_up, "w_up", x.dtype, (E, H, 2 * I)),
        _dev_on(meta, w_down, "w_down", x.dtype, (E, I, H)),
        _dev_on(meta, h_saved, "h_saved", x.dtype, (meta.capacity, 2 * I)),
        _dev_on(meta, dout, "dout", x.dtype, (N, H)),
    ]
    outs = [
        _dev_on(meta, dx, "dx", x.dtype, (N, H)),
        _dev_on(meta, dw_up, "dw_up", x.dtype, (E, H, 2 * I)),
        _dev_on(meta, dw_down, "dw_down", x.dtype, (E, I, H)),
        _dev_on(meta, d_topk_weights, "d_topk_weights", torch.float32, (N, K)),
    ]
    need = moe_expert_backward_workspace(meta, H, I, dt)
    wst, ws, nb = _workspace(workspace, need, x.device, stream)
    with _on(meta, stream):
        _check(lib().moe_expert_backward(meta.ptr, *args, H, I, dt, layout, *outs, ws, nb,
                                         _stream(stream)), "moe_expert_backward")


def moe_kernel_name(kernel: int) -> str:
    return lib().moe_kernel_name(int(kernel)).decode()


def moe_time_kernel(kernel, events=None) -> int:
    """Bracket the next len(events)//2 launches of `kernel` (an index into KERNELS or
    its name) with the given torch.cuda.Event objects (start, end, start, end, ...).
    events=None stops. Returns how many launches the previous setting bracketed."""
    if isinstance(kernel, str):
        kernel = KERNELS.index(kernel)
    n = ctypes.c_int32(0)
    if events is None:
        _check(lib().moe_time_kernel(int(kernel), None, 0, ctypes.byref(n)), "moe_time_kernel")
        return n.value
    assert len(events) % 2 == 0
    for e in events:
        if not e.cuda_event:  # torch creates the HIP event on its first record
            e.record()
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _keep_alive.append(arr)
    _check(lib().moe_time_kernel(int(kernel), arr, len(events) // 2, ctypes.byref(n)),
           "moe_time_kernel")
    return n.value


_keep_alive = []
