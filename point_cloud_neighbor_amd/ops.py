"""Python binding of the pointops C ABI (include/pointops.h).

Argument marshalling only: shape, dtype and device checks, output allocation
through torch, and the current HIP stream. Every step of the computation runs
in the HIP kernels of ``libpointops.so``; there is no CPU path. Calling an op
without the built library or on a device other than gfx950 raises
``PointopsError``.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpointops.so")

STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "UNSUPPORTED_DEVICE",
          4: "HIP_ERROR"}
KNN_KMAX = 64


class PointopsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise PointopsError(4, f"{_LIB_PATH} is not built (run __graft_entry__.build())")
        lib = ctypes.CDLL(_LIB_PATH)
        i64, vp, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
        lib.pointops_fps.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, ctypes.c_size_t, vp]
        lib.pointops_fps.restype = ctypes.c_int
        lib.pointops_fps_workspace_bytes.argtypes = [i64, i64, i64]
        lib.pointops_fps_workspace_bytes.restype = ctypes.c_size_t
        lib.pointops_knn.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp]
        lib.pointops_knn.restype = ctypes.c_int
        lib.pointops_ball_query.argtypes = [vp, vp, i64, i64, i64, f32, i64, vp, vp, vp]
        lib.pointops_ball_query.restype = ctypes.c_int
        lib.pointops_ball_query_backward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp,
                                                     vp]
        lib.pointops_ball_query_backward.restype = ctypes.c_int
        lib.pointops_device_check.argtypes = [ctypes.c_int]
        lib.pointops_device_check.restype = ctypes.c_int
        lib.pointops_status_string.argtypes = [ctypes.c_int]
        lib.pointops_status_string.restype = ctypes.c_char_p
        lib.pointops_last_error.argtypes = []
        lib.pointops_last_error.restype = ctypes.c_char_p
        lib.pointops_abi_version.argtypes = []
        lib.pointops_abi_version.restype = ctypes.c_int
        _lib = lib
        return lib


def _check(rc: int):
    if rc != 0:
        raise PointopsError(rc, _load().pointops_last_error().decode())


def _points(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise PointopsError(3, f"{name} is on {t.device}; pointops runs on the GPU only")
    if t.dtype != torch.float32:
        raise PointopsError(1, f"{name} must be float32, got {t.dtype}")
    if t.dim() != 3 or t.shape[-1] != 3:
        raise PointopsError(1, f"{name} must have shape (B, n, 3), got {tuple(t.shape)}")
    return t.contiguous()


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def device_check(device=None) -> None:
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    _check(_load().pointops_device_check(dev.index or 0))


def fps_workspace_bytes(B: int, N: int, M: int) -> int:
    return int(_load().pointops_fps_workspace_bytes(B, N, M))


def furthest_point_sample(xyz: torch.Tensor, npoint: int, start_idx: int = 0,
                          return_xyz: bool = False, workspace: torch.Tensor | None = None):
    """Farthest point sampling of (B, N, 3) float32 clouds -> int64 (B, npoint)
    (and the sampled coordinates (B, npoint, 3) when ``return_xyz``)."""
    lib = _load()
    xyz = _points(xyz, "xyz")
    B, N, _ = xyz.shape
    with torch.cuda.device(xyz.device):
        out = torch.empty((B, npoint), dtype=torch.int64, device=xyz.device)
        oxyz = torch.empty((B, npoint, 3), dtype=torch.float32, device=xyz.device) if return_xyz else None
        need = int(lib.pointops_fps_workspace_bytes(B, N, npoint))
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=xyz.device)
        rc = lib.pointops_fps(xyz.data_ptr(), B, N, npoint, int(start_idx), out.data_ptr(),
                              oxyz.data_ptr() if oxyz is not None else None,
                              workspace.data_ptr(), workspace.numel(), _stream(xyz.device))
        _check(rc)
    return (out, oxyz) if return_xyz else out


def knn(query: torch.Tensor, ref: torch.Tensor, k: int):
    """k nearest neighbours -> (Euclidean distance float32, int64 index), (B, Q, k)."""
    lib = _load()
    query = _points(query, "query")
    ref = _points(ref, "ref")
    if query.device != ref.device or query.shape[0] != ref.shape[0]:
        raise PointopsError(1, "query and ref must share the device and the batch size")
    B, Q, _ = query.shape
    P = ref.shape[1]
    with torch.cuda.device(query.device):
        dist = torch.empty((B, Q, k), dtype=torch.float32, device=query.device)
        idx = torch.empty((B, Q, k), dtype=torch.int64, device=query.device)
        rc = lib.pointops_knn(query.data_ptr(), ref.data_ptr(), B, Q, P, int(k), dist.data_ptr(),
                              idx.data_ptr(), _stream(query.device))
        _check(rc)
    return dist, idx


def ball_query(query: torch.Tensor, ref: torch.Tensor, radius: float, K: int):
    """First K references within ``radius`` in input order -> (squared distance
    float32, int64 index with -1 padding), (B, Q, K). ``radius`` is rounded to
    float32 first (the threshold is fl32(fl32(r) * fl32(r))).

    When grad mode is on and ``query`` or ``ref`` requires grad, the squared
    distances are differentiable with respect to both coordinate tensors (the
    backward runs ``ball_query_backward``); the indices are not."""
    if torch.is_grad_enabled() and (getattr(query, "requires_grad", False)
                                    or getattr(ref, "requires_grad", False)):
        return _BallQueryFn.apply(query, ref, radius, K)
    return _ball_query(query, ref, radius, K)


def _ball_query(query: torch.Tensor, ref: torch.Tensor, radius: float, K: int):
    lib = _load()
    query = _points(query, "query")
    ref = _points(ref, "ref")
    if query.device != ref.device or query.shape[0] != ref.shape[0]:
        raise PointopsError(1, "query and ref must share the device and the batch size")
    B, Q, _ = query.shape
    P = ref.shape[1]
    with torch.cuda.device(query.device):
        d2 = torch.empty((B, Q, K), dtype=torch.float32, device=query.device)
        idx = torch.empty((B, Q, K), dtype=torch.int64, device=query.device)
        rc = lib.pointops_ball_query(query.data_ptr(), ref.data_ptr(), B, Q, P,
                                     ctypes.c_float(float(radius)), int(K), d2.data_ptr(),
                                     idx.data_ptr(), _stream(query.device))
        _check(rc)
    return d2, idx


def ball_query_backward(query: torch.Tensor, ref: torch.Tensor, idx: torch.Tensor,
                        grad_dist2: torch.Tensor, need_query: bool = True,
                        need_ref: bool = True):
    """Gradients of L through Ball Query's squared distances, given
    G = dL/dS (B, Q, K) and the forward's indices -> (grad_query (B, Q, 3) or
    None, grad_ref (B, P, 3) or None), float32. Slots with a negative index
    contribute nothing."""
    lib = _load()
    query = _points(query, "query")
    ref = _points(ref, "ref")
    if query.device != ref.device or query.shape[0] != ref.shape[0]:
        raise PointopsError(1, "query and ref must share the device and the batch size")
    B, Q, _ = query.shape
    P = ref.shape[1]
    if idx.dim() != 3 or tuple(idx.shape[:2]) != (B, Q) or idx.dtype != torch.int64:
        raise PointopsError(1, f"idx must be int64 of shape (B, Q, K), got {idx.dtype} "
                               f"{tuple(idx.shape)}")
    K = idx.shape[2]
    if grad_dist2.shape != idx.shape or grad_dist2.dtype != torch.float32:
        raise PointopsError(1, f"grad_dist2 must be float32 of shape {tuple(idx.shape)}")
    if idx.device != query.device or grad_dist2.device != query.device:
        raise PointopsError(1, "idx and grad_dist2 must be on the device of query")
    idx = idx.contiguous()
    grad_dist2 = grad_dist2.contiguous()
    with torch.cuda.device(query.device):
        gq = torch.empty_like(query) if need_query else None
        gx = torch.empty_like(ref) if need_ref else None
        rc = lib.pointops_ball_query_backward(
            query.data_ptr(), ref.data_ptr(), idx.data_ptr(), grad_dist2.data_ptr(), B, Q, P,
            K, gq.data_ptr() if gq is not None else None,
            gx.data_ptr() if gx is not None else None, _stream(query.device))
        _check(rc)
    return gq, gx


class _BallQueryFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, query, ref, radius, K):
        d2, idx = _ball_query(query, ref, radius, K)
        ctx.save_for_backward(query, ref, idx)
        ctx.mark_non_differentiable(idx)
        return d2, idx

    @staticmethod
    def backward(ctx, grad_d2, grad_idx):
        query, ref, idx = ctx.saved_tensors
        if grad_d2 is None:
            return None, None, None, None
        gq, gx = ball_query_backward(query, ref, idx, grad_d2, ctx.needs_input_grad[0],
                                     ctx.needs_input_grad[1])
        return gq, gx, None, None
