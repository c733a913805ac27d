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

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpointops.so")

STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "UNSUPPORTED_DEVICE",
          4: "HIP_ERROR", 5: "EXEC_TIMEOUT"}
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
        lib.pointops_fps_status.argtypes = [vp, ctypes.c_size_t, vp, vp]
        lib.pointops_fps_status.restype = ctypes.c_int
        lib.pointops_knn.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp, ctypes.c_size_t,
                                     vp]
        lib.pointops_knn_workspace_bytes.argtypes = [i64, i64, i64]
        lib.pointops_knn_workspace_bytes.restype = ctypes.c_size_t
        lib.pointops_knn.restype = ctypes.c_int
        lib.pointops_knn_search.argtypes = [i64, i64, i64, i64, ctypes.c_int]
        lib.pointops_knn_search.restype = ctypes.c_int
        lib.pointops_ball_query_search.argtypes = [i64, i64, i64, i64, ctypes.c_int]
        lib.pointops_ball_query_search.restype = ctypes.c_int
        lib.pointops_ball_query.argtypes = [vp, vp, i64, i64, i64, f32, i64, vp, vp, vp,
                                            ctypes.c_size_t, vp]
        lib.pointops_ball_query_workspace_bytes.argtypes = [i64, i64, i64]
        lib.pointops_ball_query_workspace_bytes.restype = ctypes.c_size_t
        lib.pointops_ball_query.restype = ctypes.c_int
        lib.pointops_ball_query_backward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp,
                                                     vp, ctypes.c_size_t, vp]
        lib.pointops_ball_query_backward.restype = ctypes.c_int
        lib.pointops_ball_query_backward_workspace_bytes.argtypes = [i64, i64, i64, i64]
        lib.pointops_ball_query_backward_workspace_bytes.restype = ctypes.c_size_t
        lib.pointops_ragged_workspace_bytes.argtypes = [i64]
        lib.pointops_ragged_workspace_bytes.restype = ctypes.c_size_t
        lib.pointops_knn_ragged_workspace_bytes.argtypes = [vp, vp, i64, i64]
        lib.pointops_knn_ragged_workspace_bytes.restype = ctypes.c_size_t
        lib.pointops_ball_query_ragged_workspace_bytes.argtypes = [vp, vp, i64, i64]
        lib.pointops_ball_query_ragged_workspace_bytes.restype = ctypes.c_size_t
        lib.pointops_knn_ragged.argtypes = [vp, i64, vp, vp, vp, i64, vp, vp, i64, i64,
                                            ctypes.c_int, vp, vp, vp, ctypes.c_size_t, vp]
        lib.pointops_knn_ragged.restype = ctypes.c_int
        lib.pointops_ball_query_ragged.argtypes = [vp, i64, vp, vp, vp, i64, vp, vp, i64, f32,
                                                   i64, ctypes.c_int, vp, vp, vp,
                                                   ctypes.c_size_t, vp]
        lib.pointops_ball_query_ragged.restype = ctypes.c_int
        lib.pointops_fps_ragged_workspace_bytes.argtypes = [vp, vp, i64]
        lib.pointops_fps_ragged_workspace_bytes.restype = ctypes.c_size_t
        lib.pointops_fps_ragged.argtypes = [vp, i64, vp, vp, vp, i64, vp, vp, i64, vp, vp,
                                            ctypes.c_int, vp, ctypes.c_size_t, vp]
        lib.pointops_fps_ragged.restype = ctypes.c_int
        lib.pointops_three_nn.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, ctypes.c_size_t, vp]
        lib.pointops_three_nn.restype = ctypes.c_int
        lib.pointops_three_nn_workspace_bytes.argtypes = [i64, i64, i64]
        lib.pointops_three_nn_workspace_bytes.restype = ctypes.c_size_t
        lib.pointops_chamfer_workspace_bytes.argtypes = [i64, i64, i64]
        lib.pointops_chamfer_workspace_bytes.restype = ctypes.c_size_t
        ci = ctypes.c_int
        lib.pointops_chamfer.argtypes = [vp, vp, i64, i64, i64, vp, vp, ci, ci, ci, vp, vp, vp,
                                         vp, vp, vp, ctypes.c_size_t, vp]
        lib.pointops_chamfer.restype = ctypes.c_int
        lib.pointops_chamfer_backward.argtypes = [vp, vp, i64, i64, i64, vp, vp, ci, ci, ci, vp,
                                                  vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.pointops_chamfer_backward.restype = ctypes.c_int
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


def fps_status(workspace: torch.Tensor) -> int:
    """Wait for the current stream and raise ``PointopsError`` (EXEC_TIMEOUT)
    if the last FPS call that sampled with ``workspace`` gave up a bounded
    wait (its unreached output slots then hold -1). Returns the number of
    cross-workgroup exchanges that call's first cloud made."""
    n = ctypes.c_int64(0)
    with torch.cuda.device(workspace.device):
        _check(_load().pointops_fps_status(workspace.data_ptr(), workspace.numel(),
                                           ctypes.byref(n), _stream(workspace.device)))
    return int(n.value)


def furthest_point_sample(xyz: torch.Tensor, npoint: int, start_idx: int = 0,
                          return_xyz: bool = False, workspace: torch.Tensor | None = None,
                          check: bool = True):
    """Farthest point sampling of (B, N, 3) float32 clouds -> int64 (B, npoint)
    (and the sampled coordinates (B, npoint, 3) when ``return_xyz``).

    ``check`` (default) waits for the launch and raises ``PointopsError`` if
    it gave up a bounded wait between its workgroups. With ``check=False`` the
    call stays asynchronous; pass a ``workspace`` and call
    ``fps_status(workspace)`` later."""
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
        if check and need > 0 and B > 0 and npoint > 0:
            fps_status(workspace)
    return (out, oxyz) if return_xyz else out


def knn(query: torch.Tensor, ref: torch.Tensor, k: int, grid: bool = True):
    """k nearest neighbours -> (Euclidean distance float32, int64 index), (B, Q, k).
    ``grid`` lets large calls sort the clouds into a grid and skip far
    references (same results)."""
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
        nbytes = int(lib.pointops_knn_workspace_bytes(B, Q, P)) if grid else 0
        ws = torch.empty(nbytes, dtype=torch.uint8, device=query.device) if nbytes else None
        rc = lib.pointops_knn(query.data_ptr(), ref.data_ptr(), B, Q, P, int(k), dist.data_ptr(),
                              idx.data_ptr(), ws.data_ptr() if ws is not None else None, nbytes,
                              _stream(query.device))
        _check(rc)
    return dist, idx


KNN_SEARCHES = {0: "full scan, one query per lane", 1: "full scan, queries per wave",
                2: "grid"}


def knn_search(B: int, Q: int, P: int, k: int, grid: bool = True) -> str:
    """Which search ``knn`` takes for this shape on the current device (a key
    of the library's choice; every search gives the same results)."""
    rc = int(_load().pointops_knn_search(B, Q, P, int(k), 1 if grid else 0))
    if rc < 0:
        _check(-rc)
    return KNN_SEARCHES[rc]


BQ_SEARCHES = {0: "scan", 1: "culled scan", 2: "culled scan, then grid pass"}


def ball_query_search(B: int, Q: int, P: int, K: int, cull: bool = True) -> str:
    """Which search ``ball_query`` takes for this shape (a key of the
    library's choice; every search gives the same results)."""
    rc = int(_load().pointops_ball_query_search(B, Q, P, int(K), 1 if cull else 0))
    if rc < 0:
        _check(-rc)
    return BQ_SEARCHES[rc]


def ball_query(query: torch.Tensor, ref: torch.Tensor, radius: float, K: int,
               cull: bool = True):
    """First K references within ``radius`` in input order -> (squared distance
    float32, int64 index with -1 padding), (B, Q, K). ``radius`` is rounded to
    float32 first (the threshold is fl32(fl32(r) * fl32(r))).

    When grad mode is on and ``query`` or ``ref`` requires grad, the squared
    distances are differentiable with respect to both coordinate tensors (the
    backward runs ``ball_query_backward``); the indices are not. ``cull`` lets
    the call skip reference blocks whose bounding box is out of reach (same
    results; faster on spatially sorted references)."""
    if torch.is_grad_enabled() and (getattr(query, "requires_grad", False)
                                    or getattr(ref, "requires_grad", False)):
        return _BallQueryFn.apply(query, ref, radius, K, cull)
    return _ball_query(query, ref, radius, K, cull)


def _ball_query(query: torch.Tensor, ref: torch.Tensor, radius: float, K: int, cull: bool):
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
        nbytes = int(lib.pointops_ball_query_workspace_bytes(B, Q, P)) if cull else 0
        ws = torch.empty(nbytes, dtype=torch.uint8, device=query.device) if nbytes else None
        rc = lib.pointops_ball_query(query.data_ptr(), ref.data_ptr(), B, Q, P,
                                     ctypes.c_float(float(radius)), int(K), d2.data_ptr(),
                                     idx.data_ptr(), ws.data_ptr() if ws is not None else None,
                                     nbytes, _stream(query.device))
        _check(rc)
    return d2, idx


def ball_query_backward(query: torch.Tensor, ref: torch.Tensor, idx: torch.Tensor,
                        grad_dist2: torch.Tensor, need_query: bool = True,
                        need_ref: bool = True):
    """Gradients of L through Ball Query's squared distances, given
    G = dL/dS (B, Q, K) and the forward's indices -> (grad_query (B, Q, 3) or
    None, grad_ref (B, P, 3) or None), float32. Slots with a negative index
    contribute nothing. A cloud queried by its own points (one tensor for
    both) gets the workspace of the self-query mode."""
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
        ws = None
        if need_ref and query.data_ptr() == ref.data_ptr() and Q == P:
            nb = lib.pointops_ball_query_backward_workspace_bytes(B, Q, P, K)
            ws = torch.empty(nb, dtype=torch.uint8, device=query.device) if nb else None
        rc = lib.pointops_ball_query_backward(
            query.data_ptr(), ref.data_ptr(), idx.data_ptr(), grad_dist2.data_ptr(), B, Q, P,
            K, gq.data_ptr() if gq is not None else None,
            gx.data_ptr() if gx is not None else None,
            ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
            _stream(query.device))
        _check(rc)
    return gq, gx


class _BallQueryFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, query, ref, radius, K, cull):
        d2, idx = _ball_query(query, ref, radius, K, cull)
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
        return gq, gx, None, None, None


# ------------------------------------------------------------------ ragged batches
#
# A cloud is a segment (offset, count) of a flat (rows, 3) point tensor. The
# offsets are host arrays in the C ABI; here they may be given as lists, numpy
# arrays or tensors (a device tensor is copied to the host, which waits for
# the device).

def _host_i64(a, name) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int64))
    if a.ndim != 1:
        raise PointopsError(1, f"{name} must be one-dimensional")
    return a


def _flat_points(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise PointopsError(3, f"{name} is on {t.device}; pointops runs on the GPU only")
    if t.dtype != torch.float32:
        raise PointopsError(1, f"{name} must be float32, got {t.dtype}")
    if t.dim() != 2 or t.shape[-1] != 3:
        raise PointopsError(1, f"{name} must have shape (rows, 3), got {tuple(t.shape)}")
    return t.contiguous()


def _ptr_segments(ptr, name):
    ptr = _host_i64(ptr, name)
    if len(ptr) < 1:
        raise PointopsError(1, f"{name} needs at least one entry")
    return np.ascontiguousarray(ptr[:-1]), np.ascontiguousarray(np.diff(ptr))


def _vp(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None and a.size else None


def _search_ragged(fn, query, q_off, q_cnt, ref, r_off, r_cnt, width, extra, global_index,
                   pad_dist, out=None, ws_fn=None):
    """ws_fn: the workspace-size call that gives the grid search its room
    when it pays (pointops_knn_ragged_workspace_bytes or
    pointops_ball_query_ragged_workspace_bytes, with k or K = width); None
    for the table alone (the full scans)."""
    lib = _load()
    query = _flat_points(query, "query")
    ref = _flat_points(ref, "ref")
    if query.device != ref.device:
        raise PointopsError(1, "query and ref must share the device")
    q_off, q_cnt = _host_i64(q_off, "q_off"), _host_i64(q_cnt, "q_cnt")
    r_off, r_cnt = _host_i64(r_off, "r_off"), _host_i64(r_cnt, "r_cnt")
    B = len(q_off)
    if not (len(q_cnt) == len(r_off) == len(r_cnt) == B):
        raise PointopsError(1, "segment arrays must all have B entries")
    rows = query.shape[0]
    with torch.cuda.device(query.device):
        if out is None:
            dist = torch.full((rows, width), pad_dist, dtype=torch.float32, device=query.device)
            idx = torch.full((rows, width), -1, dtype=torch.int64, device=query.device)
        else:
            dist, idx = out
        if ws_fn is None:
            need = int(lib.pointops_ragged_workspace_bytes(B))
        else:
            need = int(ws_fn(_vp(q_cnt), _vp(r_cnt), B, int(width)))
            if need == 0:
                raise PointopsError(1, "invalid segment counts")
        ws = torch.empty(max(1, need), dtype=torch.uint8, device=query.device)
        rc = fn(query.data_ptr(), rows, _vp(q_off), _vp(q_cnt), ref.data_ptr(), ref.shape[0],
                _vp(r_off), _vp(r_cnt), B, *extra, int(bool(global_index)), dist.data_ptr(),
                idx.data_ptr(), ws.data_ptr(), ws.numel(), _stream(query.device))
        _check(rc)
    return dist, idx


def knn_ragged(query: torch.Tensor, q_ptr, ref: torch.Tensor, r_ptr, k: int,
               global_index: bool = True, grid: bool = True):
    """kNN within each cloud of a flat batch: cloud b has query rows
    q_ptr[b]..q_ptr[b+1] and reference rows r_ptr[b]..r_ptr[b+1] ->
    (dist, idx), (query rows, k). Indices are reference rows (or local indices);
    slots a cloud with fewer than k references cannot fill hold (+inf, -1).
    grid=False withholds the grid search's workspace (full scans only)."""
    q_off, q_cnt = _ptr_segments(q_ptr, "q_ptr")
    r_off, r_cnt = _ptr_segments(r_ptr, "r_ptr")
    lib = _load()
    return _search_ragged(lib.pointops_knn_ragged, query, q_off, q_cnt, ref, r_off, r_cnt,
                          int(k), (int(k),), global_index, float("inf"),
                          ws_fn=lib.pointops_knn_ragged_workspace_bytes if grid else None)


def knn_ragged_uses_grid(q_cnt, r_cnt, k: int) -> bool:
    """True when pointops_knn_ragged takes the grid search for these counts
    (given the workspace pointops_knn_ragged_workspace_bytes asks for)."""
    lib = _load()
    q_cnt, r_cnt = _host_i64(q_cnt, "q_cnt"), _host_i64(r_cnt, "r_cnt")
    B = len(q_cnt)
    return int(lib.pointops_knn_ragged_workspace_bytes(_vp(q_cnt), _vp(r_cnt), B, int(k))) > \
        int(lib.pointops_ragged_workspace_bytes(B))


def ball_query_ragged(query: torch.Tensor, q_ptr, ref: torch.Tensor, r_ptr, radius: float,
                      K: int, global_index: bool = True, grid: bool = True):
    """First-K Ball Query within each cloud of a flat batch -> (dist2, idx),
    (query rows, K), indices as reference rows (or local), (-1, 0) padding.
    Differentiable like ``ball_query`` when an input requires grad and the
    indices are global. grid=False withholds the grid pass's workspace (the
    index-order scan only)."""
    if torch.is_grad_enabled() and global_index and (
            getattr(query, "requires_grad", False) or getattr(ref, "requires_grad", False)):
        return _BallQueryRaggedFn.apply(query, q_ptr, ref, r_ptr, radius, K, grid)
    return _ball_query_ragged(query, q_ptr, ref, r_ptr, radius, K, global_index, grid)


def ball_query_ragged_uses_grid(q_cnt, r_cnt, K: int) -> bool:
    """True when pointops_ball_query_ragged takes the grid pass for these
    counts (given the workspace pointops_ball_query_ragged_workspace_bytes
    asks for)."""
    lib = _load()
    q_cnt, r_cnt = _host_i64(q_cnt, "q_cnt"), _host_i64(r_cnt, "r_cnt")
    B = len(q_cnt)
    return int(lib.pointops_ball_query_ragged_workspace_bytes(_vp(q_cnt), _vp(r_cnt), B,
                                                              int(K))) > \
        int(lib.pointops_ragged_workspace_bytes(B))


def _ball_query_ragged(query, q_ptr, ref, r_ptr, radius, K, global_index, grid=True):
    q_off, q_cnt = _ptr_segments(q_ptr, "q_ptr")
    r_off, r_cnt = _ptr_segments(r_ptr, "r_ptr")
    lib = _load()
    return _search_ragged(lib.pointops_ball_query_ragged, query, q_off, q_cnt, ref, r_off,
                          r_cnt, int(K), (ctypes.c_float(float(radius)), int(K)), global_index,
                          0.0, ws_fn=lib.pointops_ball_query_ragged_workspace_bytes if grid
                          else None)


class _BallQueryRaggedFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, query, q_ptr, ref, r_ptr, radius, K, grid):
        d2, idx = _ball_query_ragged(query, q_ptr, ref, r_ptr, radius, K, True, grid)
        ctx.save_for_backward(query, ref, idx)
        ctx.mark_non_differentiable(idx)
        return d2, idx

    @staticmethod
    def backward(ctx, grad_d2, grad_idx):
        query, ref, idx = ctx.saved_tensors
        if grad_d2 is None:
            return (None,) * 7
        # global indices: the flat batch is one cloud for the gradient formulas
        gq, gx = ball_query_backward(query[None], ref[None], idx[None], grad_d2[None],
                                     ctx.needs_input_grad[0], ctx.needs_input_grad[2])
        return (gq[0] if gq is not None else None, None, gx[0] if gx is not None else None,
                None, None, None, None)


def fps_ragged(xyz: torch.Tensor, ptr, counts, start=None, global_index: bool = True,
               return_xyz: bool = False, check: bool = True):
    """Farthest point sampling of each cloud of a flat batch (rows ptr[b] ..
    ptr[b+1]), counts[b] samples each, from local index start[b] (default 0)
    -> int64 (sum of counts,), cloud after cloud; indices are rows of ``xyz``
    (or local). With ``return_xyz`` also the sampled coordinates. ``check`` as
    for ``furthest_point_sample``."""
    lib = _load()
    xyz = _flat_points(xyz, "xyz")
    x_off, x_cnt = _ptr_segments(ptr, "ptr")
    counts = _host_i64(counts, "counts")
    B = len(x_off)
    if len(counts) != B:
        raise PointopsError(1, "counts must have one entry per cloud")
    o_off = np.ascontiguousarray(np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64))
    total = int(counts.sum()) if B else 0
    st = None if start is None else _host_i64(start, "start")
    if st is not None and len(st) != B:
        raise PointopsError(1, "start must have one entry per cloud")
    with torch.cuda.device(xyz.device):
        out = torch.empty(total, dtype=torch.int64, device=xyz.device)
        oxyz = torch.empty((total, 3), dtype=torch.float32, device=xyz.device) if return_xyz else None
        need = int(lib.pointops_fps_ragged_workspace_bytes(_vp(x_cnt), _vp(counts), B))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=xyz.device)
        rc = lib.pointops_fps_ragged(xyz.data_ptr(), xyz.shape[0], _vp(x_off), _vp(x_cnt),
                                     _vp(st), B, out.data_ptr(),
                                     oxyz.data_ptr() if oxyz is not None else None, total,
                                     _vp(o_off), _vp(counts), int(bool(global_index)),
                                     ws.data_ptr(), ws.numel(), _stream(xyz.device))
        _check(rc)
        if check and need > 0 and total > 0:
            fps_status(ws)
    return (out, oxyz) if return_xyz else out


def _lengths(lengths, B, n_max, name):
    if lengths is None:
        return np.full(B, n_max, dtype=np.int64)
    a = _host_i64(lengths, name)
    if len(a) != B:
        raise PointopsError(1, f"{name} must have B entries")
    return a


def knn_padded(query: torch.Tensor, ref: torch.Tensor, k: int, lengths1=None, lengths2=None):
    """kNN of padded clouds (B, n_max, 3) with per-cloud lengths (the
    PyTorch3D form) -> (dist, idx), (B, Q_max, k), local indices; rows past a
    cloud's length and slots past its reference count hold (+inf, -1)."""
    query = _points(query, "query")
    ref = _points(ref, "ref")
    B, Qm, _ = query.shape
    Pm = ref.shape[1]
    l1, l2 = _lengths(lengths1, B, Qm, "lengths1"), _lengths(lengths2, B, Pm, "lengths2")
    d, i = _search_ragged(_load().pointops_knn_ragged, query.view(-1, 3),
                          np.arange(B, dtype=np.int64) * Qm, l1, ref.view(-1, 3),
                          np.arange(B, dtype=np.int64) * Pm, l2, int(k), (int(k),), False,
                          float("inf"), ws_fn=_load().pointops_knn_ragged_workspace_bytes)
    return d.view(B, Qm, k), i.view(B, Qm, k)


def ball_query_padded(query: torch.Tensor, ref: torch.Tensor, radius: float, K: int,
                      lengths1=None, lengths2=None):
    """First-K Ball Query of padded clouds with per-cloud lengths -> (dist2,
    idx), (B, Q_max, K), local indices; rows past a cloud's length hold
    (0, -1)."""
    query = _points(query, "query")
    ref = _points(ref, "ref")
    B, Qm, _ = query.shape
    Pm = ref.shape[1]
    l1, l2 = _lengths(lengths1, B, Qm, "lengths1"), _lengths(lengths2, B, Pm, "lengths2")
    d, i = _search_ragged(_load().pointops_ball_query_ragged, query.view(-1, 3),
                          np.arange(B, dtype=np.int64) * Qm, l1, ref.view(-1, 3),
                          np.arange(B, dtype=np.int64) * Pm, l2, int(K),
                          (ctypes.c_float(float(radius)), int(K)), False, 0.0,
                          ws_fn=_load().pointops_ball_query_ragged_workspace_bytes)
    return d.view(B, Qm, K), i.view(B, Qm, K)


# ------------------------------------------------------------------ three_nn and Chamfer

def three_nn(unknown: torch.Tensor, known: torch.Tensor):
    """The three nearest known points of every unknown point -> (Euclidean
    distance float32, int64 index), (B, n, 3); kNN with k = 3."""
    lib = _load()
    unknown = _points(unknown, "unknown")
    known = _points(known, "known")
    if unknown.device != known.device or unknown.shape[0] != known.shape[0]:
        raise PointopsError(1, "unknown and known must share the device and the batch size")
    B, n, _ = unknown.shape
    m = known.shape[1]
    with torch.cuda.device(unknown.device):
        dist = torch.empty((B, n, 3), dtype=torch.float32, device=unknown.device)
        idx = torch.empty((B, n, 3), dtype=torch.int64, device=unknown.device)
        nbytes = int(lib.pointops_three_nn_workspace_bytes(B, n, m))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=unknown.device) if nbytes else None
        _check(lib.pointops_three_nn(unknown.data_ptr(), known.data_ptr(), B, n, m,
                                     dist.data_ptr(), idx.data_ptr(),
                                     ws.data_ptr() if ws is not None else None, nbytes,
                                     _stream(unknown.device)))
    return dist, idx


_REDUCE = {None: 0, "none": 0, "mean": 1, "sum": 2}


def _chamfer_args(x, y, x_lengths, y_lengths, point_reduction, batch_reduction):
    x = _points(x, "x")
    y = _points(y, "y")
    if x.device != y.device or x.shape[0] != y.shape[0]:
        raise PointopsError(1, "x and y must share the device and the batch size")
    if point_reduction not in ("mean", "sum"):
        raise PointopsError(1, "point_reduction must be 'mean' or 'sum'")
    if batch_reduction not in _REDUCE:
        raise PointopsError(1, "batch_reduction must be 'mean', 'sum' or None")
    B = x.shape[0]
    lx = None if x_lengths is None else _host_i64(x_lengths, "x_lengths")
    ly = None if y_lengths is None else _host_i64(y_lengths, "y_lengths")
    for l, name in ((lx, "x_lengths"), (ly, "y_lengths")):
        if l is not None and len(l) != B:
            raise PointopsError(1, f"{name} must have B entries")
    return x, y, lx, ly, _REDUCE[point_reduction], _REDUCE[batch_reduction]


def chamfer_nearest(x, y, x_lengths=None, y_lengths=None, point_reduction="mean",
                    batch_reduction="mean", single_directional=False):
    """Forward Chamfer call -> (loss, dist_xy, idx_xy, dist_yx, idx_yx): loss
    (B,) for batch_reduction None else (1,); per point of x (of y) the squared
    distance to and local index of its nearest point of the other cloud."""
    lib = _load()
    x, y, lx, ly, pr, br = _chamfer_args(x, y, x_lengths, y_lengths, point_reduction,
                                         batch_reduction)
    B, N, M = x.shape[0], x.shape[1], y.shape[1]
    dev = x.device
    with torch.cuda.device(dev):
        loss = torch.empty((B,) if br == 0 else (1,), dtype=torch.float32, device=dev)
        d_xy = torch.empty((B, N), dtype=torch.float32, device=dev)
        i_xy = torch.empty((B, N), dtype=torch.int64, device=dev)
        d_yx = torch.empty((B, M), dtype=torch.float32, device=dev) if not single_directional else None
        i_yx = torch.empty((B, M), dtype=torch.int64, device=dev) if not single_directional else None
        ws = torch.empty(int(lib.pointops_chamfer_workspace_bytes(B, N, M)), dtype=torch.uint8,
                         device=dev)
        _check(lib.pointops_chamfer(x.data_ptr(), y.data_ptr(), B, N, M, _vp(lx), _vp(ly), pr,
                                    br, int(bool(single_directional)), loss.data_ptr(),
                                    d_xy.data_ptr(), i_xy.data_ptr(),
                                    d_yx.data_ptr() if d_yx is not None else None,
                                    i_yx.data_ptr() if i_yx is not None else None,
                                    ws.data_ptr(), ws.numel(), _stream(dev)))
    return loss, d_xy, i_xy, d_yx, i_yx


def chamfer_backward(x, y, idx_xy, idx_yx, grad_loss, x_lengths=None, y_lengths=None,
                     point_reduction="mean", batch_reduction="mean", single_directional=False,
                     need_x=True, need_y=True):
    """Gradients of the Chamfer loss for fixed nearest points -> (grad_x or
    None, grad_y or None)."""
    lib = _load()
    x, y, lx, ly, pr, br = _chamfer_args(x, y, x_lengths, y_lengths, point_reduction,
                                         batch_reduction)
    B, N, M = x.shape[0], x.shape[1], y.shape[1]
    dev = x.device
    grad_loss = grad_loss.detach().to(device=dev, dtype=torch.float32).reshape(-1).contiguous()
    if grad_loss.numel() != (B if br == 0 else 1):
        raise PointopsError(1, "grad_loss has the wrong number of elements")
    with torch.cuda.device(dev):
        gx = torch.empty_like(x) if need_x else None
        gy = torch.empty_like(y) if need_y else None
        ws = torch.empty(16 * B + 256, dtype=torch.uint8, device=dev)
        _check(lib.pointops_chamfer_backward(
            x.data_ptr(), y.data_ptr(), B, N, M, _vp(lx), _vp(ly), pr, br,
            int(bool(single_directional)), idx_xy.contiguous().data_ptr(),
            idx_yx.contiguous().data_ptr() if idx_yx is not None else None,
            grad_loss.data_ptr(), gx.data_ptr() if gx is not None else None,
            gy.data_ptr() if gy is not None else None, ws.data_ptr(), ws.numel(), _stream(dev)))
    return gx, gy


class _ChamferFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, y, x_lengths, y_lengths, point_reduction, batch_reduction, single):
        loss, _, i_xy, _, i_yx = chamfer_nearest(x, y, x_lengths, y_lengths, point_reduction,
                                                 batch_reduction, single)
        ctx.save_for_backward(x, y, i_xy, i_yx if i_yx is not None else i_xy)
        ctx.args = (x_lengths, y_lengths, point_reduction, batch_reduction, single)
        return loss if batch_reduction is None else loss[0]

    @staticmethod
    def backward(ctx, grad):
        x, y, i_xy, i_yx = ctx.saved_tensors
        xl, yl, pr, br, single = ctx.args
        gx, gy = chamfer_backward(x, y, i_xy, None if single else i_yx, grad, xl, yl, pr, br,
                                  single, ctx.needs_input_grad[0], ctx.needs_input_grad[1])
        return gx, gy, None, None, None, None, None


def chamfer_distance(x: torch.Tensor, y: torch.Tensor, x_lengths=None, y_lengths=None,
                     point_reduction: str = "mean", batch_reduction="mean",
                     single_directional: bool = False):
    """Squared-L2 Chamfer distance of (B, N, 3) and (B, M, 3) clouds, with
    optional per-cloud lengths -> (loss, None): a scalar, or (B,) when
    batch_reduction is None. Differentiable with respect to both clouds."""
    return _ChamferFn.apply(x, y, x_lengths, y_lengths, point_reduction, batch_reduction,
                            single_directional), None
