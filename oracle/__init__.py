"""Python access to the pointops oracle (plain single-threaded C, float32).

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the GPU library never does, and this
package imports nothing from it.

The C source ``pointops_oracle.c`` states which passage of the pages each
function follows. This module only builds that source with gcc, marshals numpy
arrays into it and, for large inputs, fans contiguous query-row ranges out over
host threads (ctypes releases the GIL during the call), each thread running the
unchanged single-threaded routine, so the result does not depend on the thread
count. Ragged batches are composed here from those routines, one cloud at a
time (see the section at the end).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pointops_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
LIB_PATH = os.path.join(_BUILD_DIR, "libpointops_oracle.so")

# Flags: float32 per-operation rounding, no contraction, no fast-math, no FMA.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]

_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/_build``; return the library path."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    os.makedirs(_BUILD_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        f32p = ctypes.POINTER(ctypes.c_float)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.pco_s32.argtypes = [f32p, f32p]
        lib.pco_s32.restype = ctypes.c_float
        lib.pco_ball_query_r2.argtypes = [ctypes.c_float]
        lib.pco_ball_query_r2.restype = ctypes.c_float
        lib.pco_fps.argtypes = [f32p, i64, i64, i64, i64, i64p]
        lib.pco_fps.restype = ctypes.c_int
        lib.pco_knn_rows.argtypes = [f32p, f32p, i64, i64, i64, i64, f32p, i64p, i64, i64]
        lib.pco_knn_rows.restype = ctypes.c_int
        lib.pco_ball_query_rows.argtypes = [f32p, f32p, i64, i64, i64, ctypes.c_float, i64,
                                            f32p, i64p, i64, i64]
        lib.pco_ball_query_rows.restype = ctypes.c_int
        f64p = ctypes.POINTER(ctypes.c_double)
        lib.pco_ball_query_backward.argtypes = [f32p, f32p, i64p, f32p, i64, i64, i64, i64,
                                                f64p, f64p, f64p, f64p]
        lib.pco_ball_query_backward.restype = ctypes.c_int
        lib.pco_nearest_rows.argtypes = [f32p, f32p, i64, i64, i64, i64p, f32p, i64p, i64, i64]
        lib.pco_nearest_rows.restype = ctypes.c_int
        _lib = lib
        return lib


class OracleError(ValueError):
    pass


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _i64(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"oracle {what} rejected its arguments (status {rc})")


def s32(a, b) -> np.float32:
    """Squared distance of two 3-vectors in the oracle's float32 order."""
    lib = _load()
    a, pa = _f32(a)
    b, pb = _f32(b)
    assert a.shape == (3,) and b.shape == (3,)
    return np.float32(lib.pco_s32(pa, pb))


def ball_query_r2(radius) -> np.float32:
    """R2 = fl32(r32 * r32) for r32 = fl32(radius)."""
    return np.float32(_load().pco_ball_query_r2(float(np.float32(radius))))


def fps(xyz, npoint: int, start_idx: int = 0, threads: int = 1) -> np.ndarray:
    """Farthest point sampling of (B, N, 3) float32 clouds -> (B, npoint) int64.

    With threads > 1 the independent clouds are split over host threads."""
    lib = _load()
    xyz, _ = _f32(xyz)
    B, N, three = xyz.shape
    assert three == 3
    out = np.zeros((B, npoint), dtype=np.int64)
    if B == 0 or npoint == 0:
        return out

    def run(b0, b1):
        sub = np.ascontiguousarray(xyz[b0:b1])
        o = np.zeros((b1 - b0, npoint), dtype=np.int64)
        rc = lib.pco_fps(sub.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), b1 - b0, N,
                         npoint, start_idx, _i64(o))
        _check(rc, "fps")
        out[b0:b1] = o

    _fan_out(run, B, threads)
    return out


def _fan_out(run, n, threads):
    threads = max(1, min(int(threads), n))
    if threads == 1:
        run(0, n)
        return
    bounds = np.linspace(0, n, threads + 1).astype(np.int64)
    with ThreadPoolExecutor(threads) as ex:
        futs = [ex.submit(run, int(bounds[i]), int(bounds[i + 1])) for i in range(threads)
                if bounds[i + 1] > bounds[i]]
        for f in futs:
            f.result()


def knn(query, ref, k: int, rows=None, threads: int = 1):
    """kNN of (B, Q, 3) queries in (B, P, 3) references -> (dist (B,Q,k) f32, idx int64).

    ``rows``: optional (lo, hi) range of flattened query rows (b*Q + i) to compute;
    other rows are left as NaN / -2 so an unwritten slot is visible."""
    lib = _load()
    query, pq = _f32(query)
    ref, pr = _f32(ref)
    B, Q, _ = query.shape
    P = ref.shape[1]
    assert ref.shape[0] == B and ref.shape[2] == 3 and query.shape[2] == 3
    dist = np.full((B, Q, k), np.nan, dtype=np.float32)
    idx = np.full((B, Q, k), -2, dtype=np.int64)
    lo, hi = (0, B * Q) if rows is None else rows
    pd = dist.ctypes.data_as(ctypes.POINTER(ctypes.c_float))

    def run(a, b):
        _check(lib.pco_knn_rows(pq, pr, B, Q, P, k, pd, _i64(idx), lo + a, lo + b), "knn")

    if hi > lo:
        _fan_out(run, hi - lo, threads)
    return dist, idx


def ball_query(query, ref, radius, K: int, rows=None, threads: int = 1):
    """First-K Ball Query -> (dist2 (B,Q,K) f32, idx (B,Q,K) int64), radius rounded to f32."""
    lib = _load()
    query, pq = _f32(query)
    ref, pr = _f32(ref)
    B, Q, _ = query.shape
    P = ref.shape[1]
    assert ref.shape[0] == B and ref.shape[2] == 3 and query.shape[2] == 3
    dist2 = np.full((B, Q, K), np.nan, dtype=np.float32)
    idx = np.full((B, Q, K), -2, dtype=np.int64)
    lo, hi = (0, B * Q) if rows is None else rows
    pd = dist2.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    r32 = float(np.float32(radius))

    def run(a, b):
        _check(lib.pco_ball_query_rows(pq, pr, B, Q, P, r32, K, pd, _i64(idx), lo + a, lo + b),
               "ball_query")

    if hi > lo:
        _fan_out(run, hi - lo, threads)
    return dist2, idx


def ball_query_backward(query, ref, idx, grad):
    """Gradients of L = sum G * S of a Ball Query output, in float64.

    Returns (grad_query (B,Q,3), grad_ref (B,P,3), abs_query, abs_ref) where
    abs_* is the sum of absolute values of the terms of each output."""
    lib = _load()
    query, pq = _f32(query)
    ref, pr = _f32(ref)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    grad, pg = _f32(grad)
    B, Q, _ = query.shape
    P = ref.shape[1]
    K = idx.shape[-1]
    assert idx.shape == (B, Q, K) and grad.shape == (B, Q, K)
    gq = np.zeros((B, Q, 3)); gx = np.zeros((B, P, 3))
    aq = np.zeros((B, Q, 3)); ax = np.zeros((B, P, 3))
    f64 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    _check(lib.pco_ball_query_backward(pq, pr, _i64(idx), pg, B, Q, P, K, f64(gq), f64(gx),
                                       f64(aq), f64(ax)), "ball_query_backward")
    return gq, gx, aq, ax


# ------------------------------------------------------------------ ragged batches
#
# Project page, section "Flat torch_cluster subset": the clouds of a batch sit
# back to back in one flat array and are searched independently; returned
# indices point into the flat input; a cloud with fewer than k references gets
# only the neighbours it has. A cloud is a segment (off, cnt) of a flat buffer.
# Each cloud is handed, alone, to the dense routines above; the only additions
# are the index offset and the padding of missing kNN neighbours, which this
# library's ragged output marks with (+inf, -1).

def fps_ragged(xyz, x_off, x_cnt, out_off, out_cnt, out_rows, start=None, global_index=True,
               clouds=None):
    """FPS of every cloud -> (out_rows,) int64; rows no cloud writes hold -2."""
    xyz = np.ascontiguousarray(xyz, dtype=np.float32)
    out = np.full(out_rows, -2, dtype=np.int64)
    for b in (range(len(x_cnt)) if clouds is None else clouds):
        m = int(out_cnt[b])
        if m == 0:
            continue
        o, n = int(x_off[b]), int(x_cnt[b])
        s = 0 if start is None else int(start[b])
        idx = fps(xyz[None, o:o + n], m, s)[0]
        out[int(out_off[b]):int(out_off[b]) + m] = idx + (o if global_index else 0)
    return out


def knn_ragged(query, q_off, q_cnt, ref, r_off, r_cnt, k, global_index=True, clouds=None,
               threads=1):
    """kNN of every cloud -> (dist, idx), (q_rows, k); rows no cloud writes
    hold NaN / -2; missing neighbours (cloud smaller than k) are (+inf, -1)."""
    query = np.ascontiguousarray(query, dtype=np.float32)
    ref = np.ascontiguousarray(ref, dtype=np.float32)
    dist = np.full((len(query), k), np.nan, dtype=np.float32)
    idx = np.full((len(query), k), -2, dtype=np.int64)
    for b in (range(len(q_cnt)) if clouds is None else clouds):
        qo, qn, ro, rn = int(q_off[b]), int(q_cnt[b]), int(r_off[b]), int(r_cnt[b])
        if qn == 0:
            continue
        kk = min(k, rn)
        dist[qo:qo + qn] = np.inf
        idx[qo:qo + qn] = -1
        if kk == 0:
            continue
        d, i = knn(query[None, qo:qo + qn], ref[None, ro:ro + rn], kk, threads=threads)
        dist[qo:qo + qn, :kk] = d[0]
        idx[qo:qo + qn, :kk] = i[0] + (ro if global_index else 0)
    return dist, idx


def ball_query_ragged(query, q_off, q_cnt, ref, r_off, r_cnt, radius, K, global_index=True,
                      clouds=None, threads=1):
    """First-K Ball Query of every cloud -> (dist2, idx), (q_rows, K); rows no
    cloud writes hold NaN / -2."""
    query = np.ascontiguousarray(query, dtype=np.float32)
    ref = np.ascontiguousarray(ref, dtype=np.float32)
    dist2 = np.full((len(query), K), np.nan, dtype=np.float32)
    idx = np.full((len(query), K), -2, dtype=np.int64)
    for b in (range(len(q_cnt)) if clouds is None else clouds):
        qo, qn, ro, rn = int(q_off[b]), int(q_cnt[b]), int(r_off[b]), int(r_cnt[b])
        if qn == 0:
            continue
        d, i = ball_query(query[None, qo:qo + qn], ref[None, ro:ro + rn], radius, K,
                          threads=threads)
        dist2[qo:qo + qn] = d[0]
        idx[qo:qo + qn] = np.where(i[0] >= 0, i[0] + (ro if global_index else 0), -1)
    return dist2, idx



# ------------------------------------------------------------------ three_nn and Chamfer
#
# Project page: the 0.5.0 operators (section "Minimal example" calls them;
# roadmap "Phase 2" describes three_nn, "Phase 4" the Chamfer distance).

def three_nn(unknown, known, threads=1):
    """The three nearest known points of every unknown point: Euclidean
    distances and indices (roadmap, "Phase 2"), i.e. kNN with k = 3."""
    return knn(unknown, known, 3, threads=threads)


def nearest(query, ref, p_len=None, rows=None, threads=1):
    """Nearest reference (squared distance, index) of every query row; cloud b
    uses its first p_len[b] references. -> (s (B, Q) float32, idx (B, Q) int64)."""
    lib = _load()
    query, pq = _f32(query)
    ref, pr = _f32(ref)
    B, Q, _ = query.shape
    P = ref.shape[1]
    s = np.full((B, Q), np.nan, dtype=np.float32)
    idx = np.full((B, Q), -2, dtype=np.int64)
    pl = None if p_len is None else np.ascontiguousarray(p_len, dtype=np.int64)
    lo, hi = (0, B * Q) if rows is None else rows
    ps = s.ctypes.data_as(ctypes.POINTER(ctypes.c_float))

    def run(a, b):
        _check(lib.pco_nearest_rows(pq, pr, B, Q, P, None if pl is None else _i64(pl), ps,
                                    _i64(idx), lo + a, lo + b), "nearest")

    if hi > lo:
        _fan_out(run, hi - lo, threads)
    return s, idx


def _chamfer_weights(B, x_len, y_len, point_reduction, batch_reduction):
    """Per-cloud factors of the two directions' sums: 1 / length for a point
    mean (a length of 0 counts as 1), times 1 / B for a batch mean."""
    wx = np.ones(B) if point_reduction == "sum" else 1.0 / np.maximum(x_len, 1)
    wy = np.ones(B) if point_reduction == "sum" else 1.0 / np.maximum(y_len, 1)
    if batch_reduction == "mean":
        wx, wy = wx / B, wy / B
    return wx, wy


def chamfer(x, y, x_len=None, y_len=None, point_reduction="mean", batch_reduction="mean",
            single_directional=False, threads=1):
    """Squared-L2 Chamfer distance of clouds x (B, N, 3) and y (B, M, 3), the
    first x_len[b] / y_len[b] points of each cloud taking part (roadmap,
    "Phase 4"): a(i) = the nearest point of y to x_i, b(j) = the nearest of x
    to y_j; per cloud the sum (or mean) over i of |x_i - y_a(i)|^2 plus, unless
    single-directional, the same over j of |y_j - x_b(j)|^2; then the sum or
    mean over the batch, or per cloud (batch_reduction None). float64 sums of
    the float32 squared distances.
    -> (loss: float or (B,) float64, s_xy, i_xy, s_yx, i_yx)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.ascontiguousarray(y, dtype=np.float32)
    B, N, M = x.shape[0], x.shape[1], y.shape[1]
    xl = np.full(B, N) if x_len is None else np.asarray(x_len, dtype=np.int64)
    yl = np.full(B, M) if y_len is None else np.asarray(y_len, dtype=np.int64)
    s_xy, i_xy = nearest(x, y, yl, threads=threads)
    s_yx, i_yx = nearest(y, x, xl, threads=threads)
    mx = np.arange(N)[None, :] < xl[:, None]
    my = np.arange(M)[None, :] < yl[:, None]
    # points past a cloud's length take no part: reported as (0, -1)
    s_xy[~mx], i_xy[~mx] = 0.0, -1
    s_yx[~my], i_yx[~my] = 0.0, -1
    wx, wy = _chamfer_weights(B, xl, yl, point_reduction, batch_reduction)
    per = wx * np.where(mx, s_xy.astype(np.float64), 0.0).sum(axis=1)
    if not single_directional:
        per = per + wy * np.where(my, s_yx.astype(np.float64), 0.0).sum(axis=1)
    loss = per if batch_reduction is None else float(per.sum())
    return loss, s_xy, i_xy, s_yx, i_yx


def chamfer_backward(x, y, i_xy, i_yx, grad_loss, x_len=None, y_len=None,
                     point_reduction="mean", batch_reduction="mean", single_directional=False):
    """Gradients of the Chamfer loss with the nearest points held fixed
    (roadmap, "Phase 4": both directions contribute to both clouds), float64.
    grad_loss: a float, or (B,) for batch_reduction None.
    -> (grad_x, grad_y, abs_x, abs_y); abs_* sums the absolute terms."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    B, N, M = x.shape[0], x.shape[1], y.shape[1]
    xl = np.full(B, N) if x_len is None else np.asarray(x_len, dtype=np.int64)
    yl = np.full(B, M) if y_len is None else np.asarray(y_len, dtype=np.int64)
    g = np.broadcast_to(np.asarray(grad_loss, dtype=np.float64), (B,))
    wx, wy = _chamfer_weights(B, xl, yl, point_reduction, batch_reduction)
    gx, gy = np.zeros_like(x), np.zeros_like(y)
    ax, ay = np.zeros_like(x), np.zeros_like(y)
    dirs = [(x, y, i_xy, xl, g * wx, gx, gy, ax, ay)]
    if not single_directional:
        dirs.append((y, x, i_yx, yl, g * wy, gy, gx, ay, ax))
    for a, o, idx, la, w, ga, go, aa, ao in dirs:
        for b in range(B):
            for i in range(int(la[b])):
                j = int(idx[b, i])
                if j < 0:
                    continue
                t = 2.0 * w[b] * (a[b, i] - o[b, j])
                ga[b, i] += t
                go[b, j] -= t
                aa[b, i] += np.abs(t)
                ao[b, j] += np.abs(t)
    return gx, gy, ax, ay
