"""Non-finite coordinates: outside the contract (the project page states the
FPS rule for finite coordinates; its differential checker ran NaN and Inf
inputs without stating expected values), so the results are "parity
unpinned". What is required is that every call terminates and writes only
inside its outputs, and that indices stay in range.

Every output here sits inside a larger device buffer whose guard regions on
both sides are filled with a sentinel bit pattern beforehand; the test checks
the guards bit for bit afterwards. Calls go straight through the C ABI.
Each search the library can take is run: FPS (step kernel, certified
batches), kNN (grid search one and two queries per wave, grid search one
query per lane for k > 32, full scans per wave and per lane), Ball Query
(culled scan, culled scan with the grid pass, full scan)."""
import ctypes

import numpy as np
import pytest
import torch

from point_cloud_neighbor_amd import workloads as W
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

GUARD = 4096          # elements of guard on each side of an output
F_SENT = 0x7FA5A5A5   # a NaN payload no kernel writes
I_SENT = -0x5A5A5A5A5A


class Guarded:
    """An output view of `shape` inside a buffer with sentinel guards."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape))
        self.n = n
        if dtype == torch.float32:
            self.buf = torch.full((n + 2 * GUARD,), F_SENT, dtype=torch.int32, device="cuda")
            self.view = self.buf[GUARD:GUARD + n].view(torch.float32).view(shape)
            self.sent = F_SENT
        else:
            self.buf = torch.full((n + 2 * GUARD,), I_SENT, dtype=torch.int64, device="cuda")
            self.view = self.buf[GUARD:GUARD + n].view(shape)
            self.sent = I_SENT

    def ptr(self):
        return self.view.data_ptr()

    def check(self, what):
        b = self.buf.cpu().numpy()
        assert (b[:GUARD] == self.sent).all(), f"{what}: write before the output"
        assert (b[GUARD + self.n:] == self.sent).all(), f"{what}: write after the output"
        return self.view.cpu().numpy()


def poisoned(seed, N, frac=0.02):
    """Uniform points with NaN, +inf and -inf coordinates in about frac of them."""
    x = W.uniform_cube(seed, 1, N)
    rng = np.random.default_rng(seed + 1)
    bad = rng.choice(N, size=max(3, int(N * frac)), replace=False)
    vals = np.array([np.nan, np.inf, -np.inf], dtype=np.float32)
    x[0, bad, rng.integers(0, 3, size=len(bad))] = vals[np.arange(len(bad)) % 3]
    x[0, bad[:3]] = vals[:, None]  # three points with all coordinates non-finite
    return x


def lib_and_stream(gpu):
    return gpu._load(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("N,M,mode", [(1024, 200, None), (20000, 300, None),
                                      (20000, 300, "step")])
def test_fps_nonfinite(gpu, N, M, mode, monkeypatch):
    if mode:
        monkeypatch.setenv("POINTOPS_FPS_MODE", mode)
        monkeypatch.setenv("POINTOPS_FPS_WG_PER_CLOUD", "8")
    lib, s = lib_and_stream(gpu)
    x = dev(poisoned(3, N))
    for start in (0, int(np.nonzero(~np.isfinite(host_np(x)[0]).all(axis=1))[0][0])):
        out = Guarded((1, M), torch.int64)
        oxyz = Guarded((1, M, 3), torch.float32)
        ws = torch.empty(max(1, lib.pointops_fps_workspace_bytes(1, N, M)), dtype=torch.uint8,
                         device="cuda")
        assert lib.pointops_fps(x.data_ptr(), 1, N, M, start, out.ptr(), oxyz.ptr(),
                                ws.data_ptr(), ws.numel(), s) == 0
        torch.cuda.synchronize()
        gpu.fps_status(ws)
        o = out.check(f"fps N={N} start={start}")
        oxyz.check(f"fps xyz N={N} start={start}")
        assert o[0, 0] == start
        assert ((o >= 0) & (o < N)).all()


def host_np(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("seed", [3, 11])
def test_fps_nonfinite_grouped(gpu, seed, monkeypatch):
    """Grouped slices (waves culling folds by their boxes) against the same
    call without grouping, on clouds with NaN and infinite coordinates. The
    box bound stays a lower bound there (a wave holding a NaN point always
    folds; infinite gaps only skip folds whose distances are infinite or
    NaN), so the two must agree index for index and bit for bit, guards
    intact."""
    lib, s = lib_and_stream(gpu)
    N, M = 20000, 600
    x = dev(poisoned(seed, N, frac=0.01))
    monkeypatch.setenv("POINTOPS_FPS_MODE", "batch")
    monkeypatch.setenv("POINTOPS_FPS_WG_PER_CLOUD", "4")  # slices of 5000: 6 points per thread
    got = {}
    for group in ("1", "0"):
        monkeypatch.setenv("POINTOPS_FPS_GROUP", group)
        out = Guarded((1, M), torch.int64)
        oxyz = Guarded((1, M, 3), torch.float32)
        nb = lib.pointops_fps_workspace_bytes(1, N, M)
        ws = torch.empty(max(1, nb), dtype=torch.uint8, device="cuda")
        assert lib.pointops_fps(x.data_ptr(), 1, N, M, 0, out.ptr(), oxyz.ptr(),
                                ws.data_ptr(), ws.numel(), s) == 0
        torch.cuda.synchronize()
        gpu.fps_status(ws)
        got[group] = (out.check(f"fps grouped={group}"),
                      oxyz.check(f"fps xyz grouped={group}").view(np.uint32), nb)
    assert got["1"][2] >= got["0"][2] + N * 16  # the grouped plan was taken
    assert np.array_equal(got["1"][0], got["0"][0])
    assert np.array_equal(got["1"][1], got["0"][1])
    assert ((got["1"][0] >= 0) & (got["1"][0] < N)).all()


@pytest.mark.parametrize("k,Q,P,grid,env", [
    (16, 3000, 20000, True, {"POINTOPS_KNN_GRID_WAVE": "1"}),
    (16, 12000, 20000, True, {"POINTOPS_KNN_GRID_WAVE": "2"}),
    (40, 3000, 40000, True, {}),
    (16, 3000, 20000, False, {"POINTOPS_KNN_WAVE": "1"}),
    (16, 3000, 20000, False, {"POINTOPS_KNN_WAVE": "0"}),
    (40, 1000, 20000, False, {}),
])
def test_knn_nonfinite(gpu, k, Q, P, grid, env, monkeypatch):
    for key, v in env.items():
        monkeypatch.setenv(key, v)
    lib, s = lib_and_stream(gpu)
    ref = dev(poisoned(5, P))
    q = dev(poisoned(6, Q))
    d = Guarded((1, Q, k), torch.float32)
    i = Guarded((1, Q, k), torch.int64)
    nb = lib.pointops_knn_workspace_bytes(1, Q, P) if grid else 0
    ws = torch.empty(max(1, nb), dtype=torch.uint8, device="cuda")
    assert lib.pointops_knn(q.data_ptr(), ref.data_ptr(), 1, Q, P, k, d.ptr(), i.ptr(),
                            ws.data_ptr() if nb else None, nb, s) == 0
    torch.cuda.synchronize()
    what = f"knn k={k} grid={grid} {env}"
    idx = i.check(what)
    d.check(what)
    assert ((idx >= -1) & (idx < P)).all(), what
    # finite queries still get a full row of distinct references
    fin = np.isfinite(host_np(q)[0]).all(axis=1)
    rows = idx[0][fin]
    assert (rows >= 0).all(), what
    srt = np.sort(rows, axis=1)
    assert (np.diff(srt, axis=1) > 0).all(), what


@pytest.mark.parametrize("Q,P,K,cull,env", [
    (3000, 40000, 32, True, {}),
    (3000, 40000, 32, True, {"POINTOPS_BQ_GRID": "1", "POINTOPS_BQ_BUDGET": "4"}),
    (3000, 40000, 64, True, {}),
    (3000, 20000, 32, False, {}),
])
def test_ball_query_nonfinite(gpu, Q, P, K, cull, env, monkeypatch):
    for key, v in env.items():
        monkeypatch.setenv(key, v)
    lib, s = lib_and_stream(gpu)
    ref = dev(poisoned(7, P))
    q = dev(poisoned(8, Q))
    d = Guarded((1, Q, K), torch.float32)
    i = Guarded((1, Q, K), torch.int64)
    nb = lib.pointops_ball_query_workspace_bytes(1, Q, P) if cull else 0
    ws = torch.empty(max(1, nb), dtype=torch.uint8, device="cuda")
    assert lib.pointops_ball_query(q.data_ptr(), ref.data_ptr(), 1, Q, P, ctypes.c_float(0.1), K,
                                   d.ptr(), i.ptr(), ws.data_ptr() if nb else None, nb, s) == 0
    torch.cuda.synchronize()
    what = f"ball query K={K} cull={cull} {env}"
    idx = i.check(what)
    d2 = d.check(what)
    assert ((idx >= -1) & (idx < P)).all(), what
    valid = idx >= 0
    assert (valid[..., :-1] | ~valid[..., 1:]).all(), what   # hits first, then padding
    # a hit is a pair whose s32 compared below R2: never a NaN distance
    assert np.isfinite(d2[valid]).all() and (d2[valid] < np.float32(0.1) ** 2 * 1.01).all(), what
    # rows of non-finite queries hold no hit (every comparison is false)
    nonfin = ~np.isfinite(host_np(q)[0]).all(axis=1)
    assert (idx[0][nonfin] == -1).all(), what
