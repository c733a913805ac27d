"""Ragged batches on the GPU versus the oracle's ragged composition, element
by element: indices bit-exact, distances bit-exact (and within the stated
tolerance). All calls go through the C ABI (via the thin Python binding)."""
import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from point_cloud_neighbor_amd import workloads as W
from tests.gpu_util import assert_dist_close, assert_idx_equal, dev, host

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def out_ptr(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def check_fps(gpu, oracle_mod, xyz, ptr, counts, start=None, global_index=True, what=""):
    got, gx = gpu.fps_ragged(dev(xyz), ptr, counts, start=start, global_index=global_index,
                             return_xyz=True)
    op = out_ptr(counts)
    B = len(counts)
    clouds = [b for b in range(B) if counts[b] > 0]
    want = np.full(int(op[-1]), -2, dtype=np.int64)

    def one(b):  # clouds are independent: run them side by side
        w = oracle_mod.fps_ragged(xyz, ptr[:-1], np.diff(ptr), op[:-1], counts, int(op[-1]),
                                  start=start, global_index=global_index, clouds=[b])
        want[op[b]:op[b + 1]] = w[op[b]:op[b + 1]]

    with ThreadPoolExecutor(8) as ex:
        list(ex.map(one, clouds))
    assert_idx_equal(host(got), want, f"fps {what}")
    rows = want + (0 if global_index else np.repeat(ptr[:-1], counts))
    assert np.array_equal(host(gx).view(np.uint32), xyz[rows].view(np.uint32))
    return want


def check_search(gpu, oracle_mod, q, qptr, x, xptr, k, r, K, global_index=True, what=""):
    d, i = gpu.knn_ragged(dev(q), qptr, dev(x), xptr, k, global_index=global_index)
    wd, wi = oracle_mod.knn_ragged(q, qptr[:-1], np.diff(qptr), x, xptr[:-1], np.diff(xptr), k,
                                   global_index=global_index, threads=8)
    covered = np.repeat(np.diff(qptr) > 0, np.diff(qptr))
    assert_idx_equal(host(i), wi, f"knn idx {what}")
    assert_dist_close(host(d), wd, f"knn dist {what}")
    d2, j = gpu.ball_query_ragged(dev(q), qptr, dev(x), xptr, r, K, global_index=global_index)
    wd2, wj = oracle_mod.ball_query_ragged(q, qptr[:-1], np.diff(qptr), x, xptr[:-1],
                                           np.diff(xptr), r, K, global_index=global_index,
                                           threads=8)
    assert_idx_equal(host(j), wj, f"bq idx {what}")
    assert_dist_close(host(d2), wd2, f"bq dist2 {what}")
    assert covered.all()


def test_flat_example(gpu):
    with open(os.path.join(GOLDEN, "flat_example.json")) as f:
        g = json.load(f)
    x = dev(np.array(g["x"], dtype=np.float32))
    y = dev(np.array(g["y"], dtype=np.float32))
    d = g["derived"]
    c = gpu.fps_ragged(x, g["ptr_x"], d["fps_counts"])
    assert host(c).tolist() == d["fps_idx"]
    kd, ki = gpu.knn_ragged(y, g["ptr_y"], x, g["ptr_x"], d["knn_k"])
    assert host(ki).tolist() == d["knn_idx"]
    assert host(kd).tolist() == [[float(v) for v in row] for row in d["knn_dist"]]
    bd, bi = gpu.ball_query_ragged(y, g["ptr_y"], x, g["ptr_x"], d["bq_radius"], d["bq_K"])
    assert host(bi).tolist() == d["bq_idx"]
    assert host(bd).tolist() == d["bq_dist2"]


MIXES = [
    [1, 5, 0, 64, 65, 300],                 # tiny and empty clouds, one-tile edges
    [1000, 3000, 17, 2048, 2049],           # every cloud fits one workgroup
    [20000, 500, 70000, 3, 9000],           # clouds that span several workgroups
]


@pytest.mark.parametrize("sizes", MIXES)
def test_fps_ragged(gpu, oracle_mod, sizes):
    r = W.ragged_batch(7, sizes)
    counts = np.array([min(n, 257) if n else 0 for n in r.cnt]) + (np.array(r.cnt) == 1) * 2
    starts = np.array([n // 3 for n in r.cnt])
    check_fps(gpu, oracle_mod, r.xyz, r.ptr, counts, start=starts, what=str(sizes))


@pytest.mark.parametrize("mode", ["step", "batch"])
def test_fps_ragged_forced_mode(gpu, oracle_mod, mode, monkeypatch):
    monkeypatch.setenv("POINTOPS_FPS_MODE", mode)
    r = W.ragged_batch(8, [4000, 100, 12000, 1, 2500])
    counts = np.array([300, 100, 400, 3, 0])
    check_fps(gpu, oracle_mod, r.xyz, r.ptr, counts, what=mode)


def test_fps_ragged_ties_and_local_indices(gpu, oracle_mod):
    sizes = [300, 5000, 40]
    xyz = W.integer_cloud(9, 1, int(np.sum(sizes)), 0, 4)[0]
    ptr = out_ptr(sizes)
    check_fps(gpu, oracle_mod, xyz, ptr, np.array([80, 90, 50]), global_index=False,
              what="integer")


@pytest.mark.parametrize("sizes", MIXES)
def test_search_ragged(gpu, oracle_mod, sizes):
    x = W.ragged_batch(10, sizes)
    qsizes = [n // 4 + (b % 3) for b, n in enumerate(sizes)]
    q = W.ragged_batch(11, qsizes)
    for k, r, K in [(1, 0.05, 1), (16, 0.1, 32), (40, 0.3, 70)]:
        check_search(gpu, oracle_mod, q.xyz, q.ptr, x.xyz, x.ptr, k, r, K,
                     what=f"{sizes} k={k} K={K}")


def test_search_ragged_local_indices_and_small_clouds(gpu, oracle_mod):
    sizes = [0, 1, 3, 16, 17, 1000]
    x = W.ragged_batch(12, sizes)
    q = W.ragged_batch(13, [5, 5, 5, 5, 5, 70])
    check_search(gpu, oracle_mod, q.xyz, q.ptr, x.xyz, x.ptr, 16, 0.5, 8, global_index=False,
                 what="small clouds")


def test_padded_lengths(gpu, oracle_mod):
    B, Qm, Pm = 4, 90, 700
    q = W.uniform_cube(14, B, Qm)
    x = W.uniform_cube(15, B, Pm)
    l1, l2 = np.array([90, 0, 33, 7]), np.array([700, 12, 5, 1])
    d, i = gpu.knn_padded(dev(q), dev(x), 8, l1, l2)
    d2, j = gpu.ball_query_padded(dev(q), dev(x), 0.3, 16, l1, l2)
    qo, xo = np.arange(B) * Qm, np.arange(B) * Pm
    wd, wi = oracle_mod.knn_ragged(q.reshape(-1, 3), qo, l1, x.reshape(-1, 3), xo, l2, 8,
                                   global_index=False)
    wd2, wj = oracle_mod.ball_query_ragged(q.reshape(-1, 3), qo, l1, x.reshape(-1, 3), xo, l2,
                                           0.3, 16, global_index=False)
    # rows past a cloud's length: the binding's fill
    unw = wi[:, 0] == -2
    wd[unw], wi[unw] = np.inf, -1
    wd2[unw], wj[unw] = 0.0, -1
    assert_idx_equal(host(i).reshape(-1, 8), wi, "padded knn idx")
    assert_dist_close(host(d).reshape(-1, 8), wd, "padded knn dist")
    assert_idx_equal(host(j).reshape(-1, 16), wj, "padded bq idx")
    assert_dist_close(host(d2).reshape(-1, 16), wd2, "padded bq dist2")


def test_ragged_workload(gpu, oracle_mod):
    """The ragged benchmark workload in the launch configuration the benchmark
    times: FPS of every cloud against the oracle in full, then kNN and Ball
    Query of the samples on 64-row blocks at both ends of every cloud."""
    r = W.ragged_workload()
    want = check_fps(gpu, oracle_mod, r.xyz, r.ptr, r.fps_counts, what="ragged workload")
    centres = r.xyz[want]
    qptr = out_ptr(r.fps_counts)
    d, i = gpu.knn_ragged(dev(centres), qptr, dev(r.xyz), r.ptr, r.knn_k)
    d2, j = gpu.ball_query_ragged(dev(centres), qptr, dev(r.xyz), r.ptr, r.bq_radius, r.bq_k)
    d, i, d2, j = host(d), host(i), host(d2), host(j)
    for b in range(len(r.cnt)):
        for lo in {int(qptr[b]), max(int(qptr[b]), int(qptr[b + 1]) - 64)}:
            hi = min(lo + 64, int(qptr[b + 1]))
            sub_q = (np.array([lo]), np.array([hi - lo]))
            sub_x = (r.ptr[b:b + 1], r.cnt[b:b + 1])
            wd, wi = oracle_mod.knn_ragged(centres, *sub_q, r.xyz, *sub_x, r.knn_k, threads=8)
            assert_idx_equal(i[lo:hi], wi[lo:hi], f"knn cloud {b} rows {lo}:{hi}")
            assert_dist_close(d[lo:hi], wd[lo:hi], f"knn cloud {b} rows {lo}:{hi}")
            wd2, wj = oracle_mod.ball_query_ragged(centres, *sub_q, r.xyz, *sub_x, r.bq_radius,
                                                   r.bq_k, threads=8)
            assert_idx_equal(j[lo:hi], wj[lo:hi], f"bq cloud {b} rows {lo}:{hi}")
            assert_dist_close(d2[lo:hi], wd2[lo:hi], f"bq cloud {b} rows {lo}:{hi}")


def test_ragged_ball_query_autograd(gpu, oracle_mod):
    x = W.ragged_batch(16, [400, 0, 900, 30])
    q = W.ragged_batch(17, [50, 10, 80, 5])
    xt = dev(x.xyz).requires_grad_(True)
    qt = dev(q.xyz).requires_grad_(True)
    d2, idx = gpu.ball_query_ragged(qt, q.ptr, xt, x.ptr, 0.3, 24)
    g = np.random.default_rng(18).standard_normal(tuple(d2.shape)).astype(np.float32)
    (d2 * dev(g)).sum().backward()
    wq, wx, aq, ax = oracle_mod.ball_query_backward(q.xyz[None], x.xyz[None], host(idx)[None],
                                                    g[None])
    i = host(idx)
    nq = (i >= 0).sum(-1)
    nx = np.bincount(i[i >= 0], minlength=len(x.xyz))
    for got, want, a, n in ((host(qt.grad), wq[0], aq[0], nq), (host(xt.grad), wx[0], ax[0], nx)):
        bound = (n[:, None] + 4.0) * 2.0**-23 * a
        assert np.all(np.abs(got.astype(np.float64) - want) <= bound)


def test_ragged_invalid_arguments(gpu):
    x = dev(W.uniform_cube(19, 1, 50)[0])
    with pytest.raises(gpu.PointopsError):
        gpu.knn_ragged(x, [0, 30, 60], x, [0, 25, 50], 4)          # query segment past the end
    with pytest.raises(gpu.PointopsError):
        gpu.knn_ragged(x, [0, 30, 50], x, [0, 25, 50], 65)         # k above the maximum
    with pytest.raises(gpu.PointopsError):
        gpu.fps_ragged(x, [0, 0, 50], [3, 4])                      # samples from an empty cloud
    with pytest.raises(gpu.PointopsError):
        gpu.fps_ragged(x, [0, 20, 50], [3, 4], start=[0, 30])      # start outside its cloud
    from point_cloud_neighbor_amd import ops
    lib = ops._load()
    import ctypes
    off = np.array([0, 10], dtype=np.int64)
    cnt = np.array([20, 20], dtype=np.int64)                       # overlapping query rows
    o = torch.empty((50, 4), device="cuda")
    oi = torch.empty((50, 4), dtype=torch.int64, device="cuda")
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    rc = lib.pointops_knn_ragged(x.data_ptr(), 50, ctypes.c_void_p(off.ctypes.data),
                                 ctypes.c_void_p(cnt.ctypes.data), x.data_ptr(), 50,
                                 ctypes.c_void_p(off.ctypes.data), ctypes.c_void_p(cnt.ctypes.data),
                                 2, 4, 1, o.data_ptr(), oi.data_ptr(), ws.data_ptr(), 4096, None)
    assert rc == 1


def test_fps_ragged_cloud_beyond_128_workgroups(gpu, oracle_mod):
    """A cloud of 2.1M points takes more than 128 workgroups (at most 16
    points per thread), so its exchange carries up to 512 candidates (eight
    slots per lane of the certifying wave); two small clouds ride along."""
    r = W.ragged_batch(21, [2_100_000, 5000, 300])
    check_fps(gpu, oracle_mod, r.xyz, r.ptr, np.array([48, 50, 10]), what="2.1M-point cloud")
