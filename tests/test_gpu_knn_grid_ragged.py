"""The kNN grid search on ragged batches (per-cloud records over slots as
large as the batch's largest cloud) versus the oracle's ragged composition:
indices bit-exact, distances bit-exact. Forced on at small sizes
(POINTOPS_KNN_GRID=1) with empty clouds, clouds without queries, clouds with
fewer than k references, k across every list size, local and flat indices,
and padded clouds with lengths; at its default on the ragged benchmark
workload's counts. All calls go through the C ABI (via the thin Python
binding)."""
import numpy as np
import pytest

from point_cloud_neighbor_amd import workloads as W
from tests.gpu_util import assert_dist_close, assert_idx_equal, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["0", "1", "2"], ids=["per_lane", "per_wave", "two_per_wave"])
def grid(monkeypatch, request):
    """The grid search forced on, with one query per lane or (k <= 32) per
    wave."""
    monkeypatch.setenv("POINTOPS_KNN_GRID", "1")
    monkeypatch.setenv("POINTOPS_KNN_GRID_WAVE", request.param)
    return monkeypatch


def ptr_of(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def check(gpu, oracle_mod, q, qcnt, x, xcnt, k, global_index=True, what=""):
    from point_cloud_neighbor_amd import ops
    assert ops.knn_ragged_uses_grid(qcnt, xcnt, k), f"grid not taken {what}"
    qptr, xptr = ptr_of(qcnt), ptr_of(xcnt)
    d, i = gpu.knn_ragged(dev(q), qptr, dev(x), xptr, k, global_index=global_index)
    wd, wi = oracle_mod.knn_ragged(q, qptr[:-1], qcnt, x, xptr[:-1], xcnt, k,
                                   global_index=global_index, threads=8)
    assert_idx_equal(host(i), wi, f"ragged grid knn idx {what}")
    assert_dist_close(host(d), wd, f"ragged grid knn dist {what}")


MIXES = [[1, 5, 0, 64, 65, 300], [1000, 3000, 17, 2048, 2049], [20000, 500, 7000, 3, 9000]]


@pytest.mark.parametrize("sizes", MIXES)
@pytest.mark.parametrize("k", [1, 4, 16, 33, 64])
def test_mixes(gpu, oracle_mod, grid, sizes, k):
    """Queries: a prefix of each cloud (none for the third); clouds with fewer
    than k references fill the rest of their rows with (+inf, -1)."""
    r = W.ragged_batch(60 + k, sizes)
    qcnt = np.array([min(n, 97) for n in r.cnt])
    qcnt[2] = 0
    q = np.ascontiguousarray(np.concatenate([r.xyz[r.ptr[b]:r.ptr[b] + qcnt[b]]
                                             for b in range(len(sizes))], axis=0))
    check(gpu, oracle_mod, q, qcnt, r.xyz, r.cnt, k, what=f"{sizes} k={k}")


def test_local_indices_and_clouds_without_references(gpu, oracle_mod, grid):
    """A cloud with queries and no references, clouds below k, local indices."""
    xs = [0, 1, 3, 16, 17, 1000]
    x = W.ragged_batch(70, xs)
    q = W.ragged_batch(71, [5, 5, 5, 5, 5, 70])
    check(gpu, oracle_mod, q.xyz, q.cnt, x.xyz, x.cnt, 16, global_index=False,
          what="small clouds")


def test_clustered_and_outside(gpu, oracle_mod, grid):
    """Clustered clouds with exact duplicates; queries far outside their
    cloud's box; a cloud of one repeated point."""
    parts = [W.clustered_cloud(72, N=12000, n_clusters=4, sigma=0.01, dup_frac=0.05)[0],
             W.uniform_cube(73, 1, 5000)[0],
             np.full((3000, 3), 0.25, dtype=np.float32)]
    x = np.ascontiguousarray(np.concatenate(parts, axis=0))
    xcnt = np.array([len(p) for p in parts])
    qparts = [parts[0][::50],
              W.uniform_cube(74, 1, 80)[0] * np.float32(6.0) - np.float32(3.0),
              np.concatenate([parts[2][:3], W.uniform_cube(75, 1, 20)[0]], axis=0)]
    q = np.ascontiguousarray(np.concatenate(qparts, axis=0)).astype(np.float32)
    qcnt = np.array([len(p) for p in qparts])
    for k in (1, 8, 32):
        check(gpu, oracle_mod, q, qcnt, x, xcnt, k, what=f"clustered k={k}")


def test_padded_lengths(gpu, oracle_mod, grid):
    """The padded form with lengths takes the same search."""
    B, Qm, Pm = 4, 90, 700
    q = W.uniform_cube(76, B, Qm)
    x = W.uniform_cube(77, B, Pm)
    l1, l2 = np.array([90, 0, 33, 7]), np.array([700, 12, 5, 1])
    d, i = gpu.knn_padded(dev(q), dev(x), 8, l1, l2)
    qo, xo = np.arange(B) * Qm, np.arange(B) * Pm
    wd, wi = oracle_mod.knn_ragged(q.reshape(-1, 3), qo, l1, x.reshape(-1, 3), xo, l2, 8,
                                   global_index=False)
    unw = wi[:, 0] == -2  # rows past a cloud's length: the binding's fill
    wd[unw], wi[unw] = np.inf, -1
    assert_idx_equal(host(i).reshape(-1, 8), wi, "padded grid knn idx")
    assert_dist_close(host(d).reshape(-1, 8), wd, "padded grid knn dist")


def test_workload_takes_the_grid_and_matches_the_scan(gpu, oracle_mod):
    """No forcing: the ragged benchmark workload's counts (16 clouds of 1k to
    64k points, an eighth of each as queries, k = 16) take the grid; its
    results equal the full scan's (grid=False) element by element, and sampled
    rows of every cloud equal the oracle's."""
    from point_cloud_neighbor_amd import ops
    r = W.ragged_workload()
    qcnt = np.asarray(r.fps_counts)
    assert ops.knn_ragged_uses_grid(qcnt, r.cnt, r.knn_k)
    # queries: every eighth point of each cloud (the samples' count and spread)
    q = np.ascontiguousarray(np.concatenate(
        [r.xyz[r.ptr[b]:r.ptr[b] + r.cnt[b]][::8][:qcnt[b]] for b in range(len(r.cnt))],
        axis=0))
    qptr = ptr_of(qcnt)
    assert q.shape[0] == qptr[-1]
    d, i = gpu.knn_ragged(dev(q), qptr, dev(r.xyz), r.ptr, r.knn_k)
    d0, i0 = gpu.knn_ragged(dev(q), qptr, dev(r.xyz), r.ptr, r.knn_k, grid=False)
    d, i, d0, i0 = host(d), host(i), host(d0), host(i0)
    assert np.array_equal(i, i0)
    assert np.array_equal(d.view(np.uint32), d0.view(np.uint32))
    for per_wave in ("0", "1", "2"):  # every grid kernel, whichever the default is
        import os
        os.environ["POINTOPS_KNN_GRID_WAVE"] = per_wave
        try:
            d1, i1 = gpu.knn_ragged(dev(q), qptr, dev(r.xyz), r.ptr, r.knn_k)
        finally:
            del os.environ["POINTOPS_KNN_GRID_WAVE"]
        assert np.array_equal(host(i1), i0), per_wave
        assert np.array_equal(host(d1).view(np.uint32), d0.view(np.uint32)), per_wave
    for b in range(len(r.cnt)):
        lo, hi = int(qptr[b]), min(int(qptr[b]) + 48, int(qptr[b + 1]))
        wd, wi = oracle_mod.knn_ragged(q, np.array([lo]), np.array([hi - lo]), r.xyz,
                                       r.ptr[b:b + 1], r.cnt[b:b + 1], r.knn_k, threads=8)
        assert_idx_equal(i[lo:hi], wi[lo:hi], f"cloud {b}")
        assert_dist_close(d[lo:hi], wd[lo:hi], f"cloud {b}")


def test_skewed_batch_keeps_the_scan(gpu):
    """One large cloud among many small ones: the padding to the largest would
    exceed eight times the points, so the workspace stays the table's."""
    from point_cloud_neighbor_amd import ops
    xcnt = np.array([200000] + [100] * 200)
    qcnt = np.array([25000] + [10] * 200)
    assert not ops.knn_ragged_uses_grid(qcnt, xcnt, 16)
    xcnt = np.array([60000, 50000, 40000])
    qcnt = np.array([9000, 8000, 7000])
    assert ops.knn_ragged_uses_grid(qcnt, xcnt, 16)


def test_shared_reference_rows(gpu, oracle_mod, grid):
    """Clouds whose reference segments overlap (the C ABI allows it; each
    cloud's grid holds its own copies), flat and local indices."""
    from point_cloud_neighbor_amd import ops
    lib = ops._load()
    x = W.uniform_cube(78, 1, 9000)[0]
    r_off, r_cnt = np.array([0, 3000, 8990]), np.array([6000, 6000, 10])
    q = W.uniform_cube(79, 1, 300)[0]
    q_off, q_cnt = np.array([0, 100, 200]), np.array([100, 100, 100])
    for k, gi in ((16, True), (12, False)):
        d, i = ops._search_ragged(lib.pointops_knn_ragged, dev(q), q_off, q_cnt, dev(x), r_off,
                                  r_cnt, k, (k,), gi, float("inf"),
                                  ws_fn=lib.pointops_knn_ragged_workspace_bytes)
        wd, wi = oracle_mod.knn_ragged(q, q_off, q_cnt, x, r_off, r_cnt, k, global_index=gi,
                                       threads=8)
        assert_idx_equal(host(i), wi, f"shared rows k={k} global={gi}")
        assert_dist_close(host(d), wd, f"shared rows k={k} global={gi}")
