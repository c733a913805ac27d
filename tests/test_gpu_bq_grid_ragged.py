"""Ball Query's culled search on ragged batches (an index-order scan with a
budget, then, for the queries it leaves, the grid pass over per-cloud records
with slots as large as the batch's largest cloud, or the scan resumed where
each stopped) versus the oracle's ragged composition: indices bit-exact,
squared distances bit-exact. Forced on at small sizes (POINTOPS_BQ_GRID=1)
with scan budgets of one chunk (nearly every query is left holding some
hits) and the grid pass or the resumed scan taking them, a probe of one
chunk, and the defaults; with empty clouds, clouds without queries or
references, a radius that covers whole clouds, radii through dyadic points, clouds in
grid order, local indices and padded clouds with lengths; at its default on
the ragged benchmark workload's counts. All calls go through the C ABI (via
the thin Python binding)."""
import ctypes

import numpy as np
import pytest

from point_cloud_neighbor_amd import workloads as W
from tests.gpu_util import assert_dist_close, assert_idx_equal, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(params=[("64", "64", "0"), ("64", "64", "1000000000000000000"),
                        ("64", "4096", ""), ("", "", "")],
                ids=["budget64_grid", "budget64_resume", "probe64", "default"])
def grid(monkeypatch, request):
    """The culled search forced on; (probe, budget, the tests left from which
    the grid pass is taken): a one-chunk budget with the grid pass or the
    resumed scan taking every query left, a one-chunk probe, the defaults."""
    monkeypatch.setenv("POINTOPS_BQ_GRID", "1")
    for name, v in zip(("POINTOPS_BQ_PROBE", "POINTOPS_BQ_RAGGED_BUDGET",
                        "POINTOPS_BQ_GRID_PAIRS"), request.param):
        if v:
            monkeypatch.setenv(name, v)
    return monkeypatch


def ptr_of(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def check(gpu, oracle_mod, q, qcnt, x, xcnt, r, K, global_index=True, what=""):
    from point_cloud_neighbor_amd import ops
    assert ops.ball_query_ragged_uses_grid(qcnt, xcnt, K), f"grid not taken {what}"
    qptr, xptr = ptr_of(qcnt), ptr_of(xcnt)
    d2, i = gpu.ball_query_ragged(dev(q), qptr, dev(x), xptr, r, K, global_index=global_index)
    wd2, wi = oracle_mod.ball_query_ragged(q, qptr[:-1], qcnt, x, xptr[:-1], xcnt, r, K,
                                           global_index=global_index, threads=8)
    assert_idx_equal(host(i), wi, f"ragged bq grid idx {what}")
    assert_dist_close(host(d2), wd2, f"ragged bq grid dist2 {what}")


MIXES = [[1, 5, 0, 64, 65, 300], [1000, 3000, 17, 2048, 2049], [20000, 500, 7000, 3, 9000]]


@pytest.mark.parametrize("sizes", MIXES)
@pytest.mark.parametrize("K", [1, 7, 32])
def test_mixes(gpu, oracle_mod, grid, sizes, K):
    """Queries: a prefix of each cloud (none for the third); radii with a few
    and with many hits."""
    x = W.ragged_batch(80 + K, sizes)
    qcnt = np.array([min(n, 97) for n in x.cnt])
    qcnt[2] = 0
    q = np.ascontiguousarray(np.concatenate([x.xyz[x.ptr[b]:x.ptr[b] + qcnt[b]]
                                             for b in range(len(sizes))], axis=0))
    for r in (0.05, 0.3):
        check(gpu, oracle_mod, q, qcnt, x.xyz, x.cnt, r, K, what=f"{sizes} K={K} r={r}")


def test_radius_covers_every_cloud(gpu, oracle_mod, grid):
    """Every reference is a hit: the answer is each cloud's first K indices
    (from the scan, or with a one-chunk budget, through the grid pass and its
    index bound)."""
    x = W.ragged_batch(90, [30000, 5000, 12])
    q = W.ragged_batch(91, [50, 50, 50])
    for K in (1, 32):
        check(gpu, oracle_mod, q.xyz, q.cnt, x.xyz, x.cnt, 2.0, K, what=f"all hits K={K}")


def test_small_clouds_local_indices(gpu, oracle_mod, grid):
    """A cloud with queries and no references, clouds of 1 to 17 points."""
    x = W.ragged_batch(92, [0, 1, 3, 16, 17, 1000])
    q = W.ragged_batch(93, [5, 5, 5, 5, 5, 70])
    check(gpu, oracle_mod, q.xyz, q.cnt, x.xyz, x.cnt, 0.5, 8, global_index=False,
          what="small clouds")


def test_dyadic_and_sorted(gpu, oracle_mod, grid):
    """Dyadic points (pairs at exactly the radius are not hits) and a cloud
    already in grid order (indices follow space)."""
    a = W.dyadic_cloud(94, 1, 6000, 16)[0]
    raw = W.uniform_cube(95, 1, 20000)[0]
    s = raw[W.morton_order(raw)]
    x = np.ascontiguousarray(np.concatenate([a, s], axis=0))
    xcnt = np.array([len(a), len(s)])
    qa = W.dyadic_cloud(96, 1, 250, 16)[0]
    q = np.ascontiguousarray(np.concatenate([qa, s[::41]], axis=0))
    qcnt = np.array([len(qa), len(s[::41])])
    check(gpu, oracle_mod, q, qcnt, x, xcnt, 0.125, 20, what="dyadic + sorted")
    check(gpu, oracle_mod, q, qcnt, x, xcnt, 0.05, 32, what="dyadic + sorted r=0.05")


def test_k_above_32_takes_the_scan(gpu, oracle_mod, grid):
    from point_cloud_neighbor_amd import ops
    assert not ops.ball_query_ragged_uses_grid([10, 10], [5000, 6000], 33)
    x = W.ragged_batch(97, [5000, 6000])
    q = W.ragged_batch(98, [40, 40])
    qptr, xptr = ptr_of(q.cnt), ptr_of(x.cnt)
    d2, i = gpu.ball_query_ragged(dev(q.xyz), qptr, dev(x.xyz), xptr, 0.2, 40)
    wd2, wi = oracle_mod.ball_query_ragged(q.xyz, qptr[:-1], q.cnt, x.xyz, xptr[:-1], x.cnt,
                                           0.2, 40, threads=8)
    assert_idx_equal(host(i), wi, "K=40")
    assert_dist_close(host(d2), wd2, "K=40")


def test_padded_lengths(gpu, oracle_mod, grid):
    B, Qm, Pm = 4, 90, 700
    q = W.uniform_cube(99, B, Qm)
    x = W.uniform_cube(100, B, Pm)
    l1, l2 = np.array([90, 0, 33, 7]), np.array([700, 12, 5, 1])
    d2, j = gpu.ball_query_padded(dev(q), dev(x), 0.3, 16, l1, l2)
    qo, xo = np.arange(B) * Qm, np.arange(B) * Pm
    wd2, wj = oracle_mod.ball_query_ragged(q.reshape(-1, 3), qo, l1, x.reshape(-1, 3), xo, l2,
                                           0.3, 16, global_index=False)
    unw = wj[:, 0] == -2  # rows past a cloud's length: the binding's fill
    wd2[unw], wj[unw] = 0.0, -1
    assert_idx_equal(host(j).reshape(-1, 16), wj, "padded grid bq idx")
    assert_dist_close(host(d2).reshape(-1, 16), wd2, "padded grid bq dist2")


def test_workload_takes_the_grid_and_matches_the_scan(gpu, oracle_mod):
    """No forcing: the ragged benchmark workload's counts (16 clouds of 1k to
    64k points, an eighth of each as queries, r = 0.1, K = 32) take the culled
    search; its results equal the plain index-order scan's (grid=False)
    element by element, and sampled rows of every cloud equal the oracle's."""
    from point_cloud_neighbor_amd import ops
    r = W.ragged_workload()
    qcnt = np.asarray(r.fps_counts)
    assert ops.ball_query_ragged_uses_grid(qcnt, r.cnt, r.bq_k)
    q = np.ascontiguousarray(np.concatenate(
        [r.xyz[r.ptr[b]:r.ptr[b] + r.cnt[b]][::8][:qcnt[b]] for b in range(len(r.cnt))],
        axis=0))
    qptr = ptr_of(qcnt)
    d2, i = gpu.ball_query_ragged(dev(q), qptr, dev(r.xyz), r.ptr, r.bq_radius, r.bq_k)
    e2, j = gpu.ball_query_ragged(dev(q), qptr, dev(r.xyz), r.ptr, r.bq_radius, r.bq_k,
                                  grid=False)
    d2, i, e2, j = host(d2), host(i), host(e2), host(j)
    assert np.array_equal(i, j)
    assert np.array_equal(d2.view(np.uint32), e2.view(np.uint32))
    for b in range(len(r.cnt)):
        lo, hi = int(qptr[b]), min(int(qptr[b]) + 48, int(qptr[b + 1]))
        wd2, wi = oracle_mod.ball_query_ragged(q, np.array([lo]), np.array([hi - lo]), r.xyz,
                                               r.ptr[b:b + 1], r.cnt[b:b + 1], r.bq_radius,
                                               r.bq_k, threads=8)
        assert_idx_equal(i[lo:hi], wi[lo:hi], f"cloud {b}")
        assert_dist_close(d2[lo:hi], wd2[lo:hi], f"cloud {b}")


def test_small_clouds_keep_the_scan(gpu):
    from point_cloud_neighbor_amd import ops
    assert not ops.ball_query_ragged_uses_grid([100, 100], [4000, 8000], 32)
    assert ops.ball_query_ragged_uses_grid([100, 100], [4000, 8192], 32)


def test_shared_reference_rows(gpu, oracle_mod, grid):
    """Clouds whose reference segments overlap (the C ABI allows it; each
    cloud's grid holds its own copies), flat and local indices."""
    from point_cloud_neighbor_amd import ops
    lib = ops._load()
    x = W.uniform_cube(101, 1, 30000)[0]
    r_off, r_cnt = np.array([0, 10000, 29990]), np.array([20000, 20000, 10])
    q = W.uniform_cube(102, 1, 300)[0]
    q_off, q_cnt = np.array([0, 100, 200]), np.array([100, 100, 100])
    for K, gi in ((32, True), (9, False)):
        d2, i = ops._search_ragged(lib.pointops_ball_query_ragged, dev(q), q_off, q_cnt, dev(x),
                                   r_off, r_cnt, K, (ctypes.c_float(0.04), K), gi, 0.0,
                                   ws_fn=lib.pointops_ball_query_ragged_workspace_bytes)
        wd2, wi = oracle_mod.ball_query_ragged(q, q_off, q_cnt, x, r_off, r_cnt, 0.04, K,
                                               global_index=gi, threads=8)
        assert_idx_equal(host(i), wi, f"shared rows K={K} global={gi}")
        assert_dist_close(host(d2), wd2, f"shared rows K={K} global={gi}")
