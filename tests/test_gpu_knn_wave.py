"""The one-query-per-wave kNN kernel (k <= 32; one or two queries per wave),
forced on, versus the oracle:
indices bit-exact, distances bit-exact. Shapes cover the LDS tile (1024
references) and chunk (64) tails, workgroups with idle waves, every k up to the
list's 32 slots, heavy ties, identical points and a reference order that makes
every reference a candidate (the buffer overflows and merges on every chunk).
All calls go through the C ABI (via the thin Python binding)."""
import numpy as np
import pytest

from point_cloud_neighbor_amd import workloads as W
from tests.gpu_util import assert_dist_close, assert_idx_equal, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["1", "2"], ids=["qw1", "qw2"])
def wave(monkeypatch, request):
    """The kernel forced on, with one or two queries per wave."""
    monkeypatch.setenv("POINTOPS_KNN_WAVE", "1")
    monkeypatch.setenv("POINTOPS_KNN_WAVE_QW", request.param)
    monkeypatch.setenv("POINTOPS_KNN_GRID", "0")
    return monkeypatch


def check(gpu, oracle_mod, q, x, k, what):
    wd, wi = oracle_mod.knn(q, x, k, threads=8)
    d, i = gpu.knn(dev(q), dev(x), k)
    assert_idx_equal(host(i), wi, f"knn idx {what}")
    assert_dist_close(host(d), wd, f"knn dist {what}")


@pytest.mark.parametrize("k", [1, 2, 3, 7, 16, 17, 31, 32])
def test_k_values(gpu, oracle_mod, wave, k):
    x = W.uniform_cube(300 + k, 2, 1500)       # one full tile and a ragged one
    q = W.uniform_cube(400 + k, 2, 130)
    check(gpu, oracle_mod, q, x, k, f"k={k}")


@pytest.mark.parametrize("Q,P,k", [(1, 1, 1), (1, 32, 32), (5, 63, 20), (9, 64, 32),
                                   (13, 65, 32), (200, 7, 7), (3, 1024, 1), (17, 2048, 32),
                                   (129, 5003, 16), (70, 20011, 32)])
def test_shapes(gpu, oracle_mod, wave, Q, P, k):
    x = W.sphere_shell(P + 7, 1, P)
    q = W.sphere_shell(Q + 8, 1, Q)
    check(gpu, oracle_mod, q, x, k, f"Q={Q} P={P} k={k}")


@pytest.mark.parametrize("nw", ["4", "8", "16"])
def test_waves_per_workgroup(gpu, oracle_mod, wave, nw):
    wave.setenv("POINTOPS_KNN_WAVE_NW", nw)
    x = W.uniform_cube(11, 3, 3001)
    q = W.uniform_cube(12, 3, 37)               # not a multiple of any workgroup's queries
    check(gpu, oracle_mod, q, x, 32, f"nw={nw}")


def test_ties(gpu, oracle_mod, wave):
    """27 distinct locations among 4000 points: every distance repeats."""
    x = W.integer_cloud(13, 2, 4000, 0, 3)
    q = W.integer_cloud(14, 2, 50, 0, 3)
    for k in (1, 5, 32):
        check(gpu, oracle_mod, q, x, k, f"ties k={k}")


def test_identical_points(gpu, oracle_mod, wave):
    """All references equal: the answer is indices 0..k-1 in order."""
    x = np.full((1, 3000, 3), 0.5, dtype=np.float32)
    q = np.concatenate([x[:, :3], W.uniform_cube(15, 1, 10)], axis=1)
    check(gpu, oracle_mod, q, x, 32, "identical")


def test_every_reference_a_candidate(gpu, oracle_mod, wave):
    """References in decreasing distance from the query: each one beats the
    current k-th, so all 5000 pass the candidate test."""
    x = W.uniform_cube(16, 1, 5000)
    q = np.full((1, 1, 3), 0.5, dtype=np.float32)
    s = ((x[0].astype(np.float64) - 0.5) ** 2).sum(axis=1)
    x = x[:, np.argsort(-s, kind="stable")].copy()
    for k in (1, 32):
        check(gpu, oracle_mod, q, x, k, f"decreasing k={k}")


def test_grouping_workload(gpu, oracle_mod, wave):
    """32 clouds of 8192 points near the unit sphere, the oracle's 512 FPS
    samples of each as queries, k = 32."""
    w = W.workload("grouping")
    x = w.xyz
    c = oracle_mod.fps(x, w.fps_m, w.fps_start, threads=8)
    q = np.take_along_axis(x, c[..., None].repeat(3, axis=-1), axis=1)
    check(gpu, oracle_mod, q, x, w.knn_k, "grouping")


@pytest.mark.parametrize("sizes", [[1, 5, 0, 64, 65, 300], [1000, 3000, 17, 2048, 2049],
                                   [20000, 500, 7000, 3, 9000]])
@pytest.mark.parametrize("k", [4, 32])
def test_ragged(gpu, oracle_mod, wave, sizes, k):
    """Clouds with fewer than k references fill the rest with (+inf, -1)."""
    r = W.ragged_batch(17, sizes)
    qcnt = np.array([min(n, 77) for n in r.cnt])
    qcnt[2] = 0                                   # a cloud without queries
    qparts = [r.xyz[r.ptr[b]:r.ptr[b] + qcnt[b]] for b in range(len(sizes))]
    q = np.ascontiguousarray(np.concatenate(qparts, axis=0))
    qptr = np.concatenate([[0], np.cumsum(qcnt)]).astype(np.int64)
    d, i = gpu.knn_ragged(dev(q), qptr, dev(r.xyz), r.ptr, k)
    wd, wi = oracle_mod.knn_ragged(q, qptr[:-1], qcnt, r.xyz, r.ptr[:-1], r.cnt, k, threads=8)
    assert_idx_equal(host(i), wi, f"ragged knn idx {sizes} k={k}")
    assert_dist_close(host(d), wd, f"ragged knn dist {sizes} k={k}")


def test_search_choice(gpu):
    """pointops_knn_search reports the library's choice; the cases follow
    the measured rule (the grid from 8192 references per cloud and 2^22 pairs,
    for k > 32 from 32768 references; without it the wave scan for k <= 32,
    the lane scan for small k with many queries on small clouds), and a shape
    pointops_knn rejects is an error."""
    from point_cloud_neighbor_amd import ops
    assert ops.knn_search(1, 100000, 100000, 16) == "grid"
    assert ops.knn_search(1, 100000, 100000, 16, grid=False) == "full scan, queries per wave"
    assert ops.knn_search(32, 512, 8192, 32) == "grid"
    assert ops.knn_search(32, 512, 8192, 32, grid=False) == "full scan, queries per wave"
    assert ops.knn_search(1, 1024, 100000, 16) == "grid"
    assert ops.knn_search(1, 1024, 100000, 16, grid=False) == "full scan, queries per wave"
    assert ops.knn_search(1, 64, 8192, 16) == "full scan, queries per wave"  # < 2^22 pairs
    assert ops.knn_search(1, 1024, 100000, 33) == "grid"
    assert ops.knn_search(1, 1024, 20000, 33) == "full scan, one query per lane"
    assert ops.knn_search(16, 8192, 2048, 3) == "full scan, one query per lane"
    assert ops.knn_search(1, 100, 1000, 33) == "full scan, one query per lane"
    with pytest.raises(gpu.PointopsError):
        ops.knn_search(1, 10, 5, 6)
