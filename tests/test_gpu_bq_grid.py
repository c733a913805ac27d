"""Ball Query's grid pass versus the oracle: the culled index-order scan with a
budget of scanned blocks, then a uniform grid for the queries it leaves short
of K. Indices and squared distances bit-exact. Forced on at small sizes with a
budget of a few blocks, so most queries reach the grid pass holding part of
their first K from the scan; and at its default (clouds above 32768 points) on
a clustered cloud whose far samples sit in sparse regions. All calls go
through the C ABI (via the thin Python binding)."""
import numpy as np
import pytest

from point_cloud_neighbor_amd import workloads as W
from tests.gpu_util import assert_dist_close, assert_idx_equal, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture
def grid(monkeypatch):
    monkeypatch.setenv("POINTOPS_BQ_GRID", "1")
    return monkeypatch


def check(gpu, oracle_mod, q, x, r, K, what):
    wd2, wi = oracle_mod.ball_query(q, x, r, K, threads=8)
    d2, i = gpu.ball_query(dev(q), dev(x), r, K)
    assert_idx_equal(host(i), wi, f"bq idx {what}")
    assert_dist_close(host(d2), wd2, f"bq dist2 {what}")


@pytest.mark.parametrize("budget", ["1", "3", "256"])
@pytest.mark.parametrize("K", [1, 7, 31, 32])
def test_budgets_and_K(gpu, oracle_mod, grid, budget, K):
    """Budget 1 and 3: almost every query continues in the grid pass, some with
    hits from the scan; 256: the scan finishes everything and the grid kernels
    return at once."""
    grid.setenv("POINTOPS_BQ_BUDGET", budget)
    x = W.uniform_cube(31, 2, 5000)
    q = W.uniform_cube(32, 2, 300)
    for r in (0.05, 0.15):
        check(gpu, oracle_mod, q, x, r, K, f"budget={budget} K={K} r={r}")


@pytest.mark.parametrize("K", [33, 64, 100])
def test_k_above_32_takes_the_scan(gpu, oracle_mod, grid, K):
    """The grid pass keeps 32 keys per query; larger K scan every block."""
    grid.setenv("POINTOPS_BQ_BUDGET", "1")
    x = W.uniform_cube(33, 1, 3000)
    check(gpu, oracle_mod, x[:, :200].copy(), x, 0.2, K, f"K={K}")


@pytest.mark.parametrize("case", ["clustered", "sorted", "on_radius", "outside", "identical",
                                  "tails"])
def test_cases(gpu, oracle_mod, grid, case):
    grid.setenv("POINTOPS_BQ_BUDGET", "2")
    if case == "clustered":        # dense clusters with exact duplicates, sparse outskirts
        x = W.clustered_cloud(41, N=20000, n_clusters=5, sigma=0.01, dup_frac=0.05)
        q = np.concatenate([x[:, :300], W.uniform_cube(42, 1, 200)], axis=1)
        r, K = 0.03, 32
    elif case == "sorted":         # references already in grid order
        raw = W.uniform_cube(43, 1, 30000)[0]
        x = raw[W.morton_order(raw)][None].copy()
        q = x[:, ::37].copy()
        r, K = 0.05, 32
    elif case == "on_radius":      # dyadic points: many pairs at exactly the radius
        x = W.dyadic_cloud(44, 2, 6000, 16)
        q = W.dyadic_cloud(45, 2, 250, 16)
        r, K = 0.125, 20           # R2 = 1/64 exactly; s = 1/64 is not a hit
    elif case == "outside":        # queries far outside the cloud's box and on its faces
        x = W.uniform_cube(46, 1, 8000)
        q = np.concatenate([W.uniform_cube(47, 1, 100) * np.float32(6.0) - np.float32(3.0),
                            np.clip(W.uniform_cube(48, 1, 100) * np.float32(1.2), 0, 1)],
                           axis=1).astype(np.float32)
        r, K = 0.1, 16
    elif case == "identical":      # one location: its queries see every point as a hit
        x = np.full((1, 4000, 3), 0.25, dtype=np.float32)
        q = np.concatenate([x[:, :5], W.uniform_cube(49, 1, 40)], axis=1)
        r, K = 0.05, 32
    else:                          # ragged block, superblock and tile tails
        x = W.uniform_cube(50, 1, 16385)
        q = W.uniform_cube(51, 1, 129)
        r, K = 0.07, 24
    check(gpu, oracle_mod, q, x, r, K, case)


def test_default_on_a_clustered_cloud(gpu, oracle_mod):
    """No forcing: 200k clustered points (above the 32768 threshold), the
    oracle's 1024 farthest-point samples as queries (most in sparse regions,
    left by the scan's budget), r = 0.03, K = 32."""
    x = W.clustered_cloud(52, N=200000, n_clusters=16, sigma=0.02, dup_frac=0.001)
    c = oracle_mod.fps(x, 1024, 0, threads=8)
    q = np.take_along_axis(x, c[..., None].repeat(3, axis=-1), axis=1)
    check(gpu, oracle_mod, q, x, 0.03, 32, "clustered 200k")


def test_short_workspace_is_an_error(gpu):
    """Above 32768 references the workspace includes the grid pass's room; the
    boxes alone are not enough."""
    import ctypes
    import torch
    from point_cloud_neighbor_amd import ops
    lib = ops._load()
    B, Q, P = 1, 100, 40000
    full = lib.pointops_ball_query_workspace_bytes(B, Q, P)
    boxes = lib.pointops_ball_query_workspace_bytes(B, Q, 30000)
    assert full > boxes > 0
    x = dev(W.uniform_cube(53, B, P))
    d2 = torch.empty((B, Q, 8), device="cuda")
    ix = torch.empty((B, Q, 8), dtype=torch.int64, device="cuda")
    ws = torch.empty(boxes, dtype=torch.uint8, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.pointops_ball_query(x.data_ptr(), x.data_ptr(), B, Q, P, ctypes.c_float(0.1), 8,
                                 d2.data_ptr(), ix.data_ptr(), ws.data_ptr(), boxes, s)
    assert rc == 1  # POINTOPS_INVALID_ARGUMENT


def test_search_choice(gpu):
    """pointops_ball_query_search reports the library's choice."""
    from point_cloud_neighbor_amd import ops
    assert ops.ball_query_search(1, 16384, 1 << 20, 32) == "culled scan, then grid pass"
    assert ops.ball_query_search(1, 100000, 100000, 64) == "culled scan"
    assert ops.ball_query_search(1, 1000, 30000, 32) == "culled scan"
    assert ops.ball_query_search(1, 1000, 100000, 32, cull=False) == "scan"
    with pytest.raises(gpu.PointopsError):
        ops.ball_query_search(1, 10, 5, 0)
