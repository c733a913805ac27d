"""GPU path versus the oracle, element by element, on seeded inputs that span
several tiles and ragged tails, plus the edge cases of each operation.

All calls go through the C ABI (via the thin Python binding)."""
import ctypes
import json
import os

import numpy as np
import pytest
import torch

from point_cloud_neighbor_amd import workloads as W
from tests.gpu_util import assert_dist_close, assert_idx_equal, dev, gather, host

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def check_fps(gpu, oracle_mod, xyz, M, start=0, what=""):
    got, gxyz = gpu.furthest_point_sample(dev(xyz), M, start, return_xyz=True)
    want = oracle_mod.fps(xyz, M, start, threads=4)
    assert_idx_equal(host(got), want, f"fps {what}")
    # the sampled coordinates are bit copies of the chosen points
    assert np.array_equal(host(gxyz).view(np.uint32), gather(xyz, want).view(np.uint32))
    return want


def check_knn(gpu, oracle_mod, q, x, k, what=""):
    """Every search: the full scan and the grid search (forced on, whatever
    the size), the latter with one query per lane and, for k <= 32, one or
    two per wave."""
    wd, wi = oracle_mod.knn(q, x, k, threads=8)
    runs = [("0", "0"), ("1", "0")] + ([("1", "1"), ("1", "2")] if k <= 32 else [])
    for grid, per_wave in runs:
        old = {n: os.environ.get(n) for n in ("POINTOPS_KNN_GRID", "POINTOPS_KNN_GRID_WAVE")}
        os.environ["POINTOPS_KNN_GRID"] = grid
        os.environ["POINTOPS_KNN_GRID_WAVE"] = per_wave
        try:
            d, i = gpu.knn(dev(q), dev(x), k)
        finally:
            for n, v in old.items():
                if v is None:
                    del os.environ[n]
                else:
                    os.environ[n] = v
        how = f"grid={grid} per_wave={per_wave}"
        assert_idx_equal(host(i), wi, f"knn idx {what} {how}")
        assert_dist_close(host(d), wd, f"knn dist {what} {how}")


def check_bq(gpu, oracle_mod, q, x, r, K, what=""):
    """Both scans: with the bounding-box culling (the default) and without."""
    wd, wi = oracle_mod.ball_query(q, x, r, K, threads=8)
    for cull in (True, False):
        d2, i = gpu.ball_query(dev(q), dev(x), r, K, cull=cull)
        assert_idx_equal(host(i), wi, f"bq idx {what} cull={cull}")
        assert_dist_close(host(d2), wd, f"bq dist2 {what} cull={cull}")


# ------------------------------------------------------------------ the pages' example

def test_worked_example(gpu, oracle_mod):
    with open(os.path.join(GOLDEN, "unit_square.json")) as f:
        g = json.load(f)
    xyz = np.array(g["xyz"], dtype=np.float32)
    c, cx = gpu.furthest_point_sample(dev(xyz), g["fps_npoint"], g["fps_start_idx"],
                                      return_xyz=True)
    assert host(c).tolist() == g["fps_idx"]
    d, i = gpu.knn(cx, dev(xyz), g["knn_k"])
    assert host(i).tolist() == g["knn_idx"]
    assert host(d).tolist() == g["derived"]["knn_dist"]
    d2, j = gpu.ball_query(cx, dev(xyz), g["bq_radius"], g["bq_K"])
    assert host(j).tolist() == g["bq_idx"]
    assert host(d2).tolist() == g["derived"]["bq_dist2"]


# ------------------------------------------------------------------ exact (integer / dyadic) clouds

EXACT = [
    ("int4", lambda s: W.integer_cloud(s, 2, 300, 0, 4)),
    ("int2", lambda s: W.integer_cloud(s, 1, 1100, 0, 2)),
    ("int_wide", lambda s: W.integer_cloud(s, 3, 777, -1000, 1000)),
    ("dyadic", lambda s: W.dyadic_cloud(s, 2, 2049, 64)),
]


@pytest.mark.parametrize("name,make", EXACT)
def test_exact_clouds_all_ops(gpu, oracle_mod, name, make):
    xyz = make(0)
    B, N, _ = xyz.shape
    for M, start in [(1, 0), (37, N - 1), (N, 5), (N + 9, 2)]:
        check_fps(gpu, oracle_mod, xyz, M, start, f"{name} M={M}")
    q = xyz[:, ::5].copy()
    for k in (1, 3, 16, 17, 64):
        check_knn(gpu, oracle_mod, q, xyz, k, f"{name} k={k}")
    scale = 64.0 if name == "dyadic" else (300.0 if name == "int_wide" else 1.0)
    for r in (1.0, 1.5, 2.0):
        for K in (1, 31, 64, 65, 300):
            check_bq(gpu, oracle_mod, q, xyz, r * scale if name != "dyadic" else r / 8, K,
                     f"{name} r={r} K={K}")


# ------------------------------------------------------------------ float clouds, shapes and tails

@pytest.mark.parametrize("B,N", [(1, 1), (1, 2), (1, 63), (1, 64), (2, 65), (1, 1000), (3, 1025),
                                 (1, 4097), (2, 20000), (1, 70001)])
def test_fps_shapes(gpu, oracle_mod, B, N):
    xyz = W.uniform_cube(N, B, N)
    for M in sorted({1, 2, min(N, 100), N + 3 if N < 2000 else 300}):
        check_fps(gpu, oracle_mod, xyz, M, N // 3, f"B={B} N={N} M={M}")


@pytest.mark.parametrize("mode", ["batch", "step"])
@pytest.mark.parametrize("G", [2, 3, 7, 16, 33])
def test_fps_forced_workgroups_per_cloud(gpu, oracle_mod, G, mode, monkeypatch):
    """The cross-workgroup exchange, forced on mid-sized clouds, for both the
    certified-batch kernel and the one-exchange-per-step kernel; twice, same bits."""
    monkeypatch.setenv("POINTOPS_FPS_MODE", mode)
    monkeypatch.setenv("POINTOPS_FPS_WG_PER_CLOUD", str(G))
    xyz = W.sphere_shell(G, 2, 5000 + G)
    want = check_fps(gpu, oracle_mod, xyz, 700, 11, f"G={G}")
    again = host(gpu.furthest_point_sample(dev(xyz), 700, 11))
    assert np.array_equal(again, want)


@pytest.mark.parametrize("mode", ["batch", "step"])
def test_fps_ties_and_duplicates(gpu, oracle_mod, mode, monkeypatch):
    monkeypatch.setenv("POINTOPS_FPS_MODE", mode)
    xyz = W.integer_cloud(5, 2, 3000, 0, 3)      # 27 distinct locations, heavy ties
    for G in ("1", "5"):
        monkeypatch.setenv("POINTOPS_FPS_WG_PER_CLOUD", G)
        check_fps(gpu, oracle_mod, xyz, 60, 7, f"dups G={G}")
    monkeypatch.delenv("POINTOPS_FPS_WG_PER_CLOUD")
    line = W.line_cloud(1025)
    check_fps(gpu, oracle_mod, line, 1030, 0, "line")


@pytest.mark.parametrize("G,rg", [("4", "4"), ("16", "2"), ("16", "8")])
def test_fps_batches_past_the_distinct_points(gpu, oracle_mod, monkeypatch, G, rg):
    """Certified batches over several workgroups once every distinct location
    is taken: 64 locations among 5000 points, 3000 samples, so from the 65th
    sample on every key is 0 and equals the bound's, and each centre passes
    only by its index (the full test that a certification block falls back
    to); also a cloud of one repeated point."""
    monkeypatch.setenv("POINTOPS_FPS_MODE", "batch")
    monkeypatch.setenv("POINTOPS_FPS_WG_PER_CLOUD", G)
    monkeypatch.setenv("POINTOPS_FPS_RG", rg)
    xyz = W.integer_cloud(77, 1, 5000, 0, 4)
    check_fps(gpu, oracle_mod, xyz, 3000, 17, f"64 locations G={G} rg={rg}")
    same = np.full((1, 3000, 3), 0.25, dtype=np.float32)
    check_fps(gpu, oracle_mod, same, 700, 5, f"one location G={G} rg={rg}")


@pytest.mark.parametrize("G,rg", [("1", "30"), ("2", "8"), ("4", "3"), ("8", "2"), ("8", "3")])
def test_fps_candidates_in_index_order(gpu, oracle_mod, monkeypatch, G, rg):
    """A wave reports its two largest keys in key order, so the larger key can
    carry the larger index; keys that differ at the exchange can become equal
    as centres are folded in (here: 0, once every distinct point is taken),
    and then the smaller index must win. Small clouds sampled past their
    distinct points, over several workgroup and candidate counts; the first
    is the cloud where index 1 was taken instead of 0."""
    monkeypatch.setenv("POINTOPS_FPS_MODE", "batch")
    monkeypatch.setenv("POINTOPS_FPS_WG_PER_CLOUD", G)
    monkeypatch.setenv("POINTOPS_FPS_RG", rg)
    check_fps(gpu, oracle_mod, W.clustered_cloud(570096078, N=64, n_clusters=5, sigma=0.02),
              73, 63, f"clustered 64 G={G} rg={rg}")
    for seed in range(12):
        x = (W.clustered_cloud(seed, N=96, n_clusters=4, sigma=0.03) if seed % 2
             else W.uniform_cube(seed, 2, 96))
        check_fps(gpu, oracle_mod, x, 120, seed % 96, f"seed {seed} G={G} rg={rg}")


@pytest.mark.parametrize("G,rg,block", [(1, 0, 256), (1, 0, 1024), (4, 1, 1024), (4, 15, 1024),
                                        (4, 30, 1024), (9, 3, 1024), (40, 2, 1024),
                                        (63, 4, 1024), (70, 1, 1024), (130, 1, 1024),
                                        (130, 3, 1024), (200, 2, 1024), (256, 2, 1024),
                                        (3, 1, 256), (3, 6, 256)])
def test_fps_batch_shapes(gpu, oracle_mod, G, rg, block, monkeypatch):
    """Certified-batch kernel over workgroup counts, published candidates per
    workgroup (1 .. all 2 * point-wave reports) and block sizes, including more
    candidates than lanes."""
    monkeypatch.setenv("POINTOPS_FPS_MODE", "batch")
    monkeypatch.setenv("POINTOPS_FPS_WG_PER_CLOUD", str(G))
    monkeypatch.setenv("POINTOPS_FPS_BLOCK", str(block))
    if rg:
        monkeypatch.setenv("POINTOPS_FPS_RG", str(rg))
    N = min(40 * G + 2000, 60000)
    xyz = W.uniform_cube(G + 100, 1, N)
    check_fps(gpu, oracle_mod, xyz, 600, 3, f"batch G={G} rg={rg} block={block}")
    xi = W.integer_cloud(G, 1, N, 0, 5)
    check_fps(gpu, oracle_mod, xi, 200, 0, f"batch ints G={G} rg={rg} block={block}")


@pytest.mark.parametrize("G,rg", [(4, 30), (64, 4), (33, 7), (130, 3)])
def test_fps_batch_many_live_candidates(gpu, oracle_mod, G, rg, monkeypatch):
    """Every workgroup's slice (1920 points: 15 point waves of 128) is a tiny
    cluster plus `rg` far outliers, one or two per point wave, so each
    workgroup publishes outliers only and its bound is a cluster point: the
    first batches keep all G * rg candidates live (up to eight slots per lane
    above 128 workgroups, the general certification loop), later ones one or
    two."""
    monkeypatch.setenv("POINTOPS_FPS_MODE", "batch")
    monkeypatch.setenv("POINTOPS_FPS_WG_PER_CLOUD", str(G))
    monkeypatch.setenv("POINTOPS_FPS_BLOCK", "1024")
    monkeypatch.setenv("POINTOPS_FPS_RG", str(rg))
    per = 1920
    xyz = W.uniform_cube(500 + G, 1, G * per) * np.float32(0.01)
    far = W.sphere_shell(600 + G, 1, G * rg, sigma=0.0) * np.float32(10.0)
    pos = [(k % 15) * 128 + k // 15 for k in range(rg)]
    for g in range(G):
        xyz[0, [g * per + p for p in pos]] = far[0, g * rg:(g + 1) * rg]
    check_fps(gpu, oracle_mod, xyz, 700, per // 2, f"many live G={G} rg={rg}")


@pytest.mark.parametrize("k", [1, 2, 3, 5, 8, 15, 16, 17, 31, 32, 33, 63, 64])
def test_knn_k_values(gpu, oracle_mod, k):
    x = W.uniform_cube(100 + k, 2, 1500)
    q = W.uniform_cube(200 + k, 2, 130)
    check_knn(gpu, oracle_mod, q, x, k, f"k={k}")


@pytest.mark.parametrize("Q,P,k", [(1, 1, 1), (1, 16, 16), (63, 64, 7), (65, 65, 64),
                                   (64, 100, 8), (200, 7, 7), (129, 5003, 16), (70, 20011, 32)])
def test_knn_shapes(gpu, oracle_mod, Q, P, k):
    x = W.sphere_shell(P, 1, P)
    q = W.sphere_shell(Q + 1, 1, Q)
    check_knn(gpu, oracle_mod, q, x, k, f"Q={Q} P={P} k={k}")


@pytest.mark.parametrize("case", ["clustered", "outside", "identical", "sorted", "lines"])
def test_knn_grid_search_cases(gpu, oracle_mod, case):
    """Clouds that stress the grid search: dense clusters with exact
    duplicates, queries far outside the references' box (clamped cells), a
    cloud of identical points (one cell, all ties), references already in
    grid order, and points on a few lines (many equal distances)."""
    if case == "clustered":
        x = W.clustered_cloud(41, N=20000, n_clusters=5, sigma=0.01, dup_frac=0.05)
        q = np.concatenate([x[:, :300], W.uniform_cube(42, 1, 200)], axis=1)
    elif case == "outside":
        x = W.uniform_cube(43, 2, 9000)
        q = (W.uniform_cube(44, 2, 400) * np.float32(5.0) - np.float32(2.0)).astype(np.float32)
    elif case == "identical":
        x = np.full((1, 5000, 3), 0.25, dtype=np.float32)
        q = np.concatenate([x[:, :10], W.uniform_cube(45, 1, 60)], axis=1)
    elif case == "sorted":
        raw = W.uniform_cube(46, 1, 30000)[0]
        x = raw[W.morton_order(raw)][None].copy()
        q = x[:, ::37].copy()
    else:
        t = W.integer_cloud(47, 1, 12000, 0, 64).astype(np.float32)
        t[..., 1:] = np.floor(t[..., 1:] / 32) * 32      # 4 lines per axis pair
        x = t
        q = x[:, ::29].copy()
    for k in (1, 16, 33, 64):
        check_knn(gpu, oracle_mod, q, x, k, f"{case} k={k}")


@pytest.mark.parametrize("waves", ["1", "2", "4", "8"])
def test_knn_grid_waves_agree(gpu, oracle_mod, waves, monkeypatch):
    monkeypatch.setenv("POINTOPS_KNN_GRID_WAVES", waves)
    x = W.uniform_cube(10, 1, 20000)
    check_knn(gpu, oracle_mod, x[:, ::41].copy(), x, 16, f"grid waves={waves}")


@pytest.mark.parametrize("env", ["1", "2", "4", "8"])
@pytest.mark.parametrize("k", [5, 16, 32])
def test_knn_wave_split_agrees(gpu, oracle_mod, env, k, monkeypatch):
    monkeypatch.setenv("POINTOPS_KNN_WAVES", env)
    x = W.uniform_cube(9, 1, 3001)
    check_knn(gpu, oracle_mod, x[:, :97].copy(), x, k, f"waves={env} k={k}")


@pytest.mark.parametrize("Q,P,K,r", [(1, 0, 4, 0.5), (5, 1, 1, 0.5), (63, 64, 31, 0.3),
                                     (65, 65, 33, 0.3), (130, 1000, 64, 0.2),
                                     (200, 5000, 65, 0.15), (100, 3000, 200, 0.5),
                                     (64, 4096, 1, 0.05)])
def test_ball_query_shapes(gpu, oracle_mod, Q, P, K, r):
    x = W.uniform_cube(P + 1, 2, P)
    q = W.uniform_cube(Q + 2, 2, Q)
    check_bq(gpu, oracle_mod, q, x, r, K, f"Q={Q} P={P} K={K} r={r}")


@pytest.mark.parametrize("qw", ["1", "2", "4", "8", "16"])
def test_ball_query_queries_per_wave(gpu, oracle_mod, qw, monkeypatch):
    monkeypatch.setenv("POINTOPS_BQ_QUERIES_PER_WAVE", qw)
    x = W.uniform_cube(3, 1, 2500)
    check_bq(gpu, oracle_mod, x[:, :77].copy(), x, 0.12, 40, f"qw={qw}")


@pytest.mark.parametrize("case", ["dyadic", "planted", "uniform"])
def test_ball_query_culling_on_sorted_clouds(gpu, oracle_mod, case):
    """Morton-sorted clouds, where the bounding-box test skips most blocks:
    dyadic coordinates put many block bounds and distances exactly on R2, the
    planted cloud has pairs at prev(R2), R2 and next(R2)."""
    if case == "dyadic":
        raw = W.integer_cloud(31, 1, 6000, 0, 8)[0] / np.float32(8)
        x = raw[W.morton_order(raw)][None].copy()
        r = 0.25                                  # R2 = 1/16 exactly
        q = np.concatenate([x[:, ::7], x[:, 5:400]], axis=1)
    elif case == "planted":
        x = W.sorted_bq_cloud(32, N=8000, n_anchor=40)
        r = 0.05
        q = x.copy()
    else:
        raw = W.uniform_cube(33, 1, 20000)[0]
        x = raw[W.morton_order(raw)][None].copy()
        r = 0.03
        q = W.uniform_cube(34, 1, 700)
    for K in (1, 16, 64, 200):
        check_bq(gpu, oracle_mod, q, x, r, K, f"sorted {case} K={K}")


def test_ball_query_planted_boundary(gpu, oracle_mod):
    rng = np.random.default_rng(3)
    xyz = (np.round(rng.random((400, 3)) * 64) / 64).astype(np.float32)
    planted = W.plant_radius_partners(rng, xyz, np.arange(40), np.arange(40, 160),
                                      W.R2_BITS[0.05])
    x = xyz[None]
    check_bq(gpu, oracle_mod, x[:, :40].copy(), x, 0.05, 64, "planted")
    d2, idx = gpu.ball_query(dev(x[:, :40].copy()), dev(x), 0.05, 64)
    idx = host(idx)[0]
    m = W.R2_BITS[0.05] & 0x7FFFFF | 0x800000
    for a, v, num in planted:
        assert (v in idx[a]) == (num < m), (a, v, num)


def test_subnormal_distances(gpu, oracle_mod):
    x = W.subnormal_cloud(5, 300)
    q = x[:, :40].copy()
    check_knn(gpu, oracle_mod, q, x, 9, "subnormal")
    check_bq(gpu, oracle_mod, q, x, 3e-20, 50, "subnormal")
    check_fps(gpu, oracle_mod, x, 50, 0, "subnormal")


def test_self_queries_and_duplicates(gpu, oracle_mod):
    x = W.uniform_cube(8, 1, 2000)
    x[0, 1500] = x[0, 3]      # exact duplicate with a larger index
    x[0, 10] = x[0, 700]      # and with a smaller one
    check_knn(gpu, oracle_mod, x, x, 4, "self")
    check_bq(gpu, oracle_mod, x, x, 0.03, 8, "self")


def test_noncontiguous_inputs(gpu, oracle_mod):
    base = W.uniform_cube(12, 2, 2000)
    t = dev(base)[:, ::2]                      # a strided view
    d, i = gpu.knn(t, t, 5)
    wd, wi = oracle_mod.knn(base[:, ::2].copy(), base[:, ::2].copy(), 5)
    assert_idx_equal(host(i), wi, "strided")


# ------------------------------------------------------------------ unwritten slots, errors

def _raw_lib():
    from point_cloud_neighbor_amd import ops
    return ops._load()


def test_every_output_slot_written(gpu):
    """Outputs prefilled with sentinels (NaN bits, index -2) come back with no
    sentinel left, through the C ABI directly."""
    lib = _raw_lib()
    x = dev(W.uniform_cube(21, 2, 3000))
    q = x[:, :150].contiguous()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    wsb = torch.empty(lib.pointops_ball_query_workspace_bytes(2, 150, 3000), dtype=torch.uint8,
                      device="cuda")
    for K in (1, 33, 100):
        for ws in (None, wsb):
            d2 = torch.full((2, 150, K), float("nan"), device="cuda")
            ix = torch.full((2, 150, K), -2, dtype=torch.int64, device="cuda")
            assert lib.pointops_ball_query(q.data_ptr(), x.data_ptr(), 2, 150, 3000,
                                           ctypes.c_float(0.1), K, d2.data_ptr(), ix.data_ptr(),
                                           None if ws is None else ws.data_ptr(),
                                           0 if ws is None else ws.numel(), s) == 0
            assert not torch.isnan(d2).any() and not (ix == -2).any()
    # a workspace that is too small is an error, not a silent fallback
    assert lib.pointops_ball_query(q.data_ptr(), x.data_ptr(), 2, 150, 3000, ctypes.c_float(0.1),
                                   4, d2.data_ptr(), ix.data_ptr(), wsb.data_ptr(), 16, s) == 1
    d = torch.full((2, 150, 20), float("nan"), device="cuda")
    ix = torch.full((2, 150, 20), -2, dtype=torch.int64, device="cuda")
    assert lib.pointops_knn(q.data_ptr(), x.data_ptr(), 2, 150, 3000, 20, d.data_ptr(),
                            ix.data_ptr(), None, 0, s) == 0
    assert not torch.isnan(d).any() and not (ix < 0).any()
    ws = torch.empty(lib.pointops_fps_workspace_bytes(2, 3000, 64), dtype=torch.uint8, device="cuda")
    o = torch.full((2, 64), -2, dtype=torch.int64, device="cuda")
    assert lib.pointops_fps(x.data_ptr(), 2, 3000, 64, 0, o.data_ptr(), None, ws.data_ptr(),
                            ws.numel(), s) == 0
    assert not (o < 0).any()


@pytest.mark.parametrize("mode,N,G", [("batch", 20000, 8), ("step", 20000, 8),
                                      ("batch", 400000, None), ("batch", 800000, None)])
def test_fps_bounded_wait_terminates(gpu, mode, N, G, monkeypatch):
    """A tiny bound on the cross-workgroup wait (forced from the host) makes the
    kernel stop early instead of waiting: the call returns, output slots not
    reached hold -1 and the rest are valid indices. The two large clouds take
    256 workgroups, whose 2048 exchange words the point waves gather (after
    a bounded wait for their own workgroup's words); the larger one also
    groups its slices."""
    monkeypatch.setenv("POINTOPS_FPS_MODE", mode)
    if G:
        monkeypatch.setenv("POINTOPS_FPS_WG_PER_CLOUD", str(G))
    monkeypatch.setenv("POINTOPS_FPS_SPIN_LIMIT", "0")
    xyz = dev(W.uniform_cube(4, 1, N))
    ws = torch.empty(gpu.fps_workspace_bytes(1, N, 500), dtype=torch.uint8, device="cuda")
    out = host(gpu.furthest_point_sample(xyz, 500, workspace=ws, check=False))
    torch.cuda.synchronize()
    assert ((out >= 0) & (out < N) | (out == -1)).all()
    first_bad = np.argmax(out[0] == -1) if (out == -1).any() else 500
    assert (out[0, first_bad:] == -1).all()
    # the give-up is reported: through the status query of the C ABI and as
    # an exception of the checked binding (a zero bound gives up at the first
    # poll that finds a workgroup missing: over 499 steps of 8 workgroups
    # some poll always does)
    with pytest.raises(gpu.PointopsError) as err:
        gpu.fps_status(ws)
    assert err.value.status == 5
    assert (out == -1).any()
    with pytest.raises(gpu.PointopsError) as err:
        gpu.furthest_point_sample(xyz, 500)
    assert err.value.status == 5
    # without the bound the same call succeeds and its status clears
    monkeypatch.delenv("POINTOPS_FPS_SPIN_LIMIT")
    out = host(gpu.furthest_point_sample(xyz, 500, workspace=ws))
    gpu.fps_status(ws)
    assert (out >= 0).all()


def test_unsupported_device_is_an_error(gpu):
    from point_cloud_neighbor_amd import ops
    import subprocess, sys
    code = ("import os, torch; os.environ['POINTOPS_FORCE_UNSUPPORTED_DEVICE']='1';"
            "from point_cloud_neighbor_amd import ops;"
            "x=torch.zeros(1,8,3,device='cuda')\n"
            "try:\n ops.knn(x,x,2); print('NOERR')\n"
            "except ops.PointopsError as e: print('ERR', e.status)")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))), timeout=120)
    assert "ERR 3" in r.stdout, r.stdout + r.stderr


def test_invalid_arguments_raise(gpu):
    x = dev(W.uniform_cube(1, 1, 10))
    with pytest.raises(gpu.PointopsError):
        gpu.knn(x, x, 11)
    with pytest.raises(gpu.PointopsError):
        gpu.knn(x, x, 0)
    with pytest.raises(gpu.PointopsError):
        gpu.furthest_point_sample(x, 3, 10)
    with pytest.raises(gpu.PointopsError):
        gpu.ball_query(x, x, -1.0, 3)
    with pytest.raises(gpu.PointopsError):
        gpu.knn(x.double(), x.double(), 2)


def test_fps_two_large_clouds(gpu, oracle_mod):
    """Two clouds of 400k points: each would take 256 workgroups, which do not
    fit on the device at once, so the plan falls back to fewer per cloud."""
    xyz = W.uniform_cube(61, 2, 400000)
    check_fps(gpu, oracle_mod, xyz, 40, 7, "2 x 400k")
