"""Seeded random shapes against the oracle: FPS over forced workgroup and
candidate counts (heavy ties, samples past the distinct points), kNN and Ball
Query over every search path, ragged batches with empty and tiny clouds.
Indices and distance bits must equal the oracle's. The shapes come from a
fixed seed, so every run checks the same cases; a wider sweep of the same kind
is how the FPS tie order between a wave's two reports was found."""

import numpy as np
import pytest

from point_cloud_neighbor_amd import workloads as W
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu

ENV = ("POINTOPS_FPS_MODE", "POINTOPS_FPS_WG_PER_CLOUD", "POINTOPS_FPS_RG", "POINTOPS_FPS_GROUP",
       "POINTOPS_KNN_GRID",
       "POINTOPS_KNN_GRID_WAVE", "POINTOPS_KNN_WAVE", "POINTOPS_BQ_GRID", "POINTOPS_BQ_BUDGET",
       "POINTOPS_BQ_QUERIES_PER_WAVE")


@pytest.fixture
def clean_env(monkeypatch):
    for k in ENV:
        monkeypatch.delenv(k, raising=False)

    def put(d):
        for k in ENV:
            monkeypatch.delenv(k, raising=False)
        for k, v in d.items():
            monkeypatch.setenv(k, str(v))
    return put


def cloud(rng, B, N):
    kind = rng.integers(0, 4)
    s = int(rng.integers(1 << 30))
    if kind == 0:
        return W.uniform_cube(s, B, N)
    if kind == 1:
        return W.integer_cloud(s, B, N, 0, int(rng.integers(2, 6)))
    if kind == 2:
        return W.dyadic_cloud(s, B, N, 8)
    return np.concatenate([W.clustered_cloud(s + b, N=N, n_clusters=int(rng.integers(1, 6)),
                                             sigma=0.02, dup_frac=0.05) for b in range(B)])


def same_bits(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


@pytest.mark.parametrize("seed", range(6))
def test_random_fps(gpu, oracle_mod, clean_env, seed):
    rng = np.random.default_rng(1000 + seed)
    for case in range(12):
        B = int(rng.choice([1, 2, 3]))
        N = int(rng.choice([16, 64, 65, 300, 1000, 3000]))
        x = cloud(rng, B, N)
        M = int(rng.integers(1, 2 * N + 1))
        st = int(rng.integers(0, N))
        G = int(min(rng.integers(1, 13), max(1, N // 4)))
        env = {"POINTOPS_FPS_MODE": "batch" if rng.random() < 0.8 else "step",
               "POINTOPS_FPS_WG_PER_CLOUD": G, "POINTOPS_FPS_RG": int(rng.integers(1, 9))}
        clean_env(env)
        got = host(gpu.furthest_point_sample(dev(x), M, st))
        want = oracle_mod.fps(x, M, st, threads=4)
        assert np.array_equal(got, want), (seed, case, B, N, M, st, env)


@pytest.mark.parametrize("seed", range(4))
def test_random_fps_grouped(gpu, oracle_mod, clean_env, seed):
    """Slices of 4 to 10 points per thread, grouped by position with the folds
    culled per wave (and, for the same shape, not grouped): ties between waves
    that are no longer in index order, duplicates, samples past the distinct
    points of the integer clouds."""
    rng = np.random.default_rng(3000 + seed)
    lib = gpu._load()
    for case in range(5):
        B = int(rng.choice([1, 2]))
        N = int(rng.choice([8000, 12000, 20000, 30000]))
        x = cloud(rng, B, N)
        # 2 or more workgroups of 2881 to 8192 points: 4 to 10 points per thread
        Gs = [g for g in range(2, 16) if 2880 < -(-N // g) <= 8192]
        G = int(rng.choice(Gs))
        M = int(rng.integers(1, 2000 if rng.random() < 0.7 else 4000))
        st = int(rng.integers(0, N))
        want = oracle_mod.fps(x, M, st, threads=8)
        sizes = {}
        for group in (1, 0):
            env = {"POINTOPS_FPS_MODE": "batch", "POINTOPS_FPS_WG_PER_CLOUD": G,
                   "POINTOPS_FPS_RG": int(rng.integers(1, 9)), "POINTOPS_FPS_GROUP": group}
            clean_env(env)
            sizes[group] = lib.pointops_fps_workspace_bytes(B, N, M)
            got = host(gpu.furthest_point_sample(dev(x), M, st))
            assert np.array_equal(got, want), (seed, case, B, N, M, st, env)
        # the grouped plan was taken (its workspace holds the grouped points)
        assert sizes[1] >= sizes[0] + B * N * 16, (seed, case, B, N, G, sizes)


@pytest.mark.parametrize("seed", range(3))
def test_random_fps_wide(gpu, oracle_mod, clean_env, seed):
    """Plans of more than 64 workgroups per cloud (staged exchange words, up
    to 512 candidates in eight slots per lane; sets of more than 1024 words
    gathered by the point waves; slices of four or more points per thread
    grouped by position), forced on clouds with heavy ties."""
    rng = np.random.default_rng(4000 + seed)
    for case in range(4):
        N = int(rng.choice([120000, 300000]))
        x = cloud(rng, 1, N)
        G = int(rng.choice([80, 100, 128, 200, 256]))
        RG = int(rng.choice([r for r in (2, 3, 4) if G * r <= 512]))
        M = int(rng.integers(100, 1200))
        st = int(rng.integers(0, N))
        env = {"POINTOPS_FPS_MODE": "batch", "POINTOPS_FPS_WG_PER_CLOUD": G, "POINTOPS_FPS_RG": RG}
        clean_env(env)
        got = host(gpu.furthest_point_sample(dev(x), M, st))
        want = oracle_mod.fps(x, M, st, threads=8)
        assert np.array_equal(got, want), (seed, case, N, M, st, env)


def test_random_fps_wide_covers_paths():
    """The shapes of test_random_fps_wide reach the point-wave gather and the
    grouped slices (checked on the CPU from the same seeded choices)."""
    seen = set()
    for seed in range(3):
        rng = np.random.default_rng(4000 + seed)
        for case in range(4):
            N = int(rng.choice([120000, 300000]))
            cloud(rng, 1, N)
            G = int(rng.choice([80, 100, 128, 200, 256]))
            RG = int(rng.choice([r for r in (2, 3, 4) if G * r <= 512]))
            rng.integers(100, 1200)
            rng.integers(0, N)
            seen.add((G * (3 * RG + 2) > 1024, -(-N // G) > 2880))
    assert (True, True) in seen or ((True, False) in seen and (False, True) in seen), seen


@pytest.mark.parametrize("seed", range(6))
def test_random_searches(gpu, oracle_mod, clean_env, seed):
    rng = np.random.default_rng(2000 + seed)
    for case in range(6):
        B = int(rng.choice([1, 2]))
        N = int(rng.choice([1, 63, 64, 65, 700, 5000]))
        x = cloud(rng, B, N)
        Q = int(rng.integers(1, min(N, 400) + 1))
        q = x[:, rng.choice(N, size=Q, replace=False)].copy() if rng.random() < 0.5 \
            else W.uniform_cube(int(rng.integers(1 << 30)), B, Q)
        k = int(min(rng.choice([1, 3, 16, 17, 32, 40]), N))
        for env in ({"POINTOPS_KNN_GRID": 0}, {"POINTOPS_KNN_GRID": 0, "POINTOPS_KNN_WAVE": 0},
                    {"POINTOPS_KNN_GRID": 1, "POINTOPS_KNN_GRID_WAVE": 0},
                    {"POINTOPS_KNN_GRID": 1, "POINTOPS_KNN_GRID_WAVE": 2}):
            if k > 32 and env.get("POINTOPS_KNN_GRID_WAVE") == 2:
                continue
            clean_env(env)
            d, i = gpu.knn(dev(q), dev(x), k)
            wd, wi = oracle_mod.knn(q, x, k, threads=8)
            assert np.array_equal(host(i), wi) and same_bits(host(d), wd), (seed, case, env)
        K = int(rng.choice([1, 16, 32, 64, 100]))
        r = float(rng.choice([0.05, 0.2, 0.6, 2.0]))
        for env in ({}, {"POINTOPS_BQ_GRID": 1, "POINTOPS_BQ_BUDGET": 1},
                    {"POINTOPS_BQ_QUERIES_PER_WAVE": 1}):
            clean_env(env)
            d2, j = gpu.ball_query(dev(q), dev(x), r, K)
            wd2, wj = oracle_mod.ball_query(q, x, r, K, threads=8)
            assert np.array_equal(host(j), wj) and same_bits(host(d2), wd2), (seed, case, env)


@pytest.mark.parametrize("seed", range(4))
def test_random_ragged(gpu, oracle_mod, clean_env, seed):
    rng = np.random.default_rng(3000 + seed)
    for case in range(4):
        sizes = [int(rng.choice([0, 1, 5, 64, 65, 700, 3000])) for _ in range(int(rng.integers(1, 6)))]
        if sum(sizes) == 0:
            sizes[0] = 9
        x = np.concatenate([cloud(rng, 1, m)[0] if m else np.zeros((0, 3), np.float32)
                            for m in sizes]).astype(np.float32)
        ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
        counts = np.array([min(m, int(rng.integers(0, 120))) for m in sizes], np.int64)
        gi = bool(rng.random() < 0.5)
        clean_env({"POINTOPS_FPS_MODE": "batch"} if rng.random() < 0.5 else {})
        got = host(gpu.fps_ragged(dev(x), ptr, counts, global_index=gi))
        op = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        want = oracle_mod.fps_ragged(x, ptr[:-1], np.diff(ptr), op[:-1], counts, int(op[-1]),
                                     global_index=gi)
        assert np.array_equal(got, want), (seed, case, sizes, counts)
        qs = [min(m, int(rng.integers(0, 200))) for m in sizes]
        if sum(qs) == 0:
            continue
        starts = ptr[:-1]
        q = np.concatenate([x[starts[b]:starts[b] + qs[b]] for b in range(len(sizes))])
        qptr = np.concatenate([[0], np.cumsum(qs)]).astype(np.int64)
        k = int(rng.choice([1, 8, 16, 33]))
        clean_env({"POINTOPS_KNN_GRID": int(rng.integers(0, 2))})
        d, i = gpu.knn_ragged(dev(q), qptr, dev(x), ptr, k, global_index=gi)
        wd, wi = oracle_mod.knn_ragged(q, qptr[:-1], np.diff(qptr), x, ptr[:-1], np.diff(ptr), k,
                                       global_index=gi, threads=8)
        assert np.array_equal(host(i), wi) and same_bits(host(d), wd), (seed, case, sizes, k)
        K, r = int(rng.choice([4, 32, 64])), float(rng.choice([0.1, 0.5]))
        clean_env({"POINTOPS_BQ_GRID": int(rng.integers(0, 2))})
        d2, j = gpu.ball_query_ragged(dev(q), qptr, dev(x), ptr, r, K, global_index=gi)
        wd2, wj = oracle_mod.ball_query_ragged(q, qptr[:-1], np.diff(qptr), x, ptr[:-1],
                                               np.diff(ptr), r, K, global_index=gi, threads=8)
        assert np.array_equal(host(j), wj) and same_bits(host(d2), wd2), (seed, case, sizes, K)
