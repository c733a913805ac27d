"""The five benchmark workloads at full size, compared with the oracle over
their WHOLE outputs (the project page counts mismatches over whole outputs,
section "Correctness checks").

Whole outputs are compared through the oracle's stored digests
(``tests/digests.py``); a mismatch is located by chunk and shown element by
element against the oracle recomputed on those rows. Where the oracle takes
seconds (the sorted Ball Query, an FPS prefix, sampled kNN rows) it also runs
here directly, independent of the stored values.

Launch configurations: the calls the benchmark times (workspaces given, so
kNN takes the grid search and Ball Query the culled scan), the full scans
(no workspace), and the benchmark's two-stream schedule (FPS on one stream,
kNN then Ball Query on a second beside it), repeated."""
import os

import numpy as np
import pytest
import torch

from point_cloud_neighbor_amd import workloads as W
from tests import digests as D
from tests.gpu_util import assert_dist_close, assert_idx_equal, dev, gather, host

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)


def flat_rows(a, lo, hi):
    return W.output_rows(np.asarray(a))[lo:hi]


def knn_rows(oracle_mod, q, x, k):
    def f(lo, hi):
        d, i = oracle_mod.knn(q, x, k, rows=(lo, hi), threads=THREADS)
        return flat_rows(d, lo, hi), flat_rows(i, lo, hi)
    return f


def bq_rows(oracle_mod, q, x, r, K):
    def f(lo, hi):
        d, i = oracle_mod.ball_query(q, x, r, K, rows=(lo, hi), threads=THREADS)
        return flat_rows(d, lo, hi), flat_rows(i, lo, hi)
    return f


def fps_rows(oracle_mod, x, M, start):
    def f(lo, hi):
        B = x.shape[0]
        c = oracle_mod.fps(x, M if B > 1 else min(M, hi), start, threads=THREADS)
        return None, flat_rows(c, lo, hi)
    return f


def check_fps(gpu_idx, oracle_mod, w, what):
    D.assert_matches(host(gpu_idx), None, D.entry(w.name, "fps"), what,
                     fps_rows(oracle_mod, w.xyz, w.fps_m, w.fps_start))


def test_inputs_are_the_digested_ones():
    """The generators reproduce the inputs the digests were taken on."""
    for name in ("tiny", "grouping", "large", "sorted_bq", "stress"):
        assert W.output_digest(W.workload(name).xyz, "dist") == D.load()[name]["input_sha256"], name


def test_tiny(gpu, oracle_mod):
    w = W.workload("tiny")
    x = w.xyz
    c, cx = gpu.furthest_point_sample(dev(x), w.fps_m, w.fps_start, return_xyz=True)
    check_fps(c, oracle_mod, w, "tiny fps")
    centres = gather(x, host(c))
    for grid in (True, False):
        d, i = gpu.knn(cx, dev(x), w.knn_k, grid=grid)
        D.assert_matches(host(i), host(d), D.entry("tiny", "knn"), f"tiny knn grid={grid}",
                         knn_rows(oracle_mod, centres, x, w.knn_k))
        d2, j = gpu.ball_query(cx, dev(x), w.bq_radius, w.bq_k, cull=grid)
        D.assert_matches(host(j), host(d2), D.entry("tiny", "bq"), f"tiny bq cull={grid}",
                         bq_rows(oracle_mod, centres, x, w.bq_radius, w.bq_k))
    # and directly against the oracle
    wd, wi = oracle_mod.knn(centres, x, w.knn_k)
    assert_idx_equal(host(i), wi, "tiny knn")
    assert_dist_close(host(d), wd, "tiny knn")


def test_grouping(gpu, oracle_mod):
    w = W.workload("grouping")
    x = w.xyz
    c, cx = gpu.furthest_point_sample(dev(x), w.fps_m, w.fps_start, return_xyz=True)
    check_fps(c, oracle_mod, w, "grouping fps")
    centres = gather(x, host(c))
    for grid in (True, False):
        d, i = gpu.knn(cx, dev(x), w.knn_k, grid=grid)
        D.assert_matches(host(i), host(d), D.entry("grouping", "knn"), f"grouping knn grid={grid}",
                         knn_rows(oracle_mod, centres, x, w.knn_k))


def test_large(gpu, oracle_mod):
    w = W.workload("large")
    x = w.xyz
    xd = dev(x)
    c = gpu.furthest_point_sample(xd, w.fps_m, w.fps_start)
    check_fps(c, oracle_mod, w, "large fps")
    # direct: FPS in full (2 s of CPU)
    assert_idx_equal(host(c), oracle_mod.fps(x, w.fps_m, w.fps_start), "large fps (oracle)")
    for grid in (True, False):
        d, i = gpu.knn(xd, xd, w.knn_k, grid=grid)
        D.assert_matches(host(i), host(d), D.entry("large", "knn"), f"large knn grid={grid}",
                         knn_rows(oracle_mod, x, x, w.knn_k))
    # direct: sampled rows of the last call
    d, i = host(d), host(i)
    for lo in (0, 49_872, 99_744):
        wd, wi = oracle_mod.knn(x, x, w.knn_k, rows=(lo, lo + 256), threads=THREADS)
        assert_idx_equal(i[:, lo:lo + 256], wi[:, lo:lo + 256], f"large knn rows {lo}")
        assert_dist_close(d[:, lo:lo + 256], wd[:, lo:lo + 256], f"large knn rows {lo}")


def test_sorted_bq(gpu, oracle_mod):
    w = W.workload("sorted_bq")
    x = w.xyz
    xd = dev(x)
    # direct: the whole output against the oracle (seconds on the host's threads)
    wd2, wi = oracle_mod.ball_query(x, x, w.bq_radius, w.bq_k, threads=THREADS)
    for cull in (True, False):
        d2, i = gpu.ball_query(xd, xd, w.bq_radius, w.bq_k, cull=cull)
        d2, i = host(d2), host(i)
        D.assert_matches(i, d2, D.entry("sorted_bq", "bq"), f"sorted bq cull={cull}",
                         bq_rows(oracle_mod, x, x, w.bq_radius, w.bq_k))
        assert_idx_equal(i, wi, f"sorted bq cull={cull} (oracle)")
        assert_dist_close(d2, wd2, f"sorted bq cull={cull} (oracle)")


def test_stress(gpu, oracle_mod):
    w = W.workload("stress")
    x = w.xyz
    xd = dev(x)
    c, cx = gpu.furthest_point_sample(xd, w.fps_m, w.fps_start, return_xyz=True)
    check_fps(c, oracle_mod, w, "stress fps")
    prefix = 2048     # direct: the first outputs of FPS do not depend on how many follow
    assert_idx_equal(host(c)[:, :prefix], oracle_mod.fps(x, prefix, w.fps_start),
                     "stress fps prefix (oracle)")
    centres = gather(x, host(c))
    for cull in (True, False):
        d2, i = gpu.ball_query(cx, xd, w.bq_radius, w.bq_k, cull=cull)
        D.assert_matches(host(i), host(d2), D.entry("stress", "bq"), f"stress bq cull={cull}",
                         bq_rows(oracle_mod, centres, x, w.bq_radius, w.bq_k))


def test_bench_schedule(gpu, oracle_mod):
    """The benchmark's step as it runs there: FPS of the 100k cloud on one
    stream, kNN (grid) and then Ball Query (culled) on a second stream beside
    it, three times back to back; every repetition's whole outputs match."""
    large, sbq = W.workload("large"), W.workload("sorted_bq")
    x3, x4 = dev(large.xyz), dev(sbq.xyz)
    ws = torch.empty(gpu.fps_workspace_bytes(1, 100000, large.fps_m), dtype=torch.uint8,
                     device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        c = gpu.furthest_point_sample(x3, large.fps_m, 0, workspace=ws, check=False)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            d, i = gpu.knn(x3, x3, large.knn_k)
            d2, j = gpu.ball_query(x4, x4, sbq.bq_radius, sbq.bq_k)
        outs.append((c, d, i, d2, j))
    torch.cuda.synchronize()
    gpu.fps_status(ws)
    for rep, (c, d, i, d2, j) in enumerate(outs):
        check_fps(c, oracle_mod, large, f"schedule {rep} fps")
        D.assert_matches(host(i), host(d), D.entry("large", "knn"), f"schedule {rep} knn",
                         knn_rows(oracle_mod, large.xyz, large.xyz, large.knn_k))
        D.assert_matches(host(j), host(d2), D.entry("sorted_bq", "bq"), f"schedule {rep} bq",
                         bq_rows(oracle_mod, sbq.xyz, sbq.xyz, sbq.bq_radius, sbq.bq_k))
