"""Pins of the oracle's ragged-batch composition (CPU only).

The ragged oracle hands each cloud to the dense routines; what it adds (the
segment bookkeeping, the index offset, the padding of missing neighbours) is
pinned here against the flat example of the project page (results derived by
hand, tests/golden/flat_example.json), against an independent float64 brute
force over the whole flat array on integer clouds (exact arithmetic, many
ties), and against the dense batched call on equal-size clouds."""
import json
import os

import numpy as np
import pytest

from point_cloud_neighbor_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_flat_example(oracle_mod):
    with open(os.path.join(GOLDEN, "flat_example.json")) as f:
        g = json.load(f)
    x = np.array(g["x"], dtype=np.float32)
    y = np.array(g["y"], dtype=np.float32)
    px, py = np.array(g["ptr_x"]), np.array(g["ptr_y"])
    d = g["derived"]
    counts = np.array(d["fps_counts"])
    out_ptr = np.concatenate([[0], np.cumsum(counts)])
    c = oracle_mod.fps_ragged(x, px[:-1], np.diff(px), out_ptr[:-1], counts, int(out_ptr[-1]))
    assert c.tolist() == d["fps_idx"]
    dist, idx = oracle_mod.knn_ragged(y, py[:-1], np.diff(py), x, px[:-1], np.diff(px),
                                      d["knn_k"])
    assert idx.tolist() == d["knn_idx"]
    assert dist.tolist() == [[float(v) for v in row] for row in d["knn_dist"]]
    d2, bi = oracle_mod.ball_query_ragged(y, py[:-1], np.diff(py), x, px[:-1], np.diff(px),
                                          d["bq_radius"], d["bq_K"])
    assert bi.tolist() == d["bq_idx"]
    assert d2.tolist() == d["bq_dist2"]


def ragged_integer(seed, sizes, hi=4):
    rng = np.random.default_rng(seed)
    xyz = rng.integers(0, hi, size=(int(np.sum(sizes)), 3)).astype(np.float32)
    ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    return xyz, ptr


def brute(query, qptr, ref, rptr, k, r2, K):
    """Whole-array brute force: every query row against the reference rows of
    its own cloud, in float64 (exact here), indices as flat rows."""
    rows = len(query)
    kidx = np.full((rows, k), -1, dtype=np.int64)
    kd = np.full((rows, k), np.inf)
    bidx = np.full((rows, K), -1, dtype=np.int64)
    bd = np.zeros((rows, K))
    cloud_of = np.searchsorted(qptr, np.arange(rows), side="right") - 1
    for r in range(rows):
        b = cloud_of[r]
        js = np.arange(rptr[b], rptr[b + 1])
        s = ((ref[js].astype(np.float64) - query[r].astype(np.float64)) ** 2).sum(-1)
        order = js[np.lexsort((js, s))][:k]
        kidx[r, :len(order)] = order
        kd[r, :len(order)] = np.sqrt(s[order - rptr[b]])
        hit = js[s < r2][:K]
        bidx[r, :len(hit)] = hit
        bd[r, :len(hit)] = s[hit - rptr[b]]
    return kd, kidx, bd, bidx


@pytest.mark.parametrize("sizes", [[5, 0, 17, 1, 40], [64, 65, 3], [0, 0, 9]])
def test_search_matches_flat_brute_force(oracle_mod, sizes):
    x, px = ragged_integer(1, sizes)
    qsizes = [max(0, n // 2 + (i % 2)) for i, n in enumerate(sizes)]
    y, py = ragged_integer(2, qsizes)
    k, radius, K = 6, 1.5, 7               # R2 = 2.25 exactly
    kd, ki, bd, bi = brute(y, py, x, px, k, 2.25, K)
    d, i = oracle_mod.knn_ragged(y, py[:-1], np.diff(py), x, px[:-1], np.diff(px), k)
    assert np.array_equal(i, ki)
    assert np.array_equal(d.astype(np.float64), kd.astype(np.float32).astype(np.float64))
    d2, j = oracle_mod.ball_query_ragged(y, py[:-1], np.diff(py), x, px[:-1], np.diff(px),
                                         radius, K)
    assert np.array_equal(j, bi)
    assert np.array_equal(d2.astype(np.float64), bd)
    # local indices: the same minus each cloud's offset
    _, il = oracle_mod.knn_ragged(y, py[:-1], np.diff(py), x, px[:-1], np.diff(px), k,
                                  global_index=False)
    cloud_of = np.searchsorted(py, np.arange(len(y)), side="right") - 1
    assert np.array_equal(il, np.where(ki >= 0, ki - px[cloud_of][:, None], -1))


def test_fps_matches_flat_brute_force(oracle_mod):
    sizes = [30, 1, 12, 45]
    x, px = ragged_integer(3, sizes, hi=6)
    counts = np.array([7, 3, 12, 20])      # the 1-point cloud repeats its only point
    starts = np.array([4, 0, 11, 0])
    optr = np.concatenate([[0], np.cumsum(counts)])
    got = oracle_mod.fps_ragged(x, px[:-1], np.diff(px), optr[:-1], counts, int(optr[-1]),
                                start=starts)
    want = []
    for b in range(len(sizes)):
        pts = x[px[b]:px[b + 1]].astype(np.float64)
        s = ((pts[:, None] - pts[None]) ** 2).sum(-1)
        chosen = [int(starts[b])]
        for _ in range(1, counts[b]):
            m = s[:, chosen].min(axis=1)
            chosen.append(int(np.argmax(m)))
        want += [px[b] + c for c in chosen]
    assert got.tolist() == want


def test_equal_sizes_match_dense_batch(oracle_mod):
    B, N, Q = 3, 200, 50
    x = W.uniform_cube(4, B, N)
    q = W.uniform_cube(5, B, Q)
    px = np.arange(B + 1) * N
    pq = np.arange(B + 1) * Q
    flat_x, flat_q = x.reshape(-1, 3), q.reshape(-1, 3)
    d, i = oracle_mod.knn_ragged(flat_q, pq[:-1], np.diff(pq), flat_x, px[:-1], np.diff(px), 9,
                                 global_index=False)
    wd, wi = oracle_mod.knn(q, x, 9)
    assert np.array_equal(i, wi.reshape(-1, 9)) and np.array_equal(d, wd.reshape(-1, 9))
    d2, j = oracle_mod.ball_query_ragged(flat_q, pq[:-1], np.diff(pq), flat_x, px[:-1],
                                         np.diff(px), 0.2, 12, global_index=False)
    wd2, wj = oracle_mod.ball_query(q, x, 0.2, 12)
    assert np.array_equal(j, wj.reshape(-1, 12)) and np.array_equal(d2, wd2.reshape(-1, 12))
    M = 33
    c = oracle_mod.fps_ragged(flat_x, px[:-1], np.diff(px), np.arange(B) * M, np.full(B, M),
                              B * M, global_index=False)
    assert np.array_equal(c, oracle_mod.fps(x, M).reshape(-1))


def test_padded_lengths_form(oracle_mod):
    """Padded clouds with lengths are segments (b * n_max, length_b): the same
    results as the packed clouds, with local indices."""
    sizes = np.array([13, 40, 2])
    n_max = 40
    x, px = ragged_integer(6, sizes)
    padded = np.full((len(sizes) * n_max, 3), 99.0, dtype=np.float32)
    for b in range(len(sizes)):
        padded[b * n_max:b * n_max + sizes[b]] = x[px[b]:px[b + 1]]
    offs = np.arange(len(sizes)) * n_max
    d1, i1 = oracle_mod.knn_ragged(padded, offs, sizes, padded, offs, sizes, 5,
                                   global_index=False)
    d2, i2 = oracle_mod.knn_ragged(x, px[:-1], sizes, x, px[:-1], sizes, 5, global_index=False)
    for b in range(len(sizes)):
        rows1 = slice(b * n_max, b * n_max + sizes[b])
        rows2 = slice(px[b], px[b + 1])
        assert np.array_equal(i1[rows1], i2[rows2]) and np.array_equal(d1[rows1], d2[rows2])
    # rows outside every segment are not written
    assert np.all(i1[13:40] == -2)
