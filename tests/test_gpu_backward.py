"""Ball Query backward on the GPU versus the float64 oracle.

The oracle's gradients are exact sums of exactly computed terms (float64 holds
2 G (q - x) of float32 operands without rounding error for the magnitudes used
here, up to one rounding per addition); the GPU forms each term in float32
(two roundings) and adds the terms of one output in some order, so the bar per
component is

    |gpu - oracle| <= (n + 4) * 2^-23 * sum of |terms|

with n the number of terms of that output (slots of the query row, or uses of
the reference). On clouds with small integer coordinates and dyadic G every
term and partial sum is exact in float32, so there the results must be
bit-identical. All calls go through the C ABI (via the thin Python binding)."""
import numpy as np
import pytest
import torch

from point_cloud_neighbor_amd import workloads as W
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def grad_bound(abs_sum, n):
    return (np.asarray(n, dtype=np.float64)[..., None] + 4.0) * 2.0**-23 * abs_sum


def uses_per_ref(idx, P):
    B = idx.shape[0]
    out = np.zeros((B, P), dtype=np.int64)
    for b in range(B):
        j = idx[b].ravel()
        j = j[(j >= 0) & (j < P)]
        out[b] = np.bincount(j, minlength=P)
    return out


def check_backward(gpu, oracle_mod, q, x, idx, g, what, exact=False, same=False):
    """same: q is x, passed as one device tensor (the self-query mode, whose
    reference sums go through per-tile windows in a workspace)."""
    if same:
        xd = dev(x)
        gq, gx = gpu.ball_query_backward(xd, xd, dev(idx), dev(g))
    else:
        gq, gx = gpu.ball_query_backward(dev(q), dev(x), dev(idx), dev(g))
    gq, gx = host(gq), host(gx)
    clean = np.where((idx >= 0) & (idx < x.shape[1]), idx, -1)
    wq, wx, aq, ax = oracle_mod.ball_query_backward(q, x, clean, g)
    if exact:
        assert np.array_equal(gq.astype(np.float64), wq), f"{what}: grad_query not exact"
        assert np.array_equal(gx.astype(np.float64), wx), f"{what}: grad_ref not exact"
        return gq, gx
    nq = (clean >= 0).sum(-1)
    nx = uses_per_ref(clean, x.shape[1])
    for name, got, want, bound in (("grad_query", gq, wq, grad_bound(aq, nq)),
                                   ("grad_ref", gx, wx, grad_bound(ax, nx))):
        err = np.abs(got.astype(np.float64) - want)
        bad = ~(err <= bound)
        assert not bad.any(), (f"{what} {name}: {int(bad.sum())} outside the bound, first "
                               f"at {np.argwhere(bad)[0]}")
    return gq, gx


def seeded_grad(seed, shape, dyadic=False):
    rng = np.random.default_rng(seed)
    if dyadic:
        return (rng.integers(-8, 9, size=shape) / 4.0).astype(np.float32)
    return rng.standard_normal(shape).astype(np.float32)


@pytest.mark.parametrize("B,Q,P,K,r", [(1, 1, 1, 1, 0.5), (2, 37, 300, 16, 0.2),
                                       (3, 129, 1000, 64, 0.15), (1, 200, 2049, 65, 0.3),
                                       (2, 65, 513, 130, 0.5)])
def test_backward_shapes(gpu, oracle_mod, B, Q, P, K, r):
    x = W.uniform_cube(11 + P, B, P)
    q = W.uniform_cube(12 + Q, B, Q)
    _, idx = oracle_mod.ball_query(q, x, r, K, threads=8)
    g = seeded_grad(Q * P, idx.shape)
    check_backward(gpu, oracle_mod, q, x, idx, g, f"B={B} Q={Q} P={P} K={K}")


def test_backward_exact_on_integer_cloud(gpu, oracle_mod):
    x = W.integer_cloud(3, 2, 700, 0, 4)
    q = x[:, ::3].copy()
    _, idx = oracle_mod.ball_query(q, x, 1.5, 48, threads=8)
    assert (idx >= 0).sum() > 1000
    g = seeded_grad(5, idx.shape, dyadic=True)
    check_backward(gpu, oracle_mod, q, x, idx, g, "integer", exact=True)


def test_backward_sorted_workload_subset(gpu, oracle_mod):
    """The sorted Ball Query cloud (100k references, K = 64) with its first
    8192 points as queries: in Morton order neighbouring queries share their
    references, so grad_ref adds tens of terms per point in atomic order."""
    wl = W.workload("sorted_bq")
    x = wl.xyz
    q = x[:, :8192].copy()
    _, idx = oracle_mod.ball_query(q, x, wl.bq_radius, wl.bq_k, threads=8)
    g = seeded_grad(7, idx.shape)
    check_backward(gpu, oracle_mod, q, x, idx, g, "sorted_bq subset")


@pytest.mark.parametrize("same", [False, True])
def test_backward_sorted_workload_whole_output(gpu, oracle_mod, same):
    """Full size as the benchmark runs it (every point of the sorted cloud a
    query): both gradients of every row and every reference against the
    oracle. Neighbouring rows select neighbouring references here, so most
    reference terms go through the per-tile window, the others through the
    table; with one tensor for both sets (as the benchmark passes it), the
    windows are the fixed ones of the self-query mode."""
    wl = W.workload("sorted_bq")
    x = wl.xyz
    _, idx = oracle_mod.ball_query(x, x, wl.bq_radius, wl.bq_k, threads=8)
    g = seeded_grad(9, idx.shape)
    check_backward(gpu, oracle_mod, x, x, idx, g, f"sorted_bq whole same={same}", same=same)


@pytest.mark.parametrize("tile", ["4", "37", "1024"])
def test_backward_tile_sizes(gpu, oracle_mod, monkeypatch, tile):
    """Rows per workgroup forced to the extremes (and an odd size) on a sorted
    self-query, where the window and the table both take terms."""
    monkeypatch.setenv("POINTOPS_BQ_BWD_TILE", tile)
    wl = W.workload("sorted_bq")
    x = wl.xyz[:, :20000].copy()
    _, idx = oracle_mod.ball_query(x, x, 0.08, 64, threads=8)
    g = seeded_grad(10, idx.shape)
    check_backward(gpu, oracle_mod, x, x, idx, g, f"tile {tile}")


@pytest.mark.parametrize("tile", [None, "4", "37", "1024"])
def test_backward_self_query_mode(gpu, oracle_mod, monkeypatch, tile):
    """One tensor as query and reference set: the window partials in the
    workspace and their merge, against the oracle, on a sorted cloud (most
    terms in the windows), with forced tile sizes."""
    if tile:
        monkeypatch.setenv("POINTOPS_BQ_BWD_TILE", tile)
    wl = W.workload("sorted_bq")
    x = wl.xyz[:, :30000].copy()
    _, idx = oracle_mod.ball_query(x, x, 0.07, 64, threads=8)
    g = seeded_grad(11, idx.shape)
    check_backward(gpu, oracle_mod, x, x, idx, g, f"self tile {tile}", same=True)


def test_backward_self_query_unsorted_and_batched(gpu, oracle_mod):
    """Self-query on clouds in random order (few terms in the windows, most
    through the table) and on two clouds, whose tiles straddle the boundary
    between them; K above 64 (two passes per row) on the second."""
    x = W.uniform_cube(71, 2, 6000)
    _, idx = oracle_mod.ball_query(x, x, 0.12, 48, threads=8)
    g = seeded_grad(12, idx.shape)
    check_backward(gpu, oracle_mod, x, x, idx, g, "self unsorted B=2", same=True)
    wl = W.workload("sorted_bq")
    x = np.concatenate([wl.xyz[:, :5000], wl.xyz[:, 5000:10000]], axis=0).copy()
    _, idx = oracle_mod.ball_query(x, x, 0.12, 100, threads=8)
    g = seeded_grad(13, idx.shape)
    check_backward(gpu, oracle_mod, x, x, idx, g, "self sorted B=2 K=100", same=True)


def test_backward_self_query_exact(gpu, oracle_mod):
    """Self-query on a small-integer cloud with dyadic G: every sum is exact,
    so both gradients must equal the oracle's bit for bit."""
    x = W.integer_cloud(3, 2, 900, 0, 4)
    _, idx = oracle_mod.ball_query(x, x, 1.5, 48, threads=8)
    g = seeded_grad(14, idx.shape, dyadic=True)
    check_backward(gpu, oracle_mod, x, x, idx, g, "self integer", exact=True, same=True)


@pytest.mark.parametrize("same,K,B", [(True, 64, 1), (False, 64, 1), (True, 64, 2),
                                      (False, 130, 1)])
def test_backward_contended_exact(gpu, oracle_mod, same, K, B):
    """Every row selects the same K references (4096 points on {0, 1}^3, a
    radius that holds them all), so each of those references takes 4096 terms
    per cloud: in the first tile through its window, in every other tile
    through the hash table, with many lanes and waves adding into one word at
    once. The terms and sums are dyadic, exact in float32 in any order, so
    both gradients must equal the oracle's bit for bit."""
    x = W.integer_cloud(21, B, 4096, 0, 2)
    _, idx = oracle_mod.ball_query(x, x, 2.0, K, threads=8)
    assert (idx[:, :, :K] == np.arange(K)).all()
    g = seeded_grad(22, idx.shape, dyadic=True)
    check_backward(gpu, oracle_mod, x, x, idx, g, f"contended same={same} K={K} B={B}",
                   exact=True, same=same)


def test_backward_sorted_workload_full(gpu, oracle_mod):
    """Full size (every point a query, as the benchmark runs it): grad_query
    on sampled row blocks against the oracle (a row's gradient depends only on
    that row), and for grad_ref the translation invariance of s: the query and
    reference gradients of all rows sum to zero, up to rounding."""
    wl = W.workload("sorted_bq")
    x = wl.xyz
    N = x.shape[1]
    xd = dev(x)
    d2, idx = gpu.ball_query(xd, xd, wl.bq_radius, wl.bq_k)
    g = seeded_grad(8, tuple(d2.shape))
    gq, gx = gpu.ball_query_backward(xd, xd, idx, dev(g))
    gq, gx = host(gq).astype(np.float64), host(gx).astype(np.float64)
    for lo, hi in [(0, 512), (N // 3, N // 3 + 512), (N - 512, N)]:
        _, oi = oracle_mod.ball_query(x, x, wl.bq_radius, wl.bq_k, rows=(lo, hi), threads=8)
        oi = oi[:, lo:hi]
        wq, _, aq, _ = oracle_mod.ball_query_backward(x[:, lo:hi], x, oi, g[:, lo:hi])
        err = np.abs(gq[:, lo:hi] - wq)
        assert np.all(err <= grad_bound(aq, (oi >= 0).sum(-1))), f"rows {lo}:{hi}"
    # every output carries at most (n + 4) 2^-23 of its terms' absolute sum;
    # each term appears once on each side, so 2 (n_max + 4) 2^-23 A bounds the
    # total, with A the sum of all |terms| (plus float64 summation, negligible)
    i = host(idx)[0]
    sel = i >= 0
    rows = np.nonzero(sel)[0]
    t = 2.0 * g[0][sel].astype(np.float64)[:, None] * (
        x[0][rows].astype(np.float64) - x[0][i[sel]].astype(np.float64))
    A = np.abs(t).sum(axis=0)
    n_max = max(int(sel.sum(-1).max()), int(np.bincount(i[sel], minlength=N).max()))
    total = gq.sum(axis=(0, 1)) + gx.sum(axis=(0, 1))
    assert np.all(np.abs(total) <= 2 * (n_max + 4) * 2.0**-23 * A), (total, A, n_max)


def test_backward_query_sum_is_deterministic(gpu, oracle_mod):
    x = W.uniform_cube(21, 2, 3000)
    q = W.uniform_cube(22, 2, 500)
    _, idx = oracle_mod.ball_query(q, x, 0.3, 100, threads=8)
    g = seeded_grad(23, idx.shape)
    a, _ = gpu.ball_query_backward(dev(q), dev(x), dev(idx), dev(g))
    b, _ = gpu.ball_query_backward(dev(q), dev(x), dev(idx), dev(g))
    assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32))


def test_backward_skips_padding_and_out_of_range(gpu, oracle_mod):
    rng = np.random.default_rng(31)
    B, Q, P, K = 2, 50, 40, 12
    q = W.uniform_cube(32, B, Q)
    x = W.uniform_cube(33, B, P)
    idx = rng.integers(-3, P + 3, size=(B, Q, K)).astype(np.int64)
    idx[0, 0] = -1                       # a row of padding only
    g = seeded_grad(34, idx.shape)
    gq, _ = check_backward(gpu, oracle_mod, q, x, idx, g, "random indices")
    assert np.all(gq[0, 0] == 0.0)


def test_backward_optional_outputs(gpu, oracle_mod):
    x = W.uniform_cube(41, 1, 800)
    q = W.uniform_cube(42, 1, 90)
    _, idx = oracle_mod.ball_query(q, x, 0.25, 32, threads=8)
    g = seeded_grad(43, idx.shape)
    full_q, full_x = gpu.ball_query_backward(dev(q), dev(x), dev(idx), dev(g))
    only_q, none_x = gpu.ball_query_backward(dev(q), dev(x), dev(idx), dev(g), need_ref=False)
    none_q, only_x = gpu.ball_query_backward(dev(q), dev(x), dev(idx), dev(g), need_query=False)
    assert none_x is None and none_q is None
    assert np.array_equal(host(only_q), host(full_q))
    np.testing.assert_allclose(host(only_x), host(full_x), rtol=1e-5, atol=1e-6)


def test_backward_overwrites_grad_ref(gpu, oracle_mod):
    """grad_ref is cleared by the call itself: garbage in the output buffer on
    entry must not leak into the result."""
    from point_cloud_neighbor_amd import ops
    lib = ops._load()
    x = W.integer_cloud(51, 1, 300, 0, 4)
    q = x[:, :64].copy()
    _, idx = oracle_mod.ball_query(q, x, 1.5, 16, threads=8)
    g = seeded_grad(52, idx.shape, dyadic=True)
    tq, tx, ti, tg = dev(q), dev(x), dev(idx), dev(g)
    gq = torch.full_like(tq, float("nan"))
    gx = torch.full_like(tx, 12345.0)
    rc = lib.pointops_ball_query_backward(tq.data_ptr(), tx.data_ptr(), ti.data_ptr(),
                                          tg.data_ptr(), 1, 64, 300, 16, gq.data_ptr(),
                                          gx.data_ptr(), None, 0, None)
    assert rc == 0
    torch.cuda.synchronize()
    wq, wx, _, _ = oracle_mod.ball_query_backward(q, x, idx, g)
    assert np.array_equal(host(gq).astype(np.float64), wq)
    assert np.array_equal(host(gx).astype(np.float64), wx)


def test_autograd_through_ball_query(gpu, oracle_mod):
    xn = W.uniform_cube(61, 2, 1500)
    qn = W.uniform_cube(62, 2, 300)
    x = dev(xn).requires_grad_(True)
    q = dev(qn).requires_grad_(True)
    d2, idx = gpu.ball_query(q, x, 0.2, 24)
    assert d2.requires_grad and not idx.requires_grad
    g = seeded_grad(63, tuple(d2.shape))
    (d2 * dev(g)).sum().backward()
    wq, wx, aq, ax = oracle_mod.ball_query_backward(qn, xn, host(idx), g)
    i = host(idx)
    for got, want, bound in ((host(q.grad), wq, grad_bound(aq, (i >= 0).sum(-1))),
                             (host(x.grad), wx, grad_bound(ax, uses_per_ref(i, 1500)))):
        assert np.all(np.abs(got.astype(np.float64) - want) <= bound)
    # no grad requested: the plain forward, same outputs
    with torch.no_grad():
        d2b, idxb = gpu.ball_query(q, x, 0.2, 24)
    assert torch.equal(d2b, d2.detach()) and torch.equal(idxb, idx)


def test_autograd_self_query(gpu, oracle_mod):
    """query and ref the same tensor: both gradient paths land in one .grad."""
    xn = W.integer_cloud(71, 1, 400, 0, 4)
    x = dev(xn).requires_grad_(True)
    d2, idx = gpu.ball_query(x, x, 1.5, 20)
    g = seeded_grad(72, tuple(d2.shape), dyadic=True)
    (d2 * dev(g)).sum().backward()
    wq, wx, _, _ = oracle_mod.ball_query_backward(xn, xn, host(idx), g)
    assert np.array_equal(host(x.grad).astype(np.float64), wq + wx)


def test_backward_rejects_bad_arguments(gpu):
    from point_cloud_neighbor_amd import ops
    q = torch.zeros((1, 4, 3), device="cuda")
    x = torch.zeros((1, 5, 3), device="cuda")
    idx = torch.zeros((1, 4, 2), dtype=torch.int64, device="cuda")
    g = torch.zeros((1, 4, 2), device="cuda")
    with pytest.raises(ops.PointopsError):
        ops.ball_query_backward(q, x, idx.int(), g)
    with pytest.raises(ops.PointopsError):
        ops.ball_query_backward(q, x, idx, g[..., :1])
    with pytest.raises(ops.PointopsError):
        ops.ball_query_backward(q, x, idx[..., :0], g[..., :0])
    lib = ops._load()
    assert lib.pointops_ball_query_backward(q.data_ptr(), x.data_ptr(), idx.data_ptr(),
                                            g.data_ptr(), -1, 4, 5, 2, q.data_ptr(), None,
                                            None, 0, None) == 1
    # the self-query workspace, when given, must be large enough
    assert lib.pointops_ball_query_backward(x.data_ptr(), x.data_ptr(), idx.data_ptr(),
                                            g.data_ptr(), 1, 5, 5, 2, None, x.data_ptr(),
                                            x.data_ptr(), 8, None) == 1
