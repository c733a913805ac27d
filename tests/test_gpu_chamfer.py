"""three_nn and the Chamfer distance on the GPU versus the oracle: nearest
points and indices bit-exact; the loss within one float32 rounding of the
oracle's float64 value; gradients within (n + 5) 2^-23 of their terms'
absolute sum (n terms per output, three roundings per term). All calls go
through the C ABI (via the thin Python binding)."""
import json
import os

import numpy as np
import pytest
import torch

from point_cloud_neighbor_amd import workloads as W
from tests.gpu_util import assert_dist_close, assert_idx_equal, dev, host

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_v050_example(gpu):
    with open(os.path.join(GOLDEN, "v050_example.json")) as f:
        g = json.load(f)
    xyz = dev(np.array(g["xyz"], dtype=np.float32))
    d = g["derived"]
    dist, idx = gpu.three_nn(xyz[:, :2].contiguous(), xyz)
    assert host(idx).tolist() == d["three_nn_idx"]
    assert np.array_equal(host(dist), np.sqrt(np.array(d["three_nn_dist2"], dtype=np.float32)))
    loss, _ = gpu.chamfer_distance(xyz[:, :2].contiguous(), xyz)
    assert loss.item() == float(np.float32(1 / 3))


@pytest.mark.parametrize("B,n,m", [(1, 1, 3), (2, 100, 3), (3, 700, 257), (2, 4097, 1000)])
def test_three_nn(gpu, oracle_mod, B, n, m):
    u = W.uniform_cube(n + m, B, n)
    k = W.uniform_cube(n + m + 1, B, m)
    d, i = gpu.three_nn(dev(u), dev(k))
    wd, wi = oracle_mod.three_nn(u, k, threads=8)
    assert_idx_equal(host(i), wi, "three_nn idx")
    assert_dist_close(host(d), wd, "three_nn dist")


def check_chamfer(gpu, oracle_mod, x, y, xl=None, yl=None, pr="mean", br="mean", single=False,
                  what=""):
    loss, d_xy, i_xy, d_yx, i_yx = gpu.chamfer_nearest(dev(x), dev(y), xl, yl, pr, br, single)
    wl, ws_xy, wi_xy, ws_yx, wi_yx = oracle_mod.chamfer(x, y, xl, yl, pr, br, single, threads=8)
    assert_idx_equal(host(i_xy), wi_xy, f"nearest x->y {what}")
    assert_dist_close(host(d_xy), ws_xy, f"nearest x->y {what}")
    if not single:
        assert_idx_equal(host(i_yx), wi_yx, f"nearest y->x {what}")
        assert_dist_close(host(d_yx), ws_yx, f"nearest y->x {what}")
    got = host(loss).astype(np.float64)
    want = np.atleast_1d(wl)
    assert got.shape == want.shape
    assert np.all(np.abs(got - want) <= 2.0**-23 * np.abs(want)), (what, got, want)
    return loss, i_xy, i_yx


@pytest.mark.parametrize("pr", ["mean", "sum"])
@pytest.mark.parametrize("br", ["mean", "sum", None])
@pytest.mark.parametrize("single", [False, True])
def test_chamfer_reductions(gpu, oracle_mod, pr, br, single):
    x = W.uniform_cube(1, 3, 600)
    y = W.uniform_cube(2, 3, 450)
    check_chamfer(gpu, oracle_mod, x, y, pr=pr, br=br, single=single, what=f"{pr} {br} {single}")


@pytest.mark.parametrize("xl,yl", [([600, 1, 0], [450, 450, 17]), (None, [3, 0, 450]),
                                   ([5, 64, 65], None)])
def test_chamfer_lengths(gpu, oracle_mod, xl, yl):
    x = W.uniform_cube(3, 3, 600)
    y = W.uniform_cube(4, 3, 450)
    for br in ("mean", None):
        check_chamfer(gpu, oracle_mod, x, y, xl, yl, "mean", br, what=f"lengths {xl} {yl}")


def test_chamfer_ties_integer(gpu, oracle_mod):
    x = W.integer_cloud(5, 2, 3000, 0, 5)
    y = W.integer_cloud(6, 2, 2000, 0, 5)
    check_chamfer(gpu, oracle_mod, x, y, what="integer")


def grad_bound(abs_sum, n):
    return (np.asarray(n, dtype=np.float64)[..., None] + 5.0) * 2.0**-23 * abs_sum


def uses(idx, n_other, own_len=None):
    B = idx.shape[0]
    out = np.zeros((B, n_other), dtype=np.int64)
    for b in range(B):
        j = idx[b][: (idx.shape[1] if own_len is None else own_len[b])]
        j = j[j >= 0]
        out[b] = np.bincount(j, minlength=n_other)
    return out


@pytest.mark.parametrize("pr,br,single,xl,yl", [
    ("mean", "mean", False, None, None), ("sum", "sum", False, None, None),
    ("mean", None, True, None, None), ("mean", "mean", False, [300, 0, 77], [450, 9, 0])])
def test_chamfer_backward(gpu, oracle_mod, pr, br, single, xl, yl):
    x = W.uniform_cube(7, 3, 300)
    y = W.uniform_cube(8, 3, 450)
    _, i_xy, i_yx = check_chamfer(gpu, oracle_mod, x, y, xl, yl, pr, br, single)
    i_xy_h = host(i_xy)
    i_yx_h = host(i_yx) if i_yx is not None else None
    g = np.array([0.7, -1.3, 2.1], dtype=np.float32) if br is None else np.float32(1.7)
    gx, gy = gpu.chamfer_backward(dev(x), dev(y), i_xy, i_yx, torch.tensor(g).reshape(-1),
                                  xl, yl, pr, br, single)
    wx, wy, ax, ay = oracle_mod.chamfer_backward(x, y, i_xy_h, i_yx_h, g, xl, yl, pr, br, single)
    lx = np.full(3, 300) if xl is None else np.array(xl)
    ly = np.full(3, 450) if yl is None else np.array(yl)
    nx = 1 + (0 if single else uses(i_yx_h, 300, ly))
    ny = (0 if single else 1) + uses(i_xy_h, 450, lx)
    for name, got, want, bound in (("grad_x", host(gx), wx, grad_bound(ax, nx)),
                                   ("grad_y", host(gy), wy, grad_bound(ay, ny))):
        err = np.abs(got.astype(np.float64) - want)
        bad = ~(err <= bound)
        assert not bad.any(), f"{name}: {int(bad.sum())} outside, first {np.argwhere(bad)[0]}"


def test_chamfer_autograd_and_determinism(gpu, oracle_mod):
    xn, yn = W.uniform_cube(9, 2, 500), W.uniform_cube(10, 2, 800)
    x = dev(xn).requires_grad_(True)
    y = dev(yn).requires_grad_(True)
    loss, _ = gpu.chamfer_distance(x, y)
    loss.backward()
    wl, _, i_xy, _, i_yx = oracle_mod.chamfer(xn, yn)
    wx, wy, ax, ay = oracle_mod.chamfer_backward(xn, yn, i_xy, i_yx, 1.0)
    assert abs(loss.item() - wl) <= 2.0**-23 * wl
    nx = 1 + uses(i_yx, 500)
    ny = 1 + uses(i_xy, 800)
    assert np.all(np.abs(host(x.grad).astype(np.float64) - wx) <= grad_bound(ax, nx))
    assert np.all(np.abs(host(y.grad).astype(np.float64) - wy) <= grad_bound(ay, ny))
    again, _ = gpu.chamfer_distance(x.detach(), y.detach())
    assert again.item() == loss.item()


def test_chamfer_workload_size(gpu, oracle_mod):
    """The benchmark's Chamfer shape (B = 4, 16,384 points per cloud): nearest
    points on sampled rows, and the loss from the oracle's distances of all
    rows (the loss needs every row)."""
    x, y = W.uniform_cube(11, 4, 16384), W.uniform_cube(12, 4, 16384)
    loss, d_xy, i_xy, d_yx, i_yx = gpu.chamfer_nearest(dev(x), dev(y))
    for rows in [(0, 256), (4 * 16384 - 256, 4 * 16384), (30000, 30256)]:
        ws, wi = oracle_mod.nearest(x, y, rows=rows, threads=8)
        sl = (slice(None),)
        got_i, got_s = host(i_xy).reshape(-1)[rows[0]:rows[1]], host(d_xy).reshape(-1)[rows[0]:rows[1]]
        assert np.array_equal(got_i, wi.reshape(-1)[rows[0]:rows[1]])
        assert np.array_equal(got_s.view(np.uint32), ws.reshape(-1)[rows[0]:rows[1]].view(np.uint32))
    wl = oracle_mod.chamfer(x, y, threads=8)[0]
    assert abs(float(host(loss)[0]) - wl) <= 2.0**-23 * wl


def test_chamfer_invalid_arguments(gpu):
    x = dev(W.uniform_cube(13, 2, 10))
    with pytest.raises(gpu.PointopsError):
        gpu.chamfer_nearest(x, x, x_lengths=[11, 3])
    with pytest.raises(gpu.PointopsError):
        gpu.chamfer_nearest(x, x, point_reduction="max")
    with pytest.raises(gpu.PointopsError):
        gpu.three_nn(x, x[:, :2].contiguous())


@pytest.mark.parametrize("case", ["uniform", "integer"])
@pytest.mark.parametrize("lengths", [False, True])
@pytest.mark.parametrize("per_wave", ["0", "1", "2"])
def test_chamfer_and_three_nn_grid_search_forced(gpu, oracle_mod, case, lengths, per_wave,
                                                 monkeypatch):
    """The nearest points of the Chamfer distance and three_nn through the
    kNN grid search (forced on at small sizes, one query per lane or per
    wave), dense and with lengths (a cloud without y points among them),
    against the oracle."""
    monkeypatch.setenv("POINTOPS_KNN_GRID", "1")
    monkeypatch.setenv("POINTOPS_KNN_GRID_WAVE", per_wave)
    if case == "uniform":
        x, y = W.uniform_cube(21, 2, 700), W.uniform_cube(22, 2, 1300)
        xl, yl = ([700, 9], [1000, 0]) if lengths else (None, None)
    else:
        x, y = W.integer_cloud(23, 2, 900, 0, 5), W.integer_cloud(24, 2, 600, 0, 5)
        xl, yl = ([300, 900], [600, 17]) if lengths else (None, None)
    for single in (False, True):
        check_chamfer(gpu, oracle_mod, x, y, xl, yl, single=single,
                      what=f"grid {case} lengths={lengths}")
    d, i = gpu.three_nn(dev(x), dev(y))
    wd, wi = oracle_mod.three_nn(x, y, threads=8)
    assert_idx_equal(host(i), wi, "three_nn grid idx")
    assert_dist_close(host(d), wd, "three_nn grid dist")


@pytest.mark.parametrize("wave", ["0", "1"])
@pytest.mark.parametrize("lengths", [False, True])
def test_chamfer_and_three_nn_both_scans(gpu, oracle_mod, wave, lengths, monkeypatch):
    """The nearest points (and three_nn) through either full scan: one query
    per lane, or one per wave (squared distances kept), dense and with
    lengths, against the oracle."""
    monkeypatch.setenv("POINTOPS_KNN_GRID", "0")
    monkeypatch.setenv("POINTOPS_KNN_WAVE", wave)
    x, y = W.uniform_cube(25, 3, 1100), W.integer_cloud(26, 3, 700, 0, 6)
    xl, yl = ([1100, 5, 0], [700, 0, 64]) if lengths else (None, None)
    for single in (False, True):
        check_chamfer(gpu, oracle_mod, x, y, xl, yl, single=single, what=f"wave={wave}")
    d, i = gpu.three_nn(dev(x), dev(y))
    wd, wi = oracle_mod.three_nn(x, y, threads=8)
    assert_idx_equal(host(i), wi, f"three_nn wave={wave} idx")
    assert_dist_close(host(d), wd, f"three_nn wave={wave} dist")
