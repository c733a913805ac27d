"""The C ABI library loads and exports what include/pointops.h declares, and
its host-side argument checks answer before anything reaches a device.

Runs without a GPU: none of these calls launches a kernel.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pointops.h")
LIB = os.path.join(ROOT, "point_cloud_neighbor_amd", "libpointops.so")

OK, INVALID, UNSUPPORTED, UNSUPPORTED_DEVICE, HIP_ERROR, EXEC_TIMEOUT = range(6)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pointops_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from point_cloud_neighbor_amd import build
        build.build()
    lib = ctypes.CDLL(LIB)
    i64, vp, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    lib.pointops_fps.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, ctypes.c_size_t, vp]
    lib.pointops_knn.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp, ctypes.c_size_t, vp]
    lib.pointops_ball_query.argtypes = [vp, vp, i64, i64, i64, f32, i64, vp, vp, vp,
                                        ctypes.c_size_t, vp]
    lib.pointops_fps_status.argtypes = [vp, ctypes.c_size_t, vp, vp]
    lib.pointops_status_string.restype = ctypes.c_char_p
    lib.pointops_last_error.restype = ctypes.c_char_p
    return lib


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("pointops_fps", "pointops_fps_workspace_bytes", "pointops_fps_status",
                     "pointops_knn",
                     "pointops_ball_query", "pointops_device_check", "pointops_status_string",
                     "pointops_last_error", "pointops_abi_version"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in pointops.h but not exported"


def test_status_strings_and_version(lib):
    assert lib.pointops_abi_version() == 5
    for code in range(6):
        assert lib.pointops_status_string(code) != b"unknown status"
    assert lib.pointops_status_string(99) == b"unknown status"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def test_fps_status_argument_checks(lib):
    # no workspace, or too small for the status word: rejected before any HIP call
    assert lib.pointops_fps_status(None, 1 << 20, None, None) == INVALID
    assert lib.pointops_fps_status(FAKE, 7, None, None) == INVALID
    assert b"workspace" in lib.pointops_last_error()


def test_fps_argument_checks(lib):
    out = FAKE
    # start index out of range
    assert lib.pointops_fps(FAKE, 1, 10, 3, 10, out, None, FAKE, 1 << 20, None) == INVALID
    assert b"start_idx" in lib.pointops_last_error()
    assert lib.pointops_fps(FAKE, 1, 10, 3, -1, out, None, FAKE, 1 << 20, None) == INVALID
    # empty cloud with samples requested
    assert lib.pointops_fps(FAKE, 1, 0, 3, 0, out, None, FAKE, 1 << 20, None) == INVALID
    assert lib.pointops_fps(FAKE, -1, 10, 3, 0, out, None, FAKE, 1 << 20, None) == INVALID
    # no-ops: B == 0 or M == 0
    assert lib.pointops_fps(None, 0, 10, 3, 0, None, None, None, 0, None) == OK
    assert lib.pointops_fps(None, 2, 10, 0, 0, None, None, None, 0, None) == OK
    assert lib.pointops_fps(FAKE, 1, 1 << 31, 3, 0, out, None, FAKE, 1 << 20, None) == UNSUPPORTED


def test_knn_argument_checks(lib):
    assert lib.pointops_knn(FAKE, FAKE, 1, 4, 10, 11, FAKE, FAKE, None, 0, None) == INVALID  # k > P
    assert lib.pointops_knn(FAKE, FAKE, 1, 4, 10, 0, FAKE, FAKE, None, 0, None) == INVALID   # k < 1
    assert lib.pointops_knn(FAKE, FAKE, 1, 4, 100, 65, FAKE, FAKE, None, 0, None) == UNSUPPORTED
    assert b"KMAX" in lib.pointops_last_error()
    assert lib.pointops_knn(None, None, 0, 4, 10, 3, None, None, None, 0, None) == OK        # B == 0
    assert lib.pointops_knn(None, None, 2, 0, 10, 3, None, None, None, 0, None) == OK        # Q == 0
    assert lib.pointops_knn(FAKE, FAKE, 70000, 4, 10, 3, FAKE, FAKE, None, 0, None) == UNSUPPORTED


def test_ball_query_argument_checks(lib):
    for r in (0.0, -1.0, float("nan"), float("inf")):
        assert lib.pointops_ball_query(FAKE, FAKE, 1, 4, 10, r, 3, FAKE, FAKE, None, 0,
                                       None) == INVALID
    assert lib.pointops_ball_query(FAKE, FAKE, 1, 4, 10, 0.5, 0, FAKE, FAKE, None, 0,
                                   None) == INVALID
    assert lib.pointops_ball_query(None, None, 0, 4, 10, 0.5, 3, None, None, None, 0, None) == OK
    assert lib.pointops_ball_query(None, None, 3, 0, 10, 0.5, 3, None, None, None, 0, None) == OK


def test_no_gpu_means_an_error_not_a_fallback(lib):
    """Without a usable gfx950 device a well-formed call fails loudly."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; covered by the GPU tests")
    st = lib.pointops_device_check(0)
    assert st in (UNSUPPORTED_DEVICE, HIP_ERROR)
    st = lib.pointops_knn(FAKE, FAKE, 1, 4, 10, 3, FAKE, FAKE, None, 0, None)
    assert st in (UNSUPPORTED_DEVICE, HIP_ERROR)


def test_python_binding_refuses_cpu_tensors():
    import torch
    from point_cloud_neighbor_amd import ops
    x = torch.zeros(1, 8, 3)
    with pytest.raises(ops.PointopsError):
        ops.knn(x, x, 2)
    with pytest.raises(ops.PointopsError):
        ops.ball_query(x, x, 0.5, 2)
    with pytest.raises(ops.PointopsError):
        ops.furthest_point_sample(x, 2)


def test_workspace_sizes(lib):
    """Host-only size queries: the Ball Query's workspace grows by the grid
    pass's room (per query, sorted copies, histograms) above 32768 references
    and is zero for empty shapes; kNN's grid workspace starts at 8192
    references and 2^22 pairs."""
    i64 = ctypes.c_int64
    lib.pointops_ball_query_workspace_bytes.argtypes = [i64, i64, i64]
    lib.pointops_ball_query_workspace_bytes.restype = ctypes.c_size_t
    lib.pointops_knn_workspace_bytes.argtypes = [i64, i64, i64]
    lib.pointops_knn_workspace_bytes.restype = ctypes.c_size_t
    bq = lib.pointops_ball_query_workspace_bytes
    # boxes only: (blocks of 64 + runs of 64 blocks) x 32 bytes per cloud
    nblk = (30000 + 63) // 64
    assert bq(2, 10, 30000) == 2 * (nblk + (nblk + 63) // 64) * 32
    assert bq(1, 10, 32769) > bq(1, 10, 32768) + 16 * 32769   # the sorted copies alone
    assert bq(1, 2000, 40000) >= bq(1, 1000, 40000) + 1000 * (8 + 16) - 2 * 256  # alignment
    assert bq(0, 10, 100) == bq(1, 0, 100) == bq(1, 10, 0) == 0
    knn = lib.pointops_knn_workspace_bytes
    assert knn(1, 100000, 100000) > 0
    assert knn(1, 100, 8191) == 0 and knn(1, 10, 100000) == 0


def test_ragged_workspace_sizes(lib):
    """Host-only size queries of the ragged culled searches: more than the
    scan's table exactly when the search is taken (clouds of 8192 references
    or more, K <= 32 for Ball Query, padding to the largest cloud within
    eight times the points), room for every cloud's slots at the largest
    counts, and 0 for invalid counts."""
    import numpy as np
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    for f in (lib.pointops_knn_ragged_workspace_bytes,
              lib.pointops_ball_query_ragged_workspace_bytes):
        f.argtypes = [vp, vp, i64, i64]
        f.restype = ctypes.c_size_t
    lib.pointops_ragged_workspace_bytes.argtypes = [i64]
    lib.pointops_ragged_workspace_bytes.restype = ctypes.c_size_t
    table = lib.pointops_ragged_workspace_bytes

    def sizes(f, q, r, k):
        q, r = np.asarray(q, dtype=np.int64), np.asarray(r, dtype=np.int64)
        return f(q.ctypes.data, r.ctypes.data, len(q), k)

    knn, bq = lib.pointops_knn_ragged_workspace_bytes, lib.pointops_ball_query_ragged_workspace_bytes
    q, r = [6000, 3000, 200], [50000, 24000, 1600]
    for f, k in ((knn, 16), (bq, 32)):
        n = sizes(f, q, r, k)
        # sorted float4 copies of every cloud at the largest counts, at least
        assert n > table(3) + 3 * (50000 + 6000) * 16, f
    # small clouds, large K, a skewed batch: the scans' table alone
    assert sizes(knn, [100, 100], [4000, 8000], 16) == table(2)
    assert sizes(bq, [100, 100], [4000, 8000], 32) == table(2)
    assert sizes(bq, q, r, 33) == table(3)
    skew_q, skew_r = [25000] + [10] * 200, [200000] + [100] * 200
    assert sizes(knn, skew_q, skew_r, 16) == table(201)
    assert sizes(bq, skew_q, skew_r, 32) == table(201)
    # no clouds: the table's minimum; invalid counts: 0
    assert sizes(knn, [], [], 16) == table(0)
    assert sizes(knn, [-1], [10], 16) == 0 and sizes(bq, [1], [-5], 8) == 0


def test_ball_query_backward_workspace(lib):
    """The self-query workspace: one window of partials (3 planes of 2048
    floats) per tile of 128 rows at K = 64; nothing when Q != P; a call that
    would use it refuses one too small before touching the device."""
    i64 = ctypes.c_int64
    f = lib.pointops_ball_query_backward_workspace_bytes
    f.argtypes = [i64, i64, i64, i64]
    f.restype = ctypes.c_size_t
    assert f(1, 100000, 100000, 64) == 782 * 3 * 2048 * 4
    assert f(2, 1000, 1000, 64) == 16 * 3 * 2048 * 4
    assert f(1, 1000, 2000, 64) == 0
    assert f(0, 1000, 1000, 64) == 0
    vp = ctypes.c_void_p
    lib.pointops_ball_query_backward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp,
                                                 vp, ctypes.c_size_t, vp]
    lib.pointops_ball_query_backward.restype = ctypes.c_int
    fake = vp(0x1000)
    rc = lib.pointops_ball_query_backward(fake, fake, fake, fake, 1, 1000, 1000, 64, fake, fake,
                                          fake, 16, None)
    assert rc == 1, lib.pointops_last_error()
    assert b"workspace" in lib.pointops_last_error()
