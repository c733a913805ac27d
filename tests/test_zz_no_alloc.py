"""pointops_fps_noalloc (FPS on the library's static scratch, for callers
that cannot allocate) against pointops_fps with a workspace, through the C
ABI: indices and sampled coordinates bit for bit, over consecutive calls
that reuse the same scratch (the second with a smaller input), and its
refusal of a shape beyond the scratch limit (lowered from the host)."""
import ctypes

import numpy as np
import pytest
import torch

from point_cloud_neighbor_amd import workloads as W

pytestmark = pytest.mark.gpu


def lib_fns(gpu):
    lib = gpu._load()
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.pointops_fps_noalloc.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp]
    lib.pointops_fps_noalloc.restype = ctypes.c_int
    return lib


def run_both(lib, x, M, start):
    B, N, _ = x.shape
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ws = torch.empty(max(1, lib.pointops_fps_workspace_bytes(B, N, M)), dtype=torch.uint8,
                     device="cuda")
    oi = torch.full((B, M), -7, dtype=torch.int64, device="cuda")
    ox = torch.full((B, M, 3), -7.0, dtype=torch.float32, device="cuda")
    assert lib.pointops_fps(x.data_ptr(), B, N, M, start, oi.data_ptr(), ox.data_ptr(),
                            ws.data_ptr(), ws.numel(), s) == 0
    ni = torch.full((B, M), -9, dtype=torch.int64, device="cuda")
    nx = torch.full((B, M, 3), -9.0, dtype=torch.float32, device="cuda")
    rc = lib.pointops_fps_noalloc(x.data_ptr(), B, N, M, start, ni.data_ptr(), nx.data_ptr(), s)
    assert rc == 0, lib.pointops_last_error()
    torch.cuda.synchronize()
    return oi.cpu().numpy(), ox.cpu().numpy(), ni.cpu().numpy(), nx.cpu().numpy()


# consecutive calls on the same scratch: a large cloud (63 workgroups), a
# smaller one (fewer workgroups, stale words of the first call in the
# scratch), 32 clouds (one scratch region per cloud), a one-workgroup cloud
CASES = [(0, 1, 100000, 4096, 0), (1, 1, 20000, 500, 17), (2, 32, 8192, 512, 3),
         (3, 1, 1024, 128, 5)]


def test_fps_noalloc_matches_fps(gpu):
    lib = lib_fns(gpu)
    for seed, B, N, M, start in CASES:
        x = torch.from_numpy(W.uniform_cube(100 + seed, B, N)).cuda()
        oi, ox, ni, nx = run_both(lib, x, M, start)
        assert np.array_equal(oi, ni), (B, N, M)
        assert np.array_equal(ox.view(np.uint32), nx.view(np.uint32)), (B, N, M)
        assert (ni >= 0).all() and (ni[:, 0] == start).all()


def test_fps_noalloc_refuses_beyond_its_scratch(gpu, monkeypatch):
    lib = lib_fns(gpu)
    x = torch.from_numpy(W.uniform_cube(7, 1, 100000)).cuda()
    oi = torch.full((1, 64), -3, dtype=torch.int64, device="cuda")
    monkeypatch.setenv("POINTOPS_FPS_SCRATCH_LIMIT", "1024")  # below this shape's need
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.pointops_fps_noalloc(x.data_ptr(), 1, 100000, 64, 0, oi.data_ptr(), None, s) == 2
    assert b"scratch" in lib.pointops_last_error()
    torch.cuda.synchronize()
    assert (oi.cpu().numpy() == -3).all()   # nothing launched
