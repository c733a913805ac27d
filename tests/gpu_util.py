"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library, compare with the oracle.

The bar: indices bit-exact; distances within 1e-6 relative (1e-7 absolute near
zero). The design also claims bit-exact distances, which the tests assert
separately."""
import numpy as np
import torch

REL, ABS = 1e-6, 1e-7


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def assert_dist_close(got, want, what):
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    with np.errstate(invalid="ignore"):  # inf - inf where both are padding
        err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bound = np.maximum(REL * np.abs(want.astype(np.float64)), ABS)
    bad = ~((got == want) | (err <= bound))  # equal infinities (kNN padding) are fine
    assert not bad.any(), f"{what}: {int(bad.sum())} values outside tolerance, first at {np.argwhere(bad)[0]}"
    nbits = int((got.view(np.uint32) != want.view(np.uint32)).sum())
    assert nbits == 0, f"{what}: {nbits} values differ in their bits"


def assert_idx_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = got != want
    assert not bad.any(), f"{what}: {int(bad.sum())} index mismatches, first at {np.argwhere(bad)[0]}: got {got[tuple(np.argwhere(bad)[0])]} want {want[tuple(np.argwhere(bad)[0])]}"


def gather(xyz, idx):
    return np.take_along_axis(xyz, idx[..., None].repeat(3, axis=-1), axis=1)
