"""Seeded synthetic point clouds for tests, the smoke check and the benchmark.

This module only draws and arranges coordinates. It holds no distance formula,
no selection rule and no threshold arithmetic, so that the GPU path and the
oracle can both take their inputs from it without sharing any of the method.

Every generator uses numpy's PCG64 ``default_rng(seed)``; float32 values come
from ``rng.random(dtype=np.float32)`` or from float64 normals rounded once to
float32, so the arrays are identical on every machine.

Workloads (sizes follow the five benchmark configurations of the project):

* ``tiny``      B=1, N=1024 uniform in [0,1)^3; FPS 128, kNN k=16 of the
                centres, Ball Query r=0.1 K=32 of the centres.
* ``grouping``  B=32, N=8192 on the unit sphere plus N(0, 0.01^2) jitter per
                coordinate; FPS 512, kNN k=32 of the centres (Point-MAE
                style grouping).
* ``large``     B=1, N=100000 uniform, random order; FPS 4096, kNN k=16 of
                every point against every point.
* ``sorted_bq`` B=1, N=100000 uniform, 1% snapped to a 1/64 grid, planted
                on-radius partners, then sorted by a 30-bit Morton code; Ball
                Query r=0.05 K=64 of every point against every point.
* ``stress``    B=1, N=1048576 from 16 Gaussian clusters (sigma 0.02) with
                0.1% exact duplicates; FPS 16384, then Ball Query r=0.03 K=32
                of the samples against all points.

Ragged batches (``ragged_workload``): 16 clouds, sizes log-uniform in
[1024, 65536], back to back in one flat array; FPS of ceil(N_b / 8) samples
per cloud, then kNN k=16 and Ball Query r=0.1 K=32 of each cloud's samples
against that cloud.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import numpy as np

# The float32 thresholds fl32(fl32(r)^2) of the planted radius, as bit patterns.
# Stored literally (not computed here) so this module carries no threshold
# arithmetic; the test suite checks them against the oracle's rule.
R2_BITS = {
    0.1: 0x3C23D70B,
    0.05: 0x3B23D70B,
    0.03: 0x3A6BEDFA,
    1.1: 0x3F9AE148,
}


def bits_to_f32(bits: int) -> np.float32:
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


# ----------------------------------------------------------------- output digests
#
# Whole outputs at the full workload sizes are compared by SHA-256 of their
# bytes: indices as little-endian int64, distances as little-endian float32
# bit patterns, row-major. Chunk digests over fixed runs of rows locate a
# mismatch without storing the outputs. These are byte hashes only.

DIGEST_DTYPES = {"idx": "<i8", "dist": "<f4"}


def output_digest(a: np.ndarray, kind: str) -> str:
    a = np.ascontiguousarray(a, dtype=np.dtype(DIGEST_DTYPES[kind]))
    return hashlib.sha256(a.tobytes()).hexdigest()


def output_rows(a: np.ndarray) -> np.ndarray:
    """The output as rows: (B, Q, K) -> (B*Q, K); (B, M) -> (B*M, 1)."""
    return a.reshape(-1, a.shape[-1]) if a.ndim == 3 else a.reshape(-1, 1)


def chunk_digests(a: np.ndarray, kind: str, rows_per_chunk: int) -> list:
    r = output_rows(a)
    return [output_digest(r[i:i + rows_per_chunk], kind) for i in range(0, len(r), rows_per_chunk)]


@dataclasses.dataclass
class Workload:
    name: str
    xyz: np.ndarray                 # (B, N, 3) float32, C-contiguous
    fps_m: int = 0                  # samples for FPS (0: FPS not run)
    fps_start: int = 0
    knn_k: int = 0                  # k for kNN (0: kNN not run)
    knn_queries: str = "none"       # "centres" (FPS output) or "points" (all points)
    bq_radius: float = 0.0          # Ball Query radius (0: not run)
    bq_k: int = 0
    bq_queries: str = "none"        # "centres" or "points"
    description: str = ""


# ----------------------------------------------------------------- generators

def unit_square() -> np.ndarray:
    """The 4-point unit square of the project's minimal example: (1, 4, 3)."""
    return np.array([[[0, 0, 0], [1, 0, 0], [0, 1, 0], [1, 1, 0]]], dtype=np.float32)


def uniform_cube(seed: int, B: int, N: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.random((B, N, 3), dtype=np.float32)


def sphere_shell(seed: int, B: int, N: int, sigma: float = 0.01) -> np.ndarray:
    """Points on the unit sphere (normalised Gaussian directions) plus an
    additive per-coordinate N(0, sigma^2) jitter, rounded once to float32."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((B, N, 3))
    g /= np.linalg.norm(g, axis=-1, keepdims=True)
    g += sigma * rng.standard_normal((B, N, 3))
    return g.astype(np.float32)


def morton_order(xyz: np.ndarray, bits: int = 10) -> np.ndarray:
    """Stable argsort of an (N, 3) cloud by its 3*bits-bit Morton code: each
    coordinate is quantised to floor(x * 2^bits) clipped to [0, 2^bits - 1];
    bit b of x goes to code bit 3b, of y to 3b+1, of z to 3b+2."""
    q = np.floor(xyz.astype(np.float64) * (1 << bits)).astype(np.int64)
    q = np.clip(q, 0, (1 << bits) - 1)
    code = np.zeros(len(xyz), dtype=np.int64)
    for b in range(bits):
        for d in range(3):
            code |= ((q[:, d] >> b) & 1) << (3 * b + d)
    return np.argsort(code, kind="stable")


def _three_squares(rng: np.random.Generator, target: int):
    """Random integers (a, b, c) with a^2 + b^2 + c^2 == target, by search over
    batches of random (a, b) with an exact integer square-root test."""
    root = math.isqrt(target)
    for _ in range(100):
        a = rng.integers(0, root + 1, size=65536, dtype=np.int64)
        rest = target - a * a
        b = np.floor(rng.random(65536) * (np.sqrt(rest.astype(np.float64)) + 1)).astype(np.int64)
        c2 = rest - b * b
        ok = c2 >= 0
        c = np.floor(np.sqrt(np.where(ok, c2, 0).astype(np.float64))).astype(np.int64)
        c += (c + 1) * (c + 1) <= c2          # exact integer square root
        c -= c * c > c2
        hit = np.nonzero(ok & (c * c == c2))[0]
        if len(hit):
            n = hit[0]
            v = np.array([a[n], b[n], c[n]], dtype=np.int64)
            assert int(v @ v) == target
            v *= rng.choice([-1, 1], size=3)
            return v[rng.permutation(3)]
    raise RuntimeError(f"no three-square representation found for {target}")


def plant_radius_partners(rng, xyz: np.ndarray, anchors: np.ndarray, victims: np.ndarray,
                          r2_bits: int) -> np.ndarray:
    """Overwrite points so that exact on-radius cases exist.

    For each anchor (a point on the 1/64 grid) three victims become
    anchor + (a, b, c) * 2^-e, where e is chosen from the exponent of the
    float32 threshold T (given as bits) so that T = M * 2^-e with a 24-bit
    integer M, and a^2 + b^2 + c^2 is M - 1, M or M + 1. All coordinates are
    then dyadic with few bits, so every difference, square and sum of the pair
    is exact in float32 and the pair's squared distance is exactly the float
    below T, T itself, or the float above T. Returns the planted
    (anchor, victim, numerator) triples for reference."""
    exp_field = (r2_bits >> 23) & 0xFF
    mant = (r2_bits & 0x7FFFFF) | 0x800000
    e = 150 - exp_field              # T = mant * 2^(exp_field - 150)
    assert e % 2 == 0, "offset scale must be a power of two"
    scale = 2.0 ** (-(e // 2))
    planted = []
    vi = 0
    for a in anchors:
        for delta in (-1, 0, 1):
            v = victims[vi]
            vi += 1
            off = _three_squares(rng, mant + delta).astype(np.float64) * scale
            xyz[v] = (xyz[a].astype(np.float64) + off).astype(np.float32)
            assert np.all(xyz[v].astype(np.float64) == xyz[a].astype(np.float64) + off)
            planted.append((int(a), int(v), int(mant + delta)))
    return np.array(planted, dtype=np.int64)


def sorted_bq_cloud(seed: int = 0, N: int = 100000, snap_frac: float = 0.01,
                    n_anchor: int = 100, r2_bits: int = R2_BITS[0.05]) -> np.ndarray:
    """Uniform cloud, 1% snapped to the 1/64 grid (exact ties), on-radius
    partners planted around 100 of the snapped points, then Morton-sorted."""
    rng = np.random.default_rng(seed)
    xyz = rng.random((N, 3), dtype=np.float32)
    n_snap = int(round(N * snap_frac))
    perm = rng.permutation(N)
    snapped = perm[:n_snap]
    xyz[snapped] = np.round(xyz[snapped].astype(np.float64) * 64.0).astype(np.float32) / np.float32(64)
    anchors = snapped[:n_anchor]
    victims = perm[n_snap:n_snap + 3 * n_anchor]
    plant_radius_partners(rng, xyz, anchors, victims, r2_bits)
    order = morton_order(xyz)
    return np.ascontiguousarray(xyz[order])[None]


def clustered_cloud(seed: int = 0, N: int = 1 << 20, n_clusters: int = 16, sigma: float = 0.02,
                    dup_frac: float = 0.001) -> np.ndarray:
    """Gaussian clusters (centres uniform in [0,1)^3) with exact duplicates."""
    rng = np.random.default_rng(seed)
    centres = rng.random((n_clusters, 3))
    label = rng.integers(0, n_clusters, size=N)
    xyz = (centres[label] + sigma * rng.standard_normal((N, 3))).astype(np.float32)
    n_dup = int(N * dup_frac)
    perm = rng.permutation(N)
    dst, src = perm[:n_dup], perm[n_dup:2 * n_dup]
    xyz[dst] = xyz[src]
    return xyz[None]


def integer_cloud(seed: int, B: int, N: int, lo: int = 0, hi: int = 4) -> np.ndarray:
    """Small-integer coordinates: every float32 operation on them is exact and
    many distances tie exactly."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, size=(B, N, 3)).astype(np.float32)


def dyadic_cloud(seed: int, B: int, N: int, denom: int = 64) -> np.ndarray:
    """Multiples of 1/denom in [0, 1]: exact arithmetic with ties."""
    rng = np.random.default_rng(seed)
    return (rng.integers(0, denom + 1, size=(B, N, 3)).astype(np.float64) / denom).astype(np.float32)


def line_cloud(N: int) -> np.ndarray:
    """Points (j, 0, 0) for j = 0..N-1."""
    xyz = np.zeros((1, N, 3), dtype=np.float32)
    xyz[0, :, 0] = np.arange(N, dtype=np.float32)
    return xyz


def subnormal_cloud(seed: int, N: int) -> np.ndarray:
    """Points about 1e-20 from the origin and from each other, so squared
    distances are float32 subnormals (about 1e-40)."""
    rng = np.random.default_rng(seed)
    return (rng.integers(-4, 5, size=(1, N, 3)) * 1e-20).astype(np.float32)


# ----------------------------------------------------------------- named workloads

def workload(name: str) -> Workload:
    if name == "unit_square":
        return Workload(name, unit_square(), fps_m=2, knn_k=2, knn_queries="centres",
                        bq_radius=1.1, bq_k=2, bq_queries="centres",
                        description="4-point unit square, the project's minimal example")
    if name == "tiny":
        return Workload(name, uniform_cube(0, 1, 1024), fps_m=128, knn_k=16,
                        knn_queries="centres", bq_radius=0.1, bq_k=32, bq_queries="centres",
                        description="B=1 N=1024 uniform [0,1)^3 seed 0")
    if name == "grouping":
        return Workload(name, sphere_shell(0, 32, 8192, 0.01), fps_m=512, knn_k=32,
                        knn_queries="centres",
                        description="B=32 N=8192 unit sphere + N(0,0.01^2) jitter, seed 0")
    if name == "large":
        return Workload(name, uniform_cube(0, 1, 100000), fps_m=4096, knn_k=16,
                        knn_queries="points",
                        description="B=1 N=100000 uniform [0,1)^3 random order, seed 0")
    if name == "sorted_bq":
        return Workload(name, sorted_bq_cloud(0), bq_radius=0.05, bq_k=64, bq_queries="points",
                        description="B=1 N=100000 uniform, 1% on the 1/64 grid, planted "
                                    "on-radius partners, 30-bit Morton order, seed 0")
    if name == "stress":
        return Workload(name, clustered_cloud(0), fps_m=16384, bq_radius=0.03, bq_k=32,
                        bq_queries="centres",
                        description="B=1 N=1048576 16 Gaussian clusters sigma 0.02, "
                                    "0.1% duplicates, seed 0")
    raise KeyError(name)


WORKLOADS = ("unit_square", "tiny", "grouping", "large", "sorted_bq", "stress")


# ----------------------------------------------------------------- ragged batches

@dataclasses.dataclass
class Ragged:
    """Clouds back to back in one flat (rows, 3) float32 array: cloud b is rows
    ptr[b] .. ptr[b+1]."""
    xyz: np.ndarray
    ptr: np.ndarray
    fps_counts: np.ndarray = None   # samples per cloud
    knn_k: int = 0
    bq_radius: float = 0.0
    bq_k: int = 0
    description: str = ""

    @property
    def off(self) -> np.ndarray:
        return np.ascontiguousarray(self.ptr[:-1])

    @property
    def cnt(self) -> np.ndarray:
        return np.diff(self.ptr)


def ragged_sizes(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """B cloud sizes, log-uniform in [lo, hi]."""
    rng = np.random.default_rng(seed)
    u = rng.random(B)
    return np.floor(np.exp(np.log(lo) + u * (np.log(hi + 1) - np.log(lo)))).astype(np.int64)


def ragged_batch(seed: int, sizes, maker=None) -> Ragged:
    """One cloud per size, each drawn by ``maker(seed_b, 1, n)`` (default
    uniform_cube) with its own seed, concatenated."""
    maker = maker or uniform_cube
    sizes = np.asarray(sizes, dtype=np.int64)
    parts = [maker(seed * 1000 + b, 1, int(n))[0] for b, n in enumerate(sizes)]
    xyz = np.concatenate(parts, axis=0) if len(parts) else np.zeros((0, 3), np.float32)
    ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    return Ragged(np.ascontiguousarray(xyz, dtype=np.float32), ptr)


def ragged_workload(seed: int = 0) -> Ragged:
    sizes = ragged_sizes(seed, 16, 1024, 65536)
    r = ragged_batch(seed, sizes)
    r.fps_counts = (sizes + 7) // 8
    r.knn_k = 16
    r.bq_radius = 0.1
    r.bq_k = 32
    r.description = ("16 uniform clouds, sizes log-uniform in [1024, 65536] (seed %d, %d points); "
                     "FPS ceil(N/8) per cloud, kNN k=16 and Ball Query r=0.1 K=32 of the "
                     "samples" % (seed, int(sizes.sum())))
    return r
