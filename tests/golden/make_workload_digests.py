"""Write ``workload_digests.json``: SHA-256 digests of the oracle's whole
outputs on the five benchmark workloads (C1-C5) at full size.

Every value stored here comes from ``oracle/`` alone, run on the seeded inputs
of ``point_cloud_neighbor_amd.workloads``; the GPU library is never loaded.
The pages count mismatches over whole outputs (project page, section
"Correctness checks": every benchmark row records its mismatch counts), so the
GPU tests and the benchmark compare whole outputs against these digests.

Chained inputs follow the workloads: the kNN and Ball Query queries of
``tiny`` and the kNN queries of ``grouping`` are the points the oracle's FPS
selected (gathered by index, no arithmetic), the Ball Query queries of
``stress`` likewise; ``large`` and ``sorted_bq`` query every point.

Run from the repository root: ``python -m tests.golden.make_workload_digests``
(about 8 minutes on 8 host threads; the full 100k x 100k kNN dominates).
Digests: see ``point_cloud_neighbor_amd.workloads.output_digest`` (int64 /
float32 little-endian bytes, row-major) and ``chunk_digests`` (runs of
``CHUNK_ROWS`` output rows; an FPS output (B, M) is B*M rows of one index).
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from point_cloud_neighbor_amd import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload_digests.json")
CHUNK_ROWS = 4096
THREADS = int(os.environ.get("DIGEST_THREADS", os.cpu_count() or 1))


def gather(xyz, idx):
    return np.ascontiguousarray(np.take_along_axis(xyz, idx[..., None].repeat(3, axis=-1), axis=1))


def entry(idx, dist=None):
    e = {"shape": list(idx.shape), "chunk_rows": CHUNK_ROWS,
         "idx": W.output_digest(idx, "idx"), "idx_chunks": W.chunk_digests(idx, "idx", CHUNK_ROWS)}
    if dist is not None:
        e["dist"] = W.output_digest(dist, "dist")
        e["dist_chunks"] = W.chunk_digests(dist, "dist", CHUNK_ROWS)
    return e


def run_workload(name):
    w = W.workload(name)
    x = w.xyz
    res = {"input_sha256": W.output_digest(x, "dist"), "description": w.description}
    t0 = time.time()
    centres = None
    if w.fps_m:
        c = oracle.fps(x, w.fps_m, w.fps_start, threads=THREADS)
        res["fps"] = entry(c)
        res["fps"]["m"], res["fps"]["start_idx"] = w.fps_m, w.fps_start
        centres = gather(x, c)
    if w.knn_k:
        q = centres if w.knn_queries == "centres" else x
        d, i = oracle.knn(q, x, w.knn_k, threads=THREADS)
        res["knn"] = entry(i, d)
        res["knn"]["k"], res["knn"]["queries"] = w.knn_k, w.knn_queries
    if w.bq_k:
        q = centres if w.bq_queries == "centres" else x
        d2, i = oracle.ball_query(q, x, w.bq_radius, w.bq_k, threads=THREADS)
        res["bq"] = entry(i, d2)
        res["bq"]["radius"], res["bq"]["K"] = w.bq_radius, w.bq_k
        res["bq"]["queries"] = w.bq_queries
        # pairs a first-K scan in index order examines: min(P, last hit + 1)
        # for a full row, else P (the algorithmic work of the Ball Query scan)
        P = x.shape[1]
        full = i[..., -1] >= 0
        res["bq"]["scan_pairs"] = int(np.where(full, i[..., -1] + 1, P).sum())
    res["oracle_seconds"] = round(time.time() - t0, 1)
    print(f"{name}: {res['oracle_seconds']} s", flush=True)
    return res


def main(names=("tiny", "grouping", "large", "sorted_bq", "stress")):
    oracle.build(force=False)
    doc = {
        "what": "SHA-256 of the oracle's whole outputs on the benchmark workloads "
                "(project page, 'Correctness checks': mismatches are counted over whole outputs)",
        "generator": "tests/golden/make_workload_digests.py (calls only oracle/)",
        "numpy": np.__version__,
        "workloads": {},
    }
    if os.path.exists(OUT):
        with open(OUT) as f:
            old = json.load(f)
        doc["workloads"].update(old.get("workloads", {}))
    for n in names:
        doc["workloads"][n] = run_workload(n)
        with open(OUT, "w") as f:
            json.dump(doc, f, indent=1, sort_keys=True)
            f.write("\n")


if __name__ == "__main__":
    main(tuple(sys.argv[1:]) or ("tiny", "grouping", "large", "sorted_bq", "stress"))
