"""MI355X-native dense, batched float32 point-cloud neighbour search.

Operations over (B, N, 3) float32 device tensors, each a hand-written HIP
kernel for gfx950 behind the C ABI declared in ``include/pointops.h``:

* ``furthest_point_sample(xyz, npoint, start_idx=0)`` -> int64 (B, npoint)
* ``knn(query, ref, k)`` -> (Euclidean distance float32, int64 index), (B, Q, k)
* ``ball_query(query, ref, radius, K)`` -> (squared distance float32,
  int64 index with -1 padding), (B, Q, K); the squared distances are
  differentiable with respect to both coordinate tensors
* ``ball_query_backward(query, ref, idx, grad_dist2)`` -> (grad_query, grad_ref)
* ragged batches: ``fps_ragged``, ``knn_ragged``, ``ball_query_ragged`` over
  clouds packed back to back in a flat (rows, 3) tensor with ``ptr`` offsets,
  and ``knn_padded``, ``ball_query_padded`` over padded clouds with lengths
* ``three_nn(unknown, known)`` -> the 3 nearest (distance, index), kNN k=3
* ``chamfer_distance(x, y, ...)`` -> (squared-L2 Chamfer loss, None),
  differentiable, with lengths and mean / sum reductions

The ops are loaded lazily so that ``workloads`` imports without a GPU; calling
an op without the built library or a gfx950 device raises, there is no CPU
fallback.
"""

__all__ = ["furthest_point_sample", "knn", "ball_query", "ball_query_backward",
           "fps_ragged", "knn_ragged", "ball_query_ragged", "knn_padded", "ball_query_padded",
           "three_nn", "chamfer_distance", "PointopsError"]


def __getattr__(name):
    if name in __all__ or name in ("fps_workspace_bytes", "library_path", "device_check"):
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
