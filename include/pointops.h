/*
 * pointops: dense, batched float32 point-cloud neighbour search on AMD
 * Instinct MI355X (gfx950), as a C ABI.
 *
 * The operations follow the contracts of the "mps-pointops" project page
 * (PyPI, version 0.5.0), sections "The operators in equations" and
 * "Contracts", and of its "Numerical contracts" page, section "Selection and
 * output". All of them evaluate the squared distance of a query q and a
 * reference x as
 *
 *     s32(q, x) = ((dx*dx + dy*dy) + dz*dz),   dx = fl32(q.x - x.x), ...
 *
 * with every operation a float32 operation rounded to nearest-even, no fused
 * multiply-add and float32 subnormals kept (the project page, section "How
 * the kernels work", fixes this order for FPS and kNN; this library uses it
 * for Ball Query as well). Results are therefore fully determined, indices
 * and distance bits included.
 *
 * Conventions shared by every entry point:
 *   - Point buffers are device pointers (memory of the current HIP device) to
 *     row-major, contiguous float32 arrays of shape (B, n, 3); index outputs
 *     are int64. The caller owns every buffer; the library never allocates or
 *     frees device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL: the default stream).
 *     Calls are asynchronous on that stream. Argument errors are detected on
 *     the host and returned before anything is launched or written; failures
 *     during execution surface at the caller's next synchronisation.
 *   - There is no CPU fallback: an unsupported device or argument is an error.
 *   - Inputs are read-only and may alias each other (query == ref is fine).
 *     Outputs must not alias inputs or each other.
 *   - Sizes are limited to n < 2^31 points per cloud.
 *   - Non-finite coordinates are outside the contract: the calls still
 *     terminate and write only inside their outputs, but the results are
 *     unspecified.
 *   - Thread safety: the library is stateless apart from a per-device property
 *     cache and a thread-local error message.
 */
#ifndef POINTOPS_H
#define POINTOPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum pointops_status {
    POINTOPS_OK = 0,
    POINTOPS_INVALID_ARGUMENT = 1, /* a size, index, radius or pointer is out of range */
    POINTOPS_UNSUPPORTED = 2,      /* valid request beyond a compiled limit (k > KMAX, sizes) */
    POINTOPS_UNSUPPORTED_DEVICE = 3, /* current device is not gfx950 with 64-wide waves */
    POINTOPS_HIP_ERROR = 4,        /* a HIP runtime call failed; see pointops_last_error() */
    POINTOPS_EXEC_TIMEOUT = 5      /* an FPS launch gave up a bounded cross-workgroup wait;
                                      reported by pointops_fps_status */
};

/* Largest k accepted by pointops_knn. The project page, section "Contracts",
 * caps k at a kernel constant and reports an explicit error beyond it; this
 * library does the same with its own constant. */
#define POINTOPS_KNN_KMAX 64

/*
 * Farthest point sampling.
 * Project page, section "The operators in equations", "Farthest point
 * sampling"; section "Contracts" (start index, repeat-0 rule).
 *   c_0 = start_idx; m_j = min over chosen centres u of s32(x_j, x_{c_u});
 *   c_{t+1} = the smallest j whose m_j equals max_l m_l.
 * Once every point is taken, all m are 0 and the remaining slots are 0.
 *
 *   xyz       (B, N, 3) float32, device.
 *   B, N, M   clouds, points per cloud, samples per cloud. B == 0 or M == 0 is
 *             a no-op. M may exceed N. N == 0 with M >= 1 is invalid.
 *   start_idx first centre of every cloud, 0 <= start_idx < N.
 *   out_idx   (B, M) int64, device: c_0 .. c_{M-1}.
 *   out_xyz   (B, M, 3) float32, device, or NULL: the sampled coordinates
 *             x_{c_t} (bit copies of the input).
 *   workspace device scratch of at least pointops_fps_workspace_bytes(B, N, M)
 *             bytes (NULL allowed when that size is 0). Its contents on entry
 *             do not matter; the call clears what it uses, on `stream`.
 *             Calls that share a workspace must be ordered (same stream).
 */
int pointops_fps(const float *xyz, int64_t B, int64_t N, int64_t M, int64_t start_idx,
                 int64_t *out_idx, float *out_xyz, void *workspace, size_t workspace_bytes,
                 void *stream);

/* Bytes of device workspace pointops_fps needs for this shape (it may be 0). */
size_t pointops_fps_workspace_bytes(int64_t B, int64_t N, int64_t M);

/*
 * pointops_fps without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, results and errors as pointops_fps;
 * it calls no hipMalloc, hipFree or allocating library routine.
 *
 * Its scratch is a static device array of 1 MiB in the library, one per GPU,
 * held until the process ends; every FPS plan the library makes for default
 * settings fits (the largest, many clouds of 3-4k points over three
 * workgroups each, needs about 0.75 MB; 2^20 points, 32 KB). A shape that
 * needs more returns POINTOPS_UNSUPPORTED before anything is launched. The
 * call clears what it uses first, on `stream`. All calls on one GPU share its
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must be ordered by the caller. A bounded wait that gives up (see
 * pointops_fps_status) leaves -1 in the unreached output slots; its status
 * word is not readable by the caller here.
 */
int pointops_fps_noalloc(const float *xyz, int64_t B, int64_t N, int64_t M, int64_t start_idx,
                         int64_t *out_idx, float *out_xyz, void *stream);

/*
 * Execution status of the last pointops_fps or pointops_fps_ragged call that
 * used `workspace` (the workspace and byte count given to that call) and
 * sampled at least one point; a call with nothing to sample (B, M or every
 * count 0) touches no workspace and leaves its word as it was.
 * The project page's contracts never let a failure pass silently (section
 * "Quick start": no silent fallback), and errors during execution surface at
 * the caller's next synchronisation (the conventions above); this is that
 * synchronisation for FPS.
 *
 * A multi-workgroup FPS launch keeps every workgroup of a cloud waiting on the
 * others at each exchange. Every such wait is bounded. A workgroup that gives
 * up raises a status word at the start of the workspace, and the output slots
 * its cloud had not reached hold -1. That can only happen when the cloud's
 * workgroups cannot all run at once, for example when another persistent
 * launch holds the compute units.
 *
 * The call waits for `stream` (hipStreamSynchronize), then copies the status
 * word to the host. It returns POINTOPS_OK, POINTOPS_EXEC_TIMEOUT (with a
 * message in pointops_last_error), POINTOPS_INVALID_ARGUMENT (NULL workspace,
 * or fewer than 8 bytes) or POINTOPS_HIP_ERROR. It writes nothing to the
 * device. The word stays raised until the next FPS call on that workspace
 * clears it.
 *
 *   exchanges  host int64, or NULL: set to the number of cross-workgroup
 *              exchanges the first cloud of that call made (in launch order;
 *              0 when the cloud ran in one workgroup). A measure of the
 *              call's latency chain: each exchange is one round trip through
 *              device memory between the cloud's workgroups.
 */
int pointops_fps_status(const void *workspace, size_t workspace_bytes, int64_t *exchanges,
                        void *stream);

/*
 * k nearest neighbours.
 * Project page, section "The operators in equations", "k nearest neighbors";
 * "Numerical contracts" page, section "Selection and output".
 *   For every query i of cloud b: sort the references j by (s32(q_i, x_j), j),
 *   keep the first k; out_idx = j, out_dist = sqrtf(s32) correctly rounded.
 * With a workspace of pointops_knn_workspace_bytes(B, Q, P) bytes (when that
 * is not 0) the call may counting-sort references and queries into a uniform
 * grid, bound every 16 (and every 1024) sorted references by a box, start
 * each query from the references around its own grid position and skip a box
 * when the lower bound of s32 over it (taken in the float32 order of s32, so
 * never above it) exceeds the query's current k-th distance; it does so from
 * 8192 references per cloud and 2^22 query-reference pairs on, for k > 32
 * from 32768 references (pointops_knn_search tells which search a shape
 * takes). Otherwise, and
 * with workspace NULL, every reference is scanned: for k <= 32 one query per
 * wave with a merged top-32 list, else (and for k <= 8 with many queries on
 * small clouds) one query per lane. Results are identical, bit for bit,
 * whatever the search. A non-NULL workspace smaller than needed is
 * INVALID_ARGUMENT.
 *
 *   query     (B, Q, 3) float32, device.      ref (B, P, 3) float32, device.
 *   k         1 <= k <= P (INVALID_ARGUMENT otherwise) and
 *             k <= POINTOPS_KNN_KMAX (UNSUPPORTED otherwise).
 *   out_dist  (B, Q, k) float32, device.      out_idx (B, Q, k) int64, device.
 *   B == 0 or Q == 0 is a no-op.
 */
int pointops_knn(const float *query, const float *ref, int64_t B, int64_t Q, int64_t P,
                 int64_t k, float *out_dist, int64_t *out_idx, void *workspace,
                 size_t workspace_bytes, void *stream);

/* Bytes of device workspace that lets pointops_knn sort the clouds into a grid
 * and skip far references (0 when that path is not used for this shape). */
size_t pointops_knn_workspace_bytes(int64_t B, int64_t Q, int64_t P);

/* The searches pointops_knn chooses from (same results, different speed). */
#define POINTOPS_KNN_SEARCH_LANES 0 /* full scan, one query per lane */
#define POINTOPS_KNN_SEARCH_WAVES 1 /* full scan, one or two queries per wave */
#define POINTOPS_KNN_SEARCH_GRID 2  /* grid sort and culled search */

/* Which search pointops_knn takes on the current device for this shape, with
 * (with_workspace != 0) or without its workspace: one of the
 * POINTOPS_KNN_SEARCH_* values above, or minus a status code
 * (INVALID_ARGUMENT for a shape pointops_knn rejects, the device errors).
 * Reads the same environment overrides as pointops_knn. */
int pointops_knn_search(int64_t B, int64_t Q, int64_t P, int64_t k, int with_workspace);

/* Bytes of device workspace that lets pointops_ball_query skip far blocks of
 * references: one bounding box per 64 references of each cloud (32 bytes),
 * and for clouds of more than 32768 references also room for the grid pass
 * (8 bytes per query, the sorted copies of references and queries, 16 bytes
 * each, their boxes and the cell histograms). */
size_t pointops_ball_query_workspace_bytes(int64_t B, int64_t Q, int64_t P);

/* The searches pointops_ball_query chooses from (same results). */
#define POINTOPS_BQ_SEARCH_SCAN 0   /* every reference, in index order */
#define POINTOPS_BQ_SEARCH_CULLED 1 /* index order, skipping blocks whose box is too far */
#define POINTOPS_BQ_SEARCH_GRID 2   /* the culled scan with a budget, then the grid pass */

/* Which search pointops_ball_query takes for this shape, with
 * (with_workspace != 0) or without its workspace: one of the
 * POINTOPS_BQ_SEARCH_* values above, or minus INVALID_ARGUMENT for a shape it
 * rejects. Reads the same environment overrides as pointops_ball_query. */
int pointops_ball_query_search(int64_t B, int64_t Q, int64_t P, int64_t K, int with_workspace);

/*
 * Dense Ball Query: the first K references within the radius, in input order.
 * Project page, section "The operators in equations", "Ball Query: first K
 * within a radius"; "Numerical contracts" page, section "Selection and output".
 * With a workspace of pointops_ball_query_workspace_bytes(B, Q, P) bytes the
 * call first bounds every block of 64 consecutive references by a box and
 * skips, for each query, the blocks whose lower bound of s32 is >= R2 (the
 * bound is taken in the same float32 order as s32, so it never exceeds it:
 * results are identical, bit for bit). This pays when consecutive references
 * are close in space (sorted clouds). On clouds of more than 32768 references
 * (and K <= 32) that scan stops after 128 blocks per wave, and the queries it
 * leaves short of K (sparse regions of clouds in random order) find the rest
 * of their first K hits through a uniform grid of the references, built on
 * the device only when some query is left. Workspace NULL scans every
 * reference. A non-NULL workspace smaller than needed is INVALID_ARGUMENT.
 *   R2 = fl32(radius * radius) with radius already a float32 (the caller's
 *   fl32(r)); J = the references j with s32(q_i, x_j) < R2, in increasing j;
 *   slot n < min(K, |J|) holds (J[n], s32 of J[n]); the rest hold (-1, +0.0f).
 *   A zero squared distance is a real match: test out_idx >= 0 for padding.
 *
 *   query     (B, Q, 3) float32, device.      ref (B, P, 3) float32, device.
 *   radius    finite and > 0 (INVALID_ARGUMENT otherwise).
 *   K         >= 1.  P == 0 is allowed: every slot is padding.
 *   out_dist2 (B, Q, K) float32, device.      out_idx (B, Q, K) int64, device.
 *   B == 0 or Q == 0 is a no-op.
 */
int pointops_ball_query(const float *query, const float *ref, int64_t B, int64_t Q, int64_t P,
                        float radius, int64_t K, float *out_dist2, int64_t *out_idx,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Ball Query backward: gradients of L through the returned squared distances.
 * Project page, section "The operators in equations", the gradient formulas
 * under "Ball Query: first K within a radius"; "Numerical contracts" page,
 * "Differentiation". With G = dL/dS (B, Q, K):
 *   grad_query[b,i] = 2 * sum over k with I[b,i,k] >= 0 of G (q_i - x_I),
 *   grad_ref[b,j]   = 2 * sum over (i,k) with I[b,i,k] = j of G (x_j - q_i).
 * Indices and the radius are not differentiated.
 *
 *   query, ref    the forward inputs, (B, Q, 3) and (B, P, 3) float32, device.
 *   idx           the forward index output (B, Q, K) int64; slots outside
 *                 [0, P) (the -1 padding) contribute nothing.
 *   grad_dist2    G, (B, Q, K) float32, device.
 *   grad_query    (B, Q, 3) float32, device, overwritten; or NULL to skip.
 *   grad_ref      (B, P, 3) float32, device, overwritten; or NULL to skip.
 *   workspace     NULL, or pointops_ball_query_backward_workspace_bytes()
 *                 bytes of device memory (smaller: INVALID_ARGUMENT); used
 *                 only when query == ref and Q == P, ignored otherwise.
 * float32 arithmetic: each term is 2 * (G * fl32(q - x)); a query's terms are
 * summed in a fixed order (deterministic); a reference's terms are added with
 * atomics in no fixed order, so grad_ref may differ between runs in the last
 * bits. B == 0 or Q == 0 zeroes grad_ref (if given) and returns.
 */
int pointops_ball_query_backward(const float *query, const float *ref, const int64_t *idx,
                                 const float *grad_dist2, int64_t B, int64_t Q, int64_t P,
                                 int64_t K, float *grad_query, float *grad_ref,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of the Ball Query backward's optional workspace (device memory,
 * caller-owned): used only when the query and reference buffers are the same
 * (query == ref, Q == P: a cloud queried by its own points). Then each tile
 * of rows writes its partial reference sums for a fixed window of reference
 * rows there, and a second kernel adds them, in tile order, in place of
 * most of the float atomics. 0 when Q != P or nothing to do. Reads
 * POINTOPS_BQ_BWD_TILE like the call. Allocation-free.
 */
size_t pointops_ball_query_backward_workspace_bytes(int64_t B, int64_t Q, int64_t P, int64_t K);

/*
 * Ragged batches: clouds of different sizes in one call.
 * Project page, section "Flat torch_cluster subset" (clouds back to back in
 * one flat point array, delimited by offsets, with separate offsets for the
 * query and reference sets; indices into the flat input; kNN of a cloud with
 * fewer than k references yields only the available neighbours) and section
 * "PyTorch3D-style Ball Query" (padded clouds with per-cloud lengths); its
 * roadmap, "Phase 1 follow-ups" (multi-workgroup FPS over uneven batches, each
 * cloud reduced on its own).
 *
 * A cloud is a segment of a flat point buffer: cloud b of a buffer of `rows`
 * rows ((rows, 3) float32, device) is rows [off[b], off[b] + cnt[b]). The
 * offset form (ptr) is off[b] = ptr[b], cnt[b] = ptr[b+1] - ptr[b]; the padded
 * form (B, n_max, 3) with lengths is off[b] = b * n_max, cnt[b] = lengths[b].
 * off and cnt are HOST arrays of B int64, read during the call only. Every
 * segment must lie inside its buffer; segments that name output rows must not
 * overlap (INVALID_ARGUMENT otherwise). Each cloud is computed exactly as the
 * dense entry point computes a batch of one, with its own sizes.
 *
 * Indices: with global_index != 0 a returned index is a row of the flat input
 * buffer (off[b] + local index), otherwise the local index within the cloud.
 *
 * workspace: device scratch of the size the matching *_workspace_bytes call
 * returns; the call writes a small description of the clouds into it (with
 * kernels on `stream`, no host-to-device copy), so calls that share one must
 * be ordered on one stream. Output rows outside every segment are not written.
 */

/* Workspace bytes of pointops_knn_ragged and pointops_ball_query_ragged for B
 * clouds (8 KiB covers 100 clouds). */
size_t pointops_ragged_workspace_bytes(int64_t B);

/*
 * Workspace bytes with which pointops_knn_ragged takes the grid search (the
 * culled search of the dense kNN, project page "mps-pointops", roadmap:
 * spatial structures for large clouds) for clouds with these query and
 * reference counts (host arrays of B entries) and this k; the results do not
 * change. It is pointops_ragged_workspace_bytes(B) when the full scan is the
 * better search, and about 16 * B * (max q_cnt + max r_cnt) bytes plus the
 * grid's cell counts otherwise (the grid is not taken when that padding would
 * exceed eight times the points' own room). With a smaller workspace
 * pointops_knn_ragged scans every reference of each cloud. 0 for invalid
 * counts.
 */
size_t pointops_knn_ragged_workspace_bytes(const int64_t *q_cnt, const int64_t *r_cnt, int64_t B,
                                           int64_t k);

/*
 * Workspace bytes with which pointops_ball_query_ragged takes its culled
 * search for clouds with these counts (host arrays of B entries) and this K:
 * an index-order scan that stops each query at K hits or at a budget of
 * references (or early, when the query's hit rate is too low to reach K
 * within it), then, only if a query was left, a uniform grid of each cloud
 * and the dense Ball Query's grid pass for the hits from where the scan
 * stopped (project page "mps-pointops", roadmap: spatial structures for large
 * clouds). The first-K result does not change. It is
 * pointops_ragged_workspace_bytes(B) when the plain scan is taken (K > 32,
 * clouds below 8192 references, or padding to the largest cloud above eight
 * times the points' own room), about 16 * B * (max q_cnt + max r_cnt) bytes
 * plus the grid's cell counts otherwise. With a smaller workspace
 * pointops_ball_query_ragged takes the plain scan. 0 for invalid counts.
 */
size_t pointops_ball_query_ragged_workspace_bytes(const int64_t *q_cnt, const int64_t *r_cnt,
                                                  int64_t B, int64_t K);

/*
 * kNN of ragged batches. For each cloud b, the queries are rows q_off[b] ..
 * of `query` and the references rows r_off[b] .. of `ref`; output row r of
 * out_dist / out_idx ((q_rows, k), device) belongs to query row r. Where a
 * cloud has fewer than k references the remaining slots of its rows hold
 * (+inf, -1). 1 <= k <= POINTOPS_KNN_KMAX.
 */
int pointops_knn_ragged(const float *query, int64_t q_rows, const int64_t *q_off,
                        const int64_t *q_cnt, const float *ref, int64_t r_rows,
                        const int64_t *r_off, const int64_t *r_cnt, int64_t B, int64_t k,
                        int global_index, float *out_dist, int64_t *out_idx, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * Ball Query of ragged batches: the dense contract (R2 = fl32(radius^2),
 * first K in increasing reference order, (-1, +0.0f) padding) per cloud;
 * output row r ((q_rows, K), device) belongs to query row r.
 */
int pointops_ball_query_ragged(const float *query, int64_t q_rows, const int64_t *q_off,
                               const int64_t *q_cnt, const float *ref, int64_t r_rows,
                               const int64_t *r_off, const int64_t *r_cnt, int64_t B,
                               float radius, int64_t K, int global_index, float *out_dist2,
                               int64_t *out_idx, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Workspace bytes of pointops_fps_ragged for these cloud and sample counts
 * (0 if they are invalid or no launch shape fits). */
size_t pointops_fps_ragged_workspace_bytes(const int64_t *x_cnt, const int64_t *out_cnt,
                                           int64_t B);

/*
 * Farthest point sampling of ragged batches. Cloud b is rows x_off[b] .. of
 * `xyz`; its out_cnt[b] samples go to rows out_off[b] .. of out_idx
 * ((out_rows,) int64, device) and, if out_xyz is not NULL, of out_xyz
 * ((out_rows, 3) float32). start: HOST array of B local start indices, or NULL
 * for 0. A cloud with out_cnt[b] > 0 needs x_cnt[b] > 0 and
 * 0 <= start[b] < x_cnt[b]; out_cnt[b] may exceed x_cnt[b] (the repeat-0 rule
 * of the dense call). Clouds are sampled independently and concurrently; a
 * large cloud is spread over several workgroups that reduce each step among
 * themselves only.
 */
int pointops_fps_ragged(const float *xyz, int64_t rows, const int64_t *x_off,
                        const int64_t *x_cnt, const int64_t *start, int64_t B, int64_t *out_idx,
                        float *out_xyz, int64_t out_rows, const int64_t *out_off,
                        const int64_t *out_cnt, int global_index, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * three_nn: the three nearest known points of every unknown point, Euclidean
 * distances and indices. Project page, "Minimal example" (the 0.5.0 call) and
 * roadmap, "Phase 2" (PointNet++ feature propagation). It is pointops_knn
 * with k = 3 (same order and ties): unknown (B, n, 3), known (B, m, 3),
 * m >= 3; out_dist, out_idx (B, n, 3), device; workspace as for pointops_knn
 * (NULL: full scan).
 */
int pointops_three_nn(const float *unknown, const float *known, int64_t B, int64_t n, int64_t m,
                      float *out_dist, int64_t *out_idx, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Workspace bytes for pointops_three_nn's grid search (as pointops_knn's). */
size_t pointops_three_nn_workspace_bytes(int64_t B, int64_t n, int64_t m);

/* Reductions of pointops_chamfer. */
enum pointops_reduction {
    POINTOPS_REDUCE_NONE = 0, /* batch only: one loss per cloud */
    POINTOPS_REDUCE_MEAN = 1,
    POINTOPS_REDUCE_SUM = 2
};

/* Workspace bytes of pointops_chamfer (and enough for pointops_chamfer_backward)
 * for B clouds of N and M points; large clouds without lengths get the kNN
 * grid search's workspace too. */
size_t pointops_chamfer_workspace_bytes(int64_t B, int64_t N, int64_t M);

/*
 * Squared-L2 Chamfer distance of x (B, N, 3) and y (B, M, 3), device.
 * Project page, roadmap "Phase 4": a(i) = the nearest point of y to x_i and
 * b(j) = the nearest point of x to y_j (the kNN order with k = 1: ties to the
 * smaller index); per cloud, the sum over i of s(x_i, y_a(i)) plus, unless
 * single_directional, the sum over j of s(y_j, x_b(j)), with s the float32
 * squared distance s32. x_lengths / y_lengths: HOST arrays of B lengths
 * (NULL: all points), 0 <= len <= N (M); only the first len points of a cloud
 * take part. point_reduction MEAN divides each direction's sum by its length
 * (a length of 0 counts as 1), SUM does not; batch_reduction MEAN / SUM
 * combine the clouds, NONE keeps one loss per cloud. A point whose other
 * cloud is empty contributes nothing.
 *
 *   loss      device float32: (B,) for batch_reduction NONE, else (1,). Sums
 *             are taken in float64 in a fixed order (deterministic).
 *   dist_xy, idx_xy  (B, N) device: s and a(i) per point of x, local indices;
 *             (0, -1) past x's length or without partner. dist_yx, idx_yx:
 *             (B, M) likewise for y; not used (may be NULL) when
 *             single_directional. These are the inputs of the backward.
 *   workspace pointops_chamfer_workspace_bytes(B, N, M) bytes of device scratch.
 *   Without lengths, large clouds find their nearest points with the kNN
 *   grid search (same results, bit for bit).
 */
int pointops_chamfer(const float *x, const float *y, int64_t B, int64_t N, int64_t M,
                     const int64_t *x_lengths, const int64_t *y_lengths, int point_reduction,
                     int batch_reduction, int single_directional, float *loss, float *dist_xy,
                     int64_t *idx_xy, float *dist_yx, int64_t *idx_yx, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * Gradients of the Chamfer loss with the nearest points held fixed (project
 * page, roadmap "Phase 4": the gradient of each selected pair goes to both
 * points: 2 w (p - o) to the point and its negation to its nearest point).
 * Same sizes, lengths and reductions as the forward call; idx_xy / idx_yx
 * its index outputs; grad_loss the upstream gradient, device float32, (B,)
 * for batch_reduction NONE, else (1,). grad_x (B, N, 3) and grad_y (B, M, 3),
 * device, are overwritten (either may be NULL). w = fl32(upstream gradient x
 * reduction factor); terms are added with float atomics in no fixed order,
 * so the last bits may differ between runs. The workspace is needed only when
 * lengths are given (then 16 * B bytes suffice).
 */
int pointops_chamfer_backward(const float *x, const float *y, int64_t B, int64_t N, int64_t M,
                              const int64_t *x_lengths, const int64_t *y_lengths,
                              int point_reduction, int batch_reduction, int single_directional,
                              const int64_t *idx_xy, const int64_t *idx_yx,
                              const float *grad_loss, float *grad_x, float *grad_y,
                              void *workspace, size_t workspace_bytes, void *stream);

/* POINTOPS_OK if `device` is a gfx950 GPU with 64-wide wavefronts (the kernels
 * assume that width), POINTOPS_UNSUPPORTED_DEVICE otherwise. The entry points
 * above run this check on the current device (cached per device). */
int pointops_device_check(int device);

/* A static description of a status code. */
const char *pointops_status_string(int status);

/* Detail of the last error on the calling thread ("" if none). */
const char *pointops_last_error(void);

/* Library ABI version: 5. */
int pointops_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* POINTOPS_H */
