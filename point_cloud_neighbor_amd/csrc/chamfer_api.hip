// C ABI of three_nn and the Chamfer distance. Declarations and contracts are
// in include/pointops.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "../../include/pointops.h"
#include "api_internal.h"
#include "segments.h"

namespace pointops {
hipError_t launch_chamfer_pad(float*, int64_t*, int64_t, int64_t, const int64_t*, hipStream_t);
int64_t chamfer_chunks(int64_t B, int64_t N, int64_t M);
hipError_t launch_chamfer_reduce(const float*, const float*, int64_t, int64_t, int64_t,
                                 const int64_t*, const int64_t*, int, int, int, double*, float*,
                                 hipStream_t);
hipError_t launch_chamfer_backward(const float*, const float*, int64_t, int64_t, int64_t,
                                   const int64_t*, const int64_t*, int, int, int,
                                   const int64_t*, const int64_t*, const float*, float*, float*,
                                   hipStream_t);
hipError_t launch_zero_f32(float*, size_t, hipStream_t);
}  // namespace pointops

using namespace pointops::api;

namespace {

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Workspace: both length arrays, the per-cloud partial losses, the two cloud
// tables of the nearest-point searches (with lengths), then the grid of the
// kNN grid search (without lengths, for large clouds; both directions use it
// in turn).
struct ChamferLayout {
    size_t lens, part, table_xy, table_yx, grid, grid_bytes, total;
};

ChamferLayout chamfer_layout(int64_t B, int64_t N, int64_t M) {
    ChamferLayout l;
    l.lens = 0;
    l.part = align256((size_t)2 * B * sizeof(int64_t));
    // two float64 sums per (cloud, chunk of the loss reduction)
    l.table_xy = l.part + align256((size_t)B * (size_t)pointops::chamfer_chunks(B, N, M) * 2 *
                                   sizeof(double));
    const size_t t = align256((size_t)pointops::seg_table_words(B) * sizeof(int64_t));
    l.table_yx = l.table_xy + t;
    l.grid = l.table_yx + t;
    l.grid_bytes = 0;
    if (B > 0 && N > 0 && M > 0) {
        if (knn_use_grid(B, N, M))
            l.grid_bytes = std::max(l.grid_bytes, pointops::knn_grid_workspace_bytes(B, N, M));
        if (knn_use_grid(B, M, N))
            l.grid_bytes = std::max(l.grid_bytes, pointops::knn_grid_workspace_bytes(B, M, N));
    }
    l.total = std::max<size_t>(l.grid + align256(l.grid_bytes), 256);
    return l;
}

int check_lengths(const char* what, const int64_t* len, int64_t B, int64_t n) {
    if (!len) return POINTOPS_OK;
    for (int64_t b = 0; b < B; ++b)
        if (len[b] < 0 || len[b] > n)
            return fail(POINTOPS_INVALID_ARGUMENT, "%s[%lld] = %lld not in [0, %lld]", what,
                        (long long)b, (long long)len[b], (long long)n);
    return POINTOPS_OK;
}

int check_chamfer(const float* x, const float* y, int64_t B, int64_t N, int64_t M,
                  const int64_t* x_lengths, const int64_t* y_lengths, int point_reduction,
                  int batch_reduction) {
    if (B < 0 || N < 0 || M < 0) return fail(POINTOPS_INVALID_ARGUMENT, "negative size");
    if (N >= kMaxPoints || M >= kMaxPoints || B >= kMaxPoints)
        return fail(POINTOPS_UNSUPPORTED, "sizes >= 2^31");
    if (point_reduction != POINTOPS_REDUCE_MEAN && point_reduction != POINTOPS_REDUCE_SUM)
        return fail(POINTOPS_INVALID_ARGUMENT, "point_reduction must be MEAN or SUM");
    if (batch_reduction != POINTOPS_REDUCE_NONE && batch_reduction != POINTOPS_REDUCE_MEAN &&
        batch_reduction != POINTOPS_REDUCE_SUM)
        return fail(POINTOPS_INVALID_ARGUMENT, "batch_reduction must be NONE, MEAN or SUM");
    int st = check_lengths("x_lengths", x_lengths, B, N);
    if (st != POINTOPS_OK) return st;
    st = check_lengths("y_lengths", y_lengths, B, M);
    if (st != POINTOPS_OK) return st;
    if ((B * N > 0 && !x) || (B * M > 0 && !y))
        return fail(POINTOPS_INVALID_ARGUMENT, "null pointer");
    return POINTOPS_OK;
}

// Lengths (either may be NULL: the full cloud) to the device, as [lx | ly].
int upload_lengths(const int64_t* x_lengths, const int64_t* y_lengths, int64_t B, int64_t N,
                   int64_t M, int64_t* dev, hipStream_t s) {
    std::vector<int64_t> h((size_t)2 * B);
    for (int64_t b = 0; b < B; ++b) {
        h[(size_t)b] = x_lengths ? x_lengths[b] : N;
        h[(size_t)(B + b)] = y_lengths ? y_lengths[b] : M;
    }
    hipError_t e = pointops::upload_words(h.data(), 2 * B, dev, s);
    return e == hipSuccess ? POINTOPS_OK : hip_fail(e, "length upload");
}

// Nearest point of every row of `a` (B, n) among the first lb[b] points of
// `b_` (B, m), squared distance kept; rows past la[b] hold (0, -1).
int nearest(const float* a, const float* bpts, int64_t B, int64_t n, int64_t m,
            const int64_t* la, const int64_t* lb, const int64_t* dev_la, float* dist,
            int64_t* idx, void* table_ws, size_t table_bytes, void* grid_ws, size_t grid_bytes,
            const DeviceInfo& dev, hipStream_t s) {
    if (B * n == 0) return POINTOPS_OK;
    hipError_t e;
    if (!la && !lb && m > 0 && knn_use_grid(B, n, m) && knn_grid_pays(1, B, n, m) &&
        grid_bytes >= pointops::knn_grid_workspace_bytes(B, n, m)) {
        e = pointops::launch_knn_grid(a, bpts, B, n, m, 1, dist, idx, 1,
                                      knn_grid_nw(1, 1, B * n, B * m), grid_ws, 1, nullptr, s);
        return e == hipSuccess ? POINTOPS_OK : hip_fail(e, "nearest launch");
    }
    if (!la && !lb) {
        const KnnWavePlan wp = knn_wave_plan(1, B * n, m, dev.cus);
        if (wp.nw)
            e = pointops::launch_knn_wave(a, bpts, B, n, m, 1, dist, idx, wp.nw, wp.qw, nullptr,
                                          0, 0, 1, s);
        else
            e = pointops::launch_knn(a, bpts, B, n, m, 1, dist, idx, 1,
                                     knn_waves(1, B * ((n + 63) / 64), dev.cus), nullptr, 0, 0,
                                     1, s);
        return e == hipSuccess ? POINTOPS_OK : hip_fail(e, "nearest launch");
    }
    std::vector<int64_t> qo((size_t)B), qc((size_t)B), ro((size_t)B), rc((size_t)B);
    int64_t queries = 0, max_refs = 0;
    for (int64_t b = 0; b < B; ++b) {
        qo[(size_t)b] = b * n;
        qc[(size_t)b] = la ? la[b] : n;
        ro[(size_t)b] = b * m;
        rc[(size_t)b] = lb ? lb[b] : m;
        queries += qc[(size_t)b];
        if (qc[(size_t)b] > 0) max_refs = std::max(max_refs, rc[(size_t)b]);
    }
    e = pointops::launch_chamfer_pad(dist, idx, B, n, dev_la, s);
    if (e != hipSuccess) return hip_fail(e, "chamfer pad");
    // The grid search over the clouds' own counts when it pays and the grid's
    // room (sized for the full clouds) holds it; the cloud records go where
    // the full scan's table would.
    const RaggedKnnGrid g = ragged_knn_grid(qc.data(), rc.data(), B, 1);
    if (g.use && table_bytes >= g.grid && grid_bytes >= g.grid_bytes) {
        int64_t* clouds = (int64_t*)table_ws;
        int st = upload_grid_clouds(qo.data(), qc.data(), ro.data(), rc.data(), B, false, clouds,
                                    0, s);
        if (st != POINTOPS_OK) return st;
        int64_t refs = 0;
        for (int64_t b = 0; b < B; ++b) refs += rc[(size_t)b];
        e = pointops::launch_knn_grid(a, bpts, B, g.Q, g.P, 1, dist, idx, 1,
                                      knn_grid_nw(1, 1, queries, refs), grid_ws, 1, clouds, s);
        return e == hipSuccess ? POINTOPS_OK : hip_fail(e, "nearest launch");
    }
    const KnnWavePlan wp = knn_wave_plan(1, queries, max_refs, dev.cus);
    const Table t = search_table(qo.data(), qc.data(), ro.data(), rc.data(), B,
                                 wp.nw ? wp.nw * wp.qw : 64, false);
    if (t.units == 0) return POINTOPS_OK;
    int64_t* table = nullptr;
    int st = upload(t, table_ws, table_bytes, s, &table);
    if (st != POINTOPS_OK) return st;
    if (wp.nw)
        e = pointops::launch_knn_wave(a, bpts, 0, 0, 0, 1, dist, idx, wp.nw, wp.qw, table, t.nseg,
                                      t.units, 1, s);
    else
        e = pointops::launch_knn(a, bpts, 0, 0, 0, 1, dist, idx, 1,
                                 knn_waves(1, t.units, dev.cus), table, t.nseg, t.units, 1, s);
    return e == hipSuccess ? POINTOPS_OK : hip_fail(e, "nearest launch");
}

}  // namespace

extern "C" {

int pointops_three_nn(const float* unknown, const float* known, int64_t B, int64_t n, int64_t m,
                      float* out_dist, int64_t* out_idx, void* workspace, size_t workspace_bytes,
                      void* stream) {
    clear_error();
    if (m < 3 && B > 0 && n > 0)
        return fail(POINTOPS_INVALID_ARGUMENT, "three_nn needs at least 3 known points, got %lld",
                    (long long)m);
    return pointops_knn(unknown, known, B, n, m, 3, out_dist, out_idx, workspace,
                        workspace_bytes, stream);
}

size_t pointops_three_nn_workspace_bytes(int64_t B, int64_t n, int64_t m) {
    return pointops_knn_workspace_bytes(B, n, m);
}

size_t pointops_chamfer_workspace_bytes(int64_t B, int64_t N, int64_t M) {
    return B < 0 || N < 0 || M < 0 ? 0 : chamfer_layout(B, N, M).total;
}

int pointops_chamfer(const float* x, const float* y, int64_t B, int64_t N, int64_t M,
                     const int64_t* x_lengths, const int64_t* y_lengths, int point_reduction,
                     int batch_reduction, int single_directional, float* loss, float* dist_xy,
                     int64_t* idx_xy, float* dist_yx, int64_t* idx_yx, void* workspace,
                     size_t workspace_bytes, void* stream) {
    clear_error();
    int st = check_chamfer(x, y, B, N, M, x_lengths, y_lengths, point_reduction,
                           batch_reduction);
    if (st != POINTOPS_OK) return st;
    if (!loss || (B * N > 0 && (!dist_xy || !idx_xy)) ||
        (!single_directional && B * M > 0 && (!dist_yx || !idx_yx)))
        return fail(POINTOPS_INVALID_ARGUMENT, "null output pointer");
    const ChamferLayout l = chamfer_layout(B, N, M);
    if (!workspace || workspace_bytes < l.total)
        return fail(POINTOPS_INVALID_ARGUMENT, "workspace of %zu bytes given, %zu needed",
                    workspace_bytes, l.total);
    DeviceInfo* dev = nullptr;
    st = current_device(&dev);
    if (st != POINTOPS_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    int64_t* lens = (int64_t*)(ws + l.lens);
    const bool have_len = x_lengths || y_lengths;
    if (have_len && B > 0) {
        st = upload_lengths(x_lengths, y_lengths, B, N, M, lens, s);
        if (st != POINTOPS_OK) return st;
    }
    const int64_t* dlx = have_len ? lens : nullptr;
    const int64_t* dly = have_len ? lens + B : nullptr;
    const size_t tb = l.table_yx - l.table_xy;
    st = nearest(x, y, B, N, M, x_lengths, y_lengths, dlx, dist_xy, idx_xy, ws + l.table_xy, tb,
                 ws + l.grid, l.grid_bytes, *dev, s);
    if (st != POINTOPS_OK) return st;
    if (!single_directional) {
        st = nearest(y, x, B, M, N, y_lengths, x_lengths, dly, dist_yx, idx_yx, ws + l.table_yx,
                     tb, ws + l.grid, l.grid_bytes, *dev, s);
        if (st != POINTOPS_OK) return st;
    }
    hipError_t e = pointops::launch_chamfer_reduce(
        dist_xy, dist_yx, B, N, M, dlx, dly, point_reduction == POINTOPS_REDUCE_MEAN,
        batch_reduction, single_directional != 0, (double*)(ws + l.part), loss, s);
    if (e != hipSuccess) return hip_fail(e, "chamfer reduce");
    return POINTOPS_OK;
}

int pointops_chamfer_backward(const float* x, const float* y, int64_t B, int64_t N, int64_t M,
                              const int64_t* x_lengths, const int64_t* y_lengths,
                              int point_reduction, int batch_reduction, int single_directional,
                              const int64_t* idx_xy, const int64_t* idx_yx,
                              const float* grad_loss, float* grad_x, float* grad_y,
                              void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    int st = check_chamfer(x, y, B, N, M, x_lengths, y_lengths, point_reduction,
                           batch_reduction);
    if (st != POINTOPS_OK) return st;
    if (!grad_x && !grad_y) return POINTOPS_OK;
    if (B > 0 && (!grad_loss || (N > 0 && !idx_xy) ||
                  (!single_directional && M > 0 && !idx_yx)))
        return fail(POINTOPS_INVALID_ARGUMENT, "null pointer");
    // only the length arrays are used here
    const ChamferLayout l = chamfer_layout(B, 0, 0);
    const bool have_len = x_lengths || y_lengths;
    if (have_len && (!workspace || workspace_bytes < l.part))
        return fail(POINTOPS_INVALID_ARGUMENT, "workspace of %zu bytes given, %zu needed",
                    workspace_bytes, l.part);
    st = current_device(nullptr);
    if (st != POINTOPS_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (grad_x && (e = pointops::launch_zero_f32(grad_x, (size_t)(B * N * 3), s)) != hipSuccess)
        return hip_fail(e, "gradient clear");
    if (grad_y && (e = pointops::launch_zero_f32(grad_y, (size_t)(B * M * 3), s)) != hipSuccess)
        return hip_fail(e, "gradient clear");
    int64_t* lens = (int64_t*)((char*)workspace + l.lens);
    if (have_len && B > 0) {
        st = upload_lengths(x_lengths, y_lengths, B, N, M, lens, s);
        if (st != POINTOPS_OK) return st;
    }
    e = pointops::launch_chamfer_backward(
        x, y, B, N, M, have_len ? lens : nullptr, have_len ? lens + B : nullptr,
        point_reduction == POINTOPS_REDUCE_MEAN, batch_reduction, single_directional != 0,
        idx_xy, idx_yx, grad_loss, grad_x, grad_y, s);
    if (e != hipSuccess) return hip_fail(e, "chamfer backward");
    return POINTOPS_OK;
}

}  // extern "C"
