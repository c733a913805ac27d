// Squared-L2 Chamfer distance for gfx950: the reductions and the gradients.
// The nearest points themselves come from the kNN kernel (k = 1, squared
// distances kept).
//
// Contract: project page "mps-pointops", roadmap "Phase 4" (a(i) = the nearest
// point of y to x_i, b(j) = the nearest of x to y_j; the un-reduced loss sums
// |x_i - y_a(i)|^2 and |y_j - x_b(j)|^2; the gradient of each term goes to
// both of its points) and the reductions its Chamfer contract names (lengths
// mask padded points; a point mean divides each direction's sum by the
// cloud's length, a batch mean by the number of clouds).
//
// Reduction: one workgroup per cloud adds its squared distances in float64 in
// a fixed order (per-thread strided sums, then a tree), so the loss is
// deterministic and within a rounding or two of the exact sum of the float32
// distances. Gradients: one thread per point and direction forms its term
// 2 w (p - o) in float32, with w = fl32(upstream gradient x reduction factor),
// and adds it to its own point and its negation to its nearest point with
// float atomics (order not fixed).
#include <algorithm>

#include "common.h"

namespace pointops {

constexpr int kChamferThreads = 256;
constexpr int kChamferChunk = 1024;  // rows per workgroup of the loss's first stage

// Rows i >= len[b] of a (B, n) nearest-point output are set to (0, -1).
__global__ void chamfer_pad_kernel(float* __restrict__ d, int64_t* __restrict__ idx, int64_t B,
                                   int64_t n, const int64_t* __restrict__ len) {
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < B * n;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = e / n;
        if (e - b * n >= len[b]) {
            d[e] = 0.0f;
            idx[e] = -1;
        }
    }
}

__device__ __forceinline__ double block_sum_f64(double v, double* sh) {
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
#pragma unroll
    for (int w = kChamferThreads / 2; w >= 1; w /= 2) {
        if (t < w) sh[t] += sh[t + w];
        __syncthreads();
    }
    const double r = sh[0];
    __syncthreads();
    return r;
}

// Stage 1: workgroup b * nchunk + c sums rows [c * chunk, (c + 1) * chunk) of
// cloud b below the lengths, in float64, for both directions:
// part[(b * nchunk + c) * 2 + {0, 1}].
__global__ __launch_bounds__(kChamferThreads) void chamfer_reduce_kernel(
    const float* __restrict__ d_xy, const float* __restrict__ d_yx, int64_t N, int64_t M,
    const int64_t* __restrict__ lx, const int64_t* __restrict__ ly, int single, int64_t nchunk,
    int64_t chunk, double* __restrict__ part) {
    __shared__ double sh[kChamferThreads];
    const int64_t b = blockIdx.x / nchunk, c = blockIdx.x - b * nchunk;
    const int64_t nx = lx ? lx[b] : N, ny = ly ? ly[b] : M;
    const int64_t i0 = c * chunk, i1x = std::min(nx, i0 + chunk), i1y = std::min(ny, i0 + chunk);
    double sx = 0.0, sy = 0.0;
    for (int64_t i = i0 + threadIdx.x; i < i1x; i += kChamferThreads) sx += (double)d_xy[b * N + i];
    if (!single)
        for (int64_t j = i0 + threadIdx.x; j < i1y; j += kChamferThreads) sy += (double)d_yx[b * M + j];
    sx = block_sum_f64(sx, sh);
    sy = block_sum_f64(sy, sh);
    if (threadIdx.x == 0) {
        part[(b * nchunk + c) * 2 + 0] = sx;
        part[(b * nchunk + c) * 2 + 1] = sy;
    }
}

// Stage 2, one workgroup, every order fixed (the same bits on every call):
// cloud b's value is fx_b * sum_{i < lx_b} d_xy[b, i] + fy_b * sum_{j < ly_b}
// d_yx[b, j] (the second term unless single-directional), its chunk sums added
// in chunk order, f = 1 / max(len, 1) for a point mean, 1 for a sum, and / B for
// a batch mean; loss[b] = that value (no batch reduction) or loss[0] = the sum
// over the clouds.
__global__ __launch_bounds__(kChamferThreads) void chamfer_finish_kernel(
    const double* __restrict__ part, int64_t B, int64_t N, int64_t M,
    const int64_t* __restrict__ lx, const int64_t* __restrict__ ly, int point_mean,
    int batch_mean, int single, int reduce_batch, int64_t nchunk, float* __restrict__ loss) {
    __shared__ double sh[kChamferThreads];
    double s = 0.0;
    for (int64_t b = threadIdx.x; b < B; b += kChamferThreads) {
        double sx = 0.0, sy = 0.0;
        for (int64_t c = 0; c < nchunk; ++c) {
            sx += part[(b * nchunk + c) * 2 + 0];
            sy += part[(b * nchunk + c) * 2 + 1];
        }
        const int64_t nx = lx ? lx[b] : N, ny = ly ? ly[b] : M;
        const double fx = point_mean ? 1.0 / (double)std::max<int64_t>(nx, 1) : 1.0;
        const double fy = point_mean ? 1.0 / (double)std::max<int64_t>(ny, 1) : 1.0;
        double v = fx * sx + (single ? 0.0 : fy * sy);
        if (batch_mean) v /= (double)B;
        if (reduce_batch)
            s += v;
        else
            loss[b] = (float)v;
    }
    if (!reduce_batch) return;
    s = block_sum_f64(s, sh);
    if (threadIdx.x == 0) loss[0] = (float)s;
}

// One thread per (cloud, point) of x, then of y (unless single-directional).
__global__ void chamfer_backward_kernel(
    const float* __restrict__ x, const float* __restrict__ y, int64_t B, int64_t N, int64_t M,
    const int64_t* __restrict__ lx, const int64_t* __restrict__ ly, int point_mean,
    int batch_reduction, int single, const int64_t* __restrict__ i_xy,
    const int64_t* __restrict__ i_yx, const float* __restrict__ grad_loss,
    float* __restrict__ gx, float* __restrict__ gy) {
    const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int64_t nx_all = B * N, total = nx_all + (single ? 0 : B * M);
    if (e >= total) return;
    const bool side_x = e < nx_all;
    const int64_t n = side_x ? N : M, m = side_x ? M : N;
    const int64_t b = (side_x ? e : e - nx_all) / n;
    const int64_t i = (side_x ? e : e - nx_all) - b * n;
    const int64_t len = side_x ? (lx ? lx[b] : N) : (ly ? ly[b] : M);
    if (i >= len) return;
    const int64_t j = (side_x ? i_xy : i_yx)[b * n + i];
    if (j < 0 || j >= m) return;
    const float* p = (side_x ? x : y) + (b * n + i) * 3;
    const float* o = (side_x ? y : x) + (b * m + j) * 3;
    float* gp = side_x ? gx : gy;
    float* go = side_x ? gy : gx;
    // reduce_batch: 0 none (one upstream gradient per cloud), 1 mean, 2 sum
    const double g = (double)grad_loss[batch_reduction == 0 ? b : 0];
    double f = point_mean ? 1.0 / (double)std::max<int64_t>(len, 1) : 1.0;
    if (batch_reduction == 1) f /= (double)B;
    const float w = (float)(g * f);
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        const float t = 2.0f * (w * (p[d] - o[d]));
        if (gp) unsafeAtomicAdd(gp + (b * n + i) * 3 + d, t);
        if (go) unsafeAtomicAdd(go + (b * m + j) * 3 + d, -t);
    }
}

hipError_t launch_chamfer_pad(float* d, int64_t* idx, int64_t B, int64_t n, const int64_t* len,
                              hipStream_t stream) {
    const int64_t total = B * n;
    if (total == 0) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(chamfer_pad_kernel, dim3(blocks), dim3(256), 0, stream, d, idx, B, n, len);
    return hipGetLastError();
}

// Chunks of the loss's first stage: about kChamferChunk rows each, at most 2^30
// workgroups in all.
int64_t chamfer_chunks(int64_t B, int64_t N, int64_t M) {
    const int64_t rows = std::max<int64_t>(std::max(N, M), 1);
    const int64_t cap = std::max<int64_t>(1, ((int64_t)1 << 30) / std::max<int64_t>(B, 1));
    return std::min((rows + kChamferChunk - 1) / kChamferChunk, cap);
}

hipError_t launch_chamfer_reduce(const float* d_xy, const float* d_yx, int64_t B, int64_t N,
                                 int64_t M, const int64_t* lx, const int64_t* ly, int point_mean,
                                 int batch_reduction, int single, double* part, float* loss,
                                 hipStream_t stream) {
    const int64_t nchunk = chamfer_chunks(B, N, M);
    const int64_t rows = std::max<int64_t>(std::max(N, M), 1);
    const int64_t chunk = (rows + nchunk - 1) / nchunk;
    if (B > 0) {
        hipLaunchKernelGGL(chamfer_reduce_kernel, dim3((unsigned)(B * nchunk)),
                           dim3(kChamferThreads), 0, stream, d_xy, d_yx, N, M, lx, ly, single,
                           nchunk, chunk, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(chamfer_finish_kernel, dim3(1), dim3(kChamferThreads), 0, stream, part, B,
                       N, M, lx, ly, point_mean, batch_reduction == 1 ? 1 : 0, single,
                       batch_reduction != 0 ? 1 : 0, nchunk, loss);
    return hipGetLastError();
}

hipError_t launch_chamfer_backward(const float* x, const float* y, int64_t B, int64_t N,
                                   int64_t M, const int64_t* lx, const int64_t* ly,
                                   int point_mean, int batch_reduction, int single,
                                   const int64_t* i_xy, const int64_t* i_yx,
                                   const float* grad_loss, float* gx, float* gy,
                                   hipStream_t stream) {
    const int64_t total = B * N + (single ? 0 : B * M);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(chamfer_backward_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                       0, stream, x, y, B, N, M, lx, ly, point_mean, batch_reduction, single,
                       i_xy, i_yx, grad_loss, gx, gy);
    return hipGetLastError();
}

}  // namespace pointops
