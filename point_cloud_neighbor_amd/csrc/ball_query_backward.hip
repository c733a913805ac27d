// Ball Query backward for gfx950.
//
// Contract: project page "mps-pointops", section "The operators in equations",
// the two gradient formulas under "Ball Query: first K within a radius", and
// the "Numerical contracts" page, "Differentiation": for each selected slot
// (I >= 0) with G = dL/dS, the query receives 2 G (q - x_I) and the reference
// receives -2 G (q - x_I); contributions to one reference accumulate, in an
// order the contract leaves free.
//
// Mapping. One wave per query row, lane k on slot k (rows with K > 64 take
// several passes). Each lane forms its term t = 2 * (G * fl32(q - x)) (the
// doubling is exact); the query gradient is the sum of the row's terms by a
// fixed DPP tree (deterministic), the reference gradient is accumulated with
// float atomics after the output has been zeroed. Slots whose index is not in
// [0, P) contribute nothing.
#include <algorithm>
#include <cstdlib>

#include "common.h"

namespace pointops {

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float src) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(src), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes by a fixed tree; the total is returned in every lane.
__device__ __forceinline__ float wave_sum_f32(float v) {
    v = v + dpp_f32<kDppQuadSwap1>(v);
    v = v + dpp_f32<kDppQuadSwap2>(v);
    v = v + dpp_f32<kDppRowHalfMirror>(v);
    v = v + dpp_f32<kDppRowMirror>(v);
    v = v + dpp_f32<kDppRowBcast15, 0xA>(v);
    v = v + dpp_f32<kDppRowBcast31, 0xC>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

constexpr int kBqBwdWaves = 4;

// *p += v in LDS, as a float add of the current value retried through an
// integer compare-and-swap. Measured on gfx950 (random addresses in a
// 2048-word array, four waves per workgroup): the LDS float atomic add runs
// at about 0.33 lanes per clock per CU, the integer atomics at 9-12, and this
// loop at 2.6 (4.2 on distinct addresses). Each successful swap applies one
// float32 add (the VALU's: round to nearest even, subnormals kept) to the
// value it replaces, so the result is a sum of the same terms in some order,
// as with the atomic. No retry is needed unless another lane or wave changed
// the word in between.
__device__ __forceinline__ void lds_add_f32(float* p, float v) {
    uint32_t* u = reinterpret_cast<uint32_t*>(p);
    uint32_t old = *u;
    while (true) {
        const uint32_t prev = atomicCAS(u, old, __float_as_uint(__uint_as_float(old) + v));
        if (prev == old) break;
        old = prev;
    }
}

__global__ __launch_bounds__(kBqBwdWaves* kWave) void ball_query_backward_kernel(
    const float* __restrict__ query, const float* __restrict__ ref,
    const int64_t* __restrict__ idx, const float* __restrict__ grad, int64_t rows, int Q,
    int P, int K, float* __restrict__ grad_query, float* __restrict__ grad_ref) {
    const int64_t row = (int64_t)blockIdx.x * kBqBwdWaves + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (row >= rows) return;  // whole waves leave together
    const int64_t b = row / Q;
    const float qx = query[3 * row + 0], qy = query[3 * row + 1], qz = query[3 * row + 2];
    float sx = 0.f, sy = 0.f, sz = 0.f;
    for (int k0 = 0; k0 < K; k0 += kWave) {
        const int k = k0 + lane;
        if (k >= K) continue;
        const int64_t j = idx[row * K + k];
        if (j < 0 || j >= P) continue;
        const float g = grad[row * K + k];
        const float* x = ref + (b * P + j) * 3;
        const float tx = 2.0f * (g * (qx - x[0]));
        const float ty = 2.0f * (g * (qy - x[1]));
        const float tz = 2.0f * (g * (qz - x[2]));
        sx += tx;
        sy += ty;
        sz += tz;
        if (grad_ref) {
            float* o = grad_ref + (b * P + j) * 3;
            unsafeAtomicAdd(o + 0, -tx);
            unsafeAtomicAdd(o + 1, -ty);
            unsafeAtomicAdd(o + 2, -tz);
        }
    }
    if (grad_query) {
        sx = wave_sum_f32(sx);
        sy = wave_sum_f32(sy);
        sz = wave_sum_f32(sz);
        if (lane == 0) {
            grad_query[3 * row + 0] = sx;
            grad_query[3 * row + 1] = sy;
            grad_query[3 * row + 2] = sz;
        }
    }
}

// Reference gradients aggregated per tile of consecutive rows before they
// reach device memory: on a spatially sorted cloud neighbouring rows select
// mostly the same references, so one set of atomics per distinct reference of
// the tile replaces one per selected slot. A workgroup takes `tile` rows (its
// waves a row at a time) and adds each term into LDS, keyed by the
// reference's flat row b * P + j, in two levels: a direct window of kBwdWin
// consecutive flat rows placed on the data (around the middle row's middle
// selection: on a sorted cloud queried by its own points, about 85% of the
// terms), with a bit per entry marking those touched; and for the rest a
// table with open addressing (linear probing, at most kBwdProbes probes; a
// term that finds no slot goes straight to device memory, so the result
// never depends on either size). After a barrier the touched entries go out
// with float atomics. The LDS adds are lds_add_f32's read and swap, not the
// LDS float atomic (see there). On the sorted 100k cloud, K = 64: 0.166 ms
// with the table alone, 0.146 with the window in front of it, 0.139 with the
// self-query mode below, 0.095 with the swapped adds and the rows' loads
// issued kBwdRows at a time. The query gradients are the fixed DPP tree, as
// above.
//
// A cloud queried by its own points (the query and reference buffers are one,
// Q = P) with a workspace: the window of tile t is fixed by its position,
// flat rows [t * tile + tile / 2 - kBwdWin / 2, ... + kBwdWin), and is written
// whole to the workspace (its partial sums, zeros where untouched) instead of
// going out with atomics; a second kernel adds, for each reference, the
// partials of the windows that cover it in tile order. Only the table's
// entries still use atomics. (A reference is covered by kBwdWin / tile
// windows, and on a sorted cloud most of its terms are in them.)
constexpr int kBwdTableBits = 11;
constexpr int kBwdTable = 1 << kBwdTableBits;
constexpr int kBwdProbes = 64;  // probes before a term goes straight to device memory
constexpr int kBwdWin = 2048;   // window entries
constexpr int kBwdRows = 8;     // rows a wave loads at once

__global__ __launch_bounds__(kBqBwdWaves* kWave) void ball_query_backward_tiled_kernel(
    const float* __restrict__ query, const float* __restrict__ ref,
    const int64_t* __restrict__ idx, const float* __restrict__ grad, int64_t rows, int Q,
    int P, int K, int tile, float* __restrict__ grad_query, float* __restrict__ grad_ref,
    float* __restrict__ part) {
    __shared__ int key[kBwdTable];
    __shared__ float ax[kBwdTable], ay[kBwdTable], az[kBwdTable];
    __shared__ float wx[kBwdWin], wy[kBwdWin], wz[kBwdWin];
    __shared__ uint32_t wbits[kBwdWin / 32];
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = uniform((int)(tid / kWave));
    for (int i = tid; i < kBwdTable; i += kBqBwdWaves * kWave) {
        key[i] = -1;
        ax[i] = ay[i] = az[i] = 0.0f;
    }
    for (int i = tid; i < kBwdWin; i += kBqBwdWaves * kWave) wx[i] = wy[i] = wz[i] = 0.0f;
    for (int i = tid; i < kBwdWin / 32; i += kBqBwdWaves * kWave) wbits[i] = 0u;
    const int64_t r0 = (int64_t)blockIdx.x * tile;  // < rows
    // the window: fixed by the tile's position (partials to `part`), or
    // centred on the middle row's middle selection (else its first; none when
    // neither is a reference)
    int64_t wbase = -(int64_t)2 * kBwdWin;
    if (part) {
        wbase = r0 + tile / 2 - kBwdWin / 2;
    } else {
        const int64_t rm = min(r0 + tile / 2, rows - 1);
        int64_t j = idx[rm * K + K / 2];
        if (j < 0 || j >= P) j = idx[rm * K];
        if (j >= 0 && j < P) wbase = (rm / Q) * P + j - kBwdWin / 2;
    }
    __syncthreads();
    // Adds a term: into the window, or the table (a free or matching slot
    // within the table, which holds at most half its size of distinct keys).
    auto add_ref = [&](int flat, float tx, float ty, float tz) {
        const int64_t wi = (int64_t)flat - wbase;
        if (wi >= 0 && wi < kBwdWin) {
            lds_add_f32(&wx[wi], -tx);
            lds_add_f32(&wy[wi], -ty);
            lds_add_f32(&wz[wi], -tz);
            if (!part) atomicOr(&wbits[wi >> 5], 1u << (wi & 31));
            return;
        }
        uint32_t h = ((uint32_t)flat * 2654435761u) >> (32 - kBwdTableBits);  // a slot
        // not unrolled: unrolled, each probe kept its own exec masks in scalar
        // registers, which spilled
#pragma nounroll
        for (int probe = 0; probe < kBwdProbes; ++probe) {
            const int old = atomicCAS(&key[h], -1, flat);
            if (old == -1 || old == flat) {
                lds_add_f32(&ax[h], -tx);
                lds_add_f32(&ay[h], -ty);
                lds_add_f32(&az[h], -tz);
                return;
            }
            h = (h + 1) & (kBwdTable - 1);
        }
        float* o = grad_ref + (size_t)flat * 3;  // no slot within the probes: straight out
        unsafeAtomicAdd(o + 0, -tx);
        unsafeAtomicAdd(o + 1, -ty);
        unsafeAtomicAdd(o + 2, -tz);
    };
    auto finish_row = [&](int64_t row, float sx, float sy, float sz) {
        if (!grad_query) return;
        sx = wave_sum_f32(sx);
        sy = wave_sum_f32(sy);
        sz = wave_sum_f32(sz);
        if (lane == 0) {
            grad_query[3 * row + 0] = sx;
            grad_query[3 * row + 1] = sy;
            grad_query[3 * row + 2] = sz;
        }
    };
    if (K <= kWave && P > 0) {
        // One slot per lane; a wave's rows are r0 + wave, + kBqBwdWaves, ...,
        // taken kBwdRows at a time: the indices and G of all of them are
        // loaded, then the query points and the references they name, then
        // the rows are added in. A wave so waits out two round trips per
        // kBwdRows rows instead of two per row (index, then the reference it
        // names). Every load is issued unconditionally (rows past the tile
        // and lanes past K read a clamped, valid address and are flagged):
        // loads complete in order, so each wait covers exactly the loads it
        // needs, which a load that may be skipped would prevent. The query
        // point goes through a vector load for the same reason (scalar loads
        // complete out of order).
        constexpr int W = kBqBwdWaves;
        const int64_t rend = min(r0 + (int64_t)tile, rows);
        const int kc = lane < K ? lane : K - 1;
        int64_t bg = (r0 + wave) / Q, rqg = (r0 + wave) - bg * Q;  // batch of the next row
        for (int64_t rb = r0 + wave; rb < rend; rb += kBwdRows * W) {
            int64_t j[kBwdRows];
            float g[kBwdRows], x[kBwdRows], y[kBwdRows], z[kBwdRows], qx[kBwdRows],
                qy[kBwdRows], qz[kBwdRows];
            int f[kBwdRows];  // flat reference row, -1 when the slot contributes nothing
            int64_t rowb[kBwdRows];  // the rows' batches (before the loads: no branch among them)
#pragma unroll
            for (int i = 0; i < kBwdRows; ++i) {
                rowb[i] = bg;
                rqg += W;
                while (rqg >= Q) {
                    rqg -= Q;
                    ++bg;
                }
            }
#pragma unroll
            for (int i = 0; i < kBwdRows; ++i) {
                const int64_t r = rb + i * W, rc = r < rend ? r : rend - 1;
                j[i] = idx[rc * K + kc];
                g[i] = grad[rc * K + kc];
            }
#pragma unroll
            for (int i = 0; i < kBwdRows; ++i) {
                const int64_t r = rb + i * W;
                // the row's offset in the tile (< tile; rows may pass 2^31)
                int rv = (int)((r < rend ? r : rend - 1) - r0);
                __asm__("v_mov_b32 %0, %1" : "=v"(rv) : "s"(rv));  // a vector load, see above
                const float* q = query + (size_t)(r0 + rv) * 3;
                qx[i] = q[0];
                qy[i] = q[1];
                qz[i] = q[2];
                // bitwise, not short-circuit: no branch for the compiler to
                // sink the index load into
                const bool ok = (r < rend) & (lane < K) & ((uint64_t)j[i] < (uint64_t)P);
                f[i] = ok ? (int)(rowb[i] * P + j[i]) : -1;
                const float* p = ref + (size_t)(ok ? f[i] : 0) * 3;
                x[i] = p[0];
                y[i] = p[1];
                z[i] = p[2];
            }
#pragma unroll
            for (int i = 0; i < kBwdRows; ++i) {
                const int64_t r = rb + i * W;
                if (r >= rend) break;
                const bool ok = f[i] >= 0;
                const float tx = ok ? 2.0f * (g[i] * (qx[i] - x[i])) : 0.f;
                const float ty = ok ? 2.0f * (g[i] * (qy[i] - y[i])) : 0.f;
                const float tz = ok ? 2.0f * (g[i] * (qz[i] - z[i])) : 0.f;
                // a sum from +0, as for any row (a -0 term leaves +0)
                finish_row(r, 0.f + tx, 0.f + ty, 0.f + tz);
                if (grad_ref && ok) add_ref(f[i], tx, ty, tz);
            }
        }
    } else {
        for (int rr = wave; rr < tile; rr += kBqBwdWaves) {
            const int64_t r = r0 + rr;
            if (r >= rows) break;
            const int64_t b = r / Q;
            const float px = query[3 * r + 0], py = query[3 * r + 1], pz = query[3 * r + 2];
            float sx = 0.f, sy = 0.f, sz = 0.f;
            for (int k0 = 0; k0 < K; k0 += kWave) {
                const int k = k0 + lane;
                if (k >= K) continue;
                const int64_t jj = idx[r * K + k];
                if (jj < 0 || jj >= P) continue;
                const float gg = grad[r * K + k];
                const float* x = ref + (b * P + jj) * 3;
                const float tx = 2.0f * (gg * (px - x[0]));
                const float ty = 2.0f * (gg * (py - x[1]));
                const float tz = 2.0f * (gg * (pz - x[2]));
                sx += tx;
                sy += ty;
                sz += tz;
                if (grad_ref) add_ref((int)(b * P + jj), tx, ty, tz);
            }
            finish_row(r, sx, sy, sz);
        }
    }
    if (!grad_ref) return;
    __syncthreads();
    if (part) {  // the whole window, x then y then z planes
        float* pt = part + (size_t)blockIdx.x * 3 * kBwdWin;
        for (int i = tid; i < kBwdWin; i += kBqBwdWaves * kWave) {
            pt[i] = wx[i];
            pt[kBwdWin + i] = wy[i];
            pt[2 * kBwdWin + i] = wz[i];
        }
    }
    for (int i = tid; i < kBwdWin && !part; i += kBqBwdWaves * kWave) {
        if ((wbits[i >> 5] >> (i & 31)) & 1u) {  // touched: wbase + i is a reference row
            float* o = grad_ref + (size_t)(wbase + i) * 3;
            unsafeAtomicAdd(o + 0, wx[i]);
            unsafeAtomicAdd(o + 1, wy[i]);
            unsafeAtomicAdd(o + 2, wz[i]);
        }
    }
    for (int i = tid; i < kBwdTable; i += kBqBwdWaves * kWave) {
        const int flat = key[i];
        if (flat >= 0) {
            float* o = grad_ref + (size_t)flat * 3;
            unsafeAtomicAdd(o + 0, ax[i]);
            unsafeAtomicAdd(o + 1, ay[i]);
            unsafeAtomicAdd(o + 2, az[i]);
        }
    }
}

// Adds to each reference row f its partials from the fixed windows that cover
// it (tile t covers [t * tile + tile / 2 - kBwdWin / 2, ... + kBwdWin)), in
// tile order; each row has one thread, so no atomics.
__global__ void ball_query_backward_merge_kernel(const float* __restrict__ part, int64_t ntiles,
                                                 int tile, int64_t nref,
                                                 float* __restrict__ grad_ref) {
    for (int64_t f = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; f < nref;
         f += (int64_t)gridDim.x * blockDim.x) {
        const int64_t lo_num = f - kBwdWin / 2 - tile / 2 + 1;  // t >= ceil(lo_num / tile)
        const int64_t t_lo = lo_num <= 0 ? 0 : (lo_num + tile - 1) / tile;
        const int64_t t_hi = min(ntiles - 1, (f + kBwdWin / 2 - tile / 2) / tile);
        float sx = 0.f, sy = 0.f, sz = 0.f;
        for (int64_t t = t_lo; t <= t_hi; ++t) {
            const int64_t i = f - (t * tile + tile / 2 - kBwdWin / 2);  // in [0, kBwdWin)
            const float* pt = part + (size_t)t * 3 * kBwdWin;
            sx += pt[i];
            sy += pt[kBwdWin + i];
            sz += pt[2 * kBwdWin + i];
        }
        grad_ref[3 * f + 0] += sx;
        grad_ref[3 * f + 1] += sy;
        grad_ref[3 * f + 2] += sz;
    }
}

__global__ void zero_f32_kernel(float* __restrict__ p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0.0f;
}

// Zeroes n floats with a fill kernel (not a memset node, so callers can be
// captured into a graph).
hipError_t launch_zero_f32(float* p, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_f32_kernel, dim3(blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

// Rows per tile: about 8192 selected slots (128 rows at K = 64; the sorted
// 100k workload, rows per tile 16 / 32 / 64 / 128 / 256: 0.224 / 0.185 /
// 0.170 / 0.166 / 0.163 ms): a sorted cloud's tile selects a few hundred
// distinct references; a tile with more than the table takes sends the excess
// straight out, so any shape is exact. POINTOPS_BQ_BWD_TILE sets it.
int64_t bq_backward_tile(int64_t K) {
    const char* te = getenv("POINTOPS_BQ_BWD_TILE");
    int64_t tile = std::min<int64_t>(128, std::max<int64_t>(kBqBwdWaves, 8192 / std::max<int64_t>(K, 1)));
    if (te && atol(te) >= kBqBwdWaves && atol(te) <= 1024) tile = atol(te);
    return tile;
}

// Workspace of the self-query mode: one window of partials (3 planes) per tile.
size_t bq_backward_workspace_bytes(int64_t B, int64_t Q, int64_t K) {
    const int64_t tile = bq_backward_tile(K);
    const int64_t ntiles = (B * Q + tile - 1) / tile;
    return (size_t)ntiles * 3 * kBwdWin * sizeof(float);
}

hipError_t launch_ball_query_backward(const float* query, const float* ref, const int64_t* idx,
                                      const float* grad, int64_t B, int64_t Q, int64_t P,
                                      int64_t K, float* grad_query, float* grad_ref,
                                      void* workspace, hipStream_t stream) {
    if (grad_ref && B * P > 0) {
        hipError_t e = launch_zero_f32(grad_ref, (size_t)B * P * 3, stream);
        if (e != hipSuccess) return e;
    }
    const int64_t rows = B * Q;
    const int64_t tile = bq_backward_tile(K);
    if (B * P < ((int64_t)1 << 31)) {
        const unsigned blocks = (unsigned)((rows + tile - 1) / tile);
        // the self-query mode: the caller's workspace holds the windows
        float* part = workspace && grad_ref && query == ref && Q == P && rows > 0
                          ? (float*)workspace
                          : nullptr;
        hipLaunchKernelGGL(ball_query_backward_tiled_kernel, dim3(blocks),
                           dim3(kBqBwdWaves * kWave), 0, stream, query, ref, idx, grad, rows,
                           (int)Q, (int)P, (int)K, (int)tile, grad_query, grad_ref, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || !part) return e;
        const int64_t nref = B * P;
        hipLaunchKernelGGL(ball_query_backward_merge_kernel,
                           dim3((unsigned)std::min<int64_t>((nref + 255) / 256, 8192)), dim3(256),
                           0, stream, part, (int64_t)blocks, (int)tile, nref, grad_ref);
        return hipGetLastError();
    }
    const unsigned blocks = (unsigned)((rows + kBqBwdWaves - 1) / kBqBwdWaves);
    hipLaunchKernelGGL(ball_query_backward_kernel, dim3(blocks), dim3(kBqBwdWaves * kWave), 0,
                       stream, query, ref, idx, grad, rows, (int)Q, (int)P, (int)K, grad_query,
                       grad_ref);
    return hipGetLastError();
}

}  // namespace pointops
