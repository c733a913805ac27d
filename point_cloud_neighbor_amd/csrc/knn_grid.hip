// Exact k nearest neighbours with spatial culling, for gfx950.
//
// Contract: as the plain kNN kernel (project page "mps-pointops", section "The
// operators in equations", "k nearest neighbors": sort the references by
// (s, j), keep the first k, return sqrt(s); "Numerical contracts", "Selection
// and output": exact ties go to the smaller index). The result does not depend
// on the order in which references are examined, which is what this kernel
// changes: it visits nearby references first and skips far ones, the
// direction the project page's roadmap gives for large clouds (spatial
// structures; uniform grid).
//
// 1. Grid. Each cloud's references and queries are counting-sorted by the
//    Morton code of a uniform grid cell (2^L cells per axis over the
//    references' bounding box). The cell formula only decides the order; no
//    result depends on it.
// 2. Boxes. Every 64 consecutive sorted references form a block with its
//    bounding box, every 64 blocks a superblock with the union box.
// 3. Search. A workgroup holds 64 sorted queries (one per lane) and NW waves.
//    The waves first scan the blocks around the group's own grid position
//    (seeding each lane's list with near neighbours), then test every
//    superblock and, inside a surviving one, every block: a lane needs a box
//    only if the box's lower bound of s32 does not exceed the lane's current
//    k-th distance. The bound is computed from the per-axis gaps with the
//    float32 operations of s32; rounding is monotone, so it never exceeds the
//    s32 of any point in the box, and a box is skipped only when no point in
//    it could enter the final list. Keys are 64-bit, (bits(s) + 1) << 32 |
//    original index, so any visiting order gives the (s, j) order. The waves
//    share their lanes' k-th keys through LDS (the smallest of them bounds the
//    final k-th key too), then merge their lists.
#include <algorithm>

#include "common.h"

namespace pointops {

constexpr int kGridBuf = 16;  // candidate slots per lane (>= 8 + 1)

// ------------------------------------------------------------------ grid build

struct GridParams {
    float lo[3];
    float inv[3];  // cells per unit length
    float pad[2];
};

__device__ __forceinline__ uint32_t spread3(uint32_t v) {
    // bit b of v -> bit 3b
    v &= 0x3FF;
    v = (v | (v << 16)) & 0x030000FF;
    v = (v | (v << 8)) & 0x0300F00F;
    v = (v | (v << 4)) & 0x030C30C3;
    v = (v | (v << 2)) & 0x09249249;
    return v;
}

__device__ __forceinline__ uint32_t cell_code(const GridParams& g, float x, float y, float z,
                                              int L) {
    // clamped in float first, so points outside the box (queries) convert safely
    const float top = (float)((1 << L) - 1);
    const int cx = (int)fminf(fmaxf((x - g.lo[0]) * g.inv[0], 0.0f), top);
    const int cy = (int)fminf(fmaxf((y - g.lo[1]) * g.inv[1], 0.0f), top);
    const int cz = (int)fminf(fmaxf((z - g.lo[2]) * g.inv[2], 0.0f), top);
    return spread3((uint32_t)cx) | (spread3((uint32_t)cy) << 1) | (spread3((uint32_t)cz) << 2);
}

// One workgroup per cloud: the references' bounding box -> cell mapping.
__global__ __launch_bounds__(256) void grid_bounds_kernel(const float* __restrict__ ref, int P,
                                                          int L, GridParams* __restrict__ gp) {
    __shared__ float sh[6][256];
    const int b = blockIdx.x;
    const float* xb = ref + (size_t)b * P * 3;
    const float inf = __builtin_inff();
    float mn[3] = {inf, inf, inf}, mx[3] = {-inf, -inf, -inf};
    for (int j = threadIdx.x; j < P; j += 256)
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            const float v = xb[(size_t)3 * j + d];
            mn[d] = fminf(mn[d], v);
            mx[d] = fmaxf(mx[d], v);
        }
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        sh[d][threadIdx.x] = mn[d];
        sh[3 + d][threadIdx.x] = mx[d];
    }
    __syncthreads();
    for (int s = 128; s >= 1; s /= 2) {
        if ((int)threadIdx.x < s)
#pragma unroll
            for (int d = 0; d < 3; ++d) {
                sh[d][threadIdx.x] = fminf(sh[d][threadIdx.x], sh[d][threadIdx.x + s]);
                sh[3 + d][threadIdx.x] = fmaxf(sh[3 + d][threadIdx.x], sh[3 + d][threadIdx.x + s]);
            }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        GridParams g{};
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            const float ext = sh[3 + d][0] - sh[d][0];
            g.lo[d] = sh[d][0];
            g.inv[d] = ext > 0.0f ? (float)(1 << L) / ext : 0.0f;
        }
        gp[b] = g;
    }
}

__global__ void grid_zero_kernel(uint32_t* __restrict__ p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// Histogram of cell codes: cnt[b * C + code]++.
__global__ void grid_count_kernel(const float* __restrict__ pts, int64_t B, int n, int L,
                                  const GridParams* __restrict__ gp, uint32_t* __restrict__ cnt) {
    const int64_t C = (int64_t)1 << (3 * L);
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < B * n;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = e / n;
        const float* p = pts + e * 3;
        atomicAdd(&cnt[b * C + cell_code(gp[b], p[0], p[1], p[2], L)], 1u);
    }
}

// One workgroup per cloud: exclusive scan of its C counts in place; `fill`
// (the scatter cursors) is cleared.
__global__ __launch_bounds__(1024) void grid_scan_kernel(uint32_t* __restrict__ cnt,
                                                         uint32_t* __restrict__ fill, int L) {
    __shared__ uint32_t part[1024];
    const int64_t C = (int64_t)1 << (3 * L);
    uint32_t* c = cnt + (int64_t)blockIdx.x * C;
    uint32_t* f = fill + (int64_t)blockIdx.x * C;
    const int64_t per = (C + 1023) / 1024;
    const int64_t a = threadIdx.x * per, e = min(C, a + per);
    uint32_t s = 0;
    for (int64_t i = a; i < e; ++i) s += c[i];
    part[threadIdx.x] = s;
    __syncthreads();
    // Hillis-Steele inclusive scan of the 1024 partial sums
    for (int o = 1; o < 1024; o *= 2) {
        const uint32_t v = (int)threadIdx.x >= o ? part[threadIdx.x - o] : 0u;
        __syncthreads();
        part[threadIdx.x] += v;
        __syncthreads();
    }
    uint32_t run = threadIdx.x ? part[threadIdx.x - 1] : 0u;
    for (int64_t i = a; i < e; ++i) {
        const uint32_t v = c[i];
        c[i] = run;
        f[i] = 0;
        run += v;
    }
}

// Sorted copy: out[b * n + start[code] + k] = (x, y, z, original index).
__global__ void grid_scatter_kernel(const float* __restrict__ pts, int64_t B, int n, int L,
                                    const GridParams* __restrict__ gp,
                                    const uint32_t* __restrict__ start, uint32_t* __restrict__ fill,
                                    float4* __restrict__ out) {
    const int64_t C = (int64_t)1 << (3 * L);
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < B * n;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = e / n;
        const int j = (int)(e - b * n);
        const float* p = pts + e * 3;
        const uint32_t code = cell_code(gp[b], p[0], p[1], p[2], L);
        const uint32_t pos = start[b * C + code] + atomicAdd(&fill[b * C + code], 1u);
        out[b * n + pos] = make_float4(p[0], p[1], p[2], __int_as_float(j));
    }
}

// One wave per block of 64 sorted references: box[(b * nblk + k) * 8 + 0..5].
__global__ __launch_bounds__(256) void grid_boxes_kernel(const float4* __restrict__ sr, int64_t B,
                                                         int P, int nblk,
                                                         float* __restrict__ box) {
    const int64_t w = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (w >= B * nblk) return;
    const int64_t b = w / nblk;
    const int k = (int)(w - b * nblk);
    const int j = k * kWave + lane;
    const float inf = __builtin_inff();
    float v[6] = {inf, inf, inf, -inf, -inf, -inf};
    if (j < P) {
        const float4 p = sr[b * P + j];
        v[0] = v[3] = p.x;
        v[1] = v[4] = p.y;
        v[2] = v[5] = p.z;
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o /= 2)
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            v[d] = fminf(v[d], __shfl_xor(v[d], o));
            v[3 + d] = fmaxf(v[3 + d], __shfl_xor(v[3 + d], o));
        }
    if (lane == 0) {
        float* o = box + (size_t)w * 8;
#pragma unroll
        for (int d = 0; d < 6; ++d) o[d] = v[d];
    }
}

// One wave per superblock (64 blocks): the union of its blocks' boxes.
__global__ __launch_bounds__(256) void grid_superboxes_kernel(const float* __restrict__ box,
                                                              int64_t B, int nblk, int nsb,
                                                              float* __restrict__ sbox) {
    const int64_t w = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (w >= B * nsb) return;
    const int64_t b = w / nsb;
    const int s = (int)(w - b * nsb);
    const int k = s * kWave + lane;
    const float inf = __builtin_inff();
    float v[6] = {inf, inf, inf, -inf, -inf, -inf};
    if (k < nblk) {
        const float* o = box + ((size_t)b * nblk + k) * 8;
#pragma unroll
        for (int d = 0; d < 6; ++d) v[d] = o[d];
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o /= 2)
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            v[d] = fminf(v[d], __shfl_xor(v[d], o));
            v[3 + d] = fmaxf(v[3 + d], __shfl_xor(v[3 + d], o));
        }
    if (lane == 0) {
        float* o = sbox + (size_t)w * 8;
#pragma unroll
        for (int d = 0; d < 6; ++d) o[d] = v[d];
    }
}

// ------------------------------------------------------------------ search

template <int KCAP>
struct TopK64 {
    uint64_t key[KCAP];  // ascending; front sentinels 0, empty slots ~0

    __device__ __forceinline__ void init(int k) {
#pragma unroll
        for (int p = 0; p < KCAP; ++p) key[p] = p < KCAP - k ? 0ull : ~0ull;
    }

    // Insert kk (~0 inserts nothing); the largest key drops out.
    __device__ __forceinline__ void insert(uint64_t kk) {
#pragma unroll
        for (int p = KCAP - 1; p >= 1; --p) {
            const uint64_t hi = key[p - 1] > kk ? key[p - 1] : kk;
            key[p] = hi < key[p] ? hi : key[p];
        }
        key[0] = kk < key[0] ? kk : key[0];
    }

    __device__ __forceinline__ uint32_t last_hi() const { return (uint32_t)(key[KCAP - 1] >> 32); }
};

// Lower bound of s32 between a point and a box (see the file comment).
__device__ __forceinline__ float box_bound(const float* __restrict__ o, float qx, float qy,
                                           float qz) {
    const float gx = fmaxf(fmaxf(o[0] - qx, qx - o[3]), 0.0f);
    const float gy = fmaxf(fmaxf(o[1] - qy, qy - o[4]), 0.0f);
    const float gz = fmaxf(fmaxf(o[2] - qz, qz - o[5]), 0.0f);
    return (gx * gx + gy * gy) + gz * gz;
}

template <int KCAP, int NW>
__global__ __launch_bounds__(NW* kWave) void knn_grid_kernel(
    const float4* __restrict__ sq, const float4* __restrict__ sr, int Q, int P, int k,
    const float* __restrict__ box, const float* __restrict__ sbox, int nblk, int nsb,
    const uint32_t* __restrict__ ref_start, const GridParams* __restrict__ gp, int L,
    float* __restrict__ out_dist, int64_t* __restrict__ out_idx) {
    constexpr int ROWS = kGridBuf > KCAP ? kGridBuf : KCAP;
    extern __shared__ uint2 lds[];             // per wave ROWS x 64 entries
    __shared__ uint32_t thr[NW][kWave];        // each wave's lanes' k-th key (high half)

    const int b = blockIdx.y;
    const int lane = threadIdx.x % kWave;
    const int w = uniform((int)(threadIdx.x / kWave));
    const int qi = blockIdx.x * kWave + lane;
    const bool qvalid = qi < Q;
    const float4 q = sq[(size_t)b * Q + (qvalid ? qi : Q - 1)];
    const float4* rb = sr + (size_t)b * P;
    const float* bx = box + (size_t)b * nblk * 8;
    const float* sbx = sbox + (size_t)b * nsb * 8;
    uint2* buf = lds + (size_t)w * ROWS * kWave;

    TopK64<KCAP> top;
    top.init(k);
    // a lane without a query takes nothing
    uint32_t lim = qvalid ? 0xFFFFFFFFu : 0u;  // accept key high half u <= lim
    thr[w][lane] = lim;
    int cnt = 0;

    auto flush = [&]() {
        const int rounds = wave_max_i32(cnt);
#pragma unroll 1
        for (int e = 0; e < rounds; ++e) {
            const uint2 c = buf[e * kWave + lane];
            top.insert(e < cnt ? ((uint64_t)c.x << 32) | c.y : ~0ull);
        }
        cnt = 0;
        const uint32_t t = top.last_hi();
        lim = min(lim, t);
        __hip_atomic_store(&thr[w][lane], lim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    // the tightest k-th key of any wave bounds the final one
    auto refresh = [&]() {
#pragma unroll
        for (int v = 0; v < NW; ++v)
            lim = min(lim, __hip_atomic_load(&thr[v][lane], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_WORKGROUP));
    };
    auto scan_block = [&](int blk) {
        const int j0 = blk * kWave, j1 = min(P, j0 + kWave);
        int j = j0;
        for (; j + 8 <= j1; j += 8) {
            uint32_t u[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float4 p = rb[j + r];
                u[r] = f2u(s32(q.x, q.y, q.z, p.x, p.y, p.z)) + 1u;
            }
            uint32_t mn = u[0];
#pragma unroll
            for (int r = 1; r < 8; ++r) mn = min(mn, u[r]);
            if (ballot(mn <= lim)) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    if (u[r] <= lim) {
                        buf[cnt * kWave + lane] =
                            make_uint2(u[r], (uint32_t)__float_as_int(rb[j + r].w));
                        ++cnt;
                    }
                }
                if (ballot(cnt > kGridBuf - 8)) flush();
            }
        }
        for (; j < j1; ++j) {
            const float4 p = rb[j];
            const uint32_t u = f2u(s32(q.x, q.y, q.z, p.x, p.y, p.z)) + 1u;
            if (u <= lim) {
                buf[cnt * kWave + lane] = make_uint2(u, (uint32_t)__float_as_int(p.w));
                ++cnt;
            }
            if (ballot(cnt >= kGridBuf)) flush();
        }
        flush();
    };

    // 1. Seed: the NW blocks around the grid position of the group's first query.
    int s0 = 0;
    {
        const float4 q0 = sq[(size_t)b * Q + (size_t)blockIdx.x * kWave];
        const uint32_t code = cell_code(gp[b], q0.x, q0.y, q0.z, L);
        const int64_t C = (int64_t)1 << (3 * L);
        const int home = (int)min<int64_t>(ref_start[(int64_t)b * C + code] / kWave, nblk - 1);
        s0 = max(0, min(home - NW / 2, nblk - NW));
    }
    const int seed_end = min(nblk, s0 + NW);
    if (s0 + w < seed_end) scan_block(s0 + w);
    __syncthreads();
    refresh();

    // 2. Every superblock whose box some lane still needs; inside it, the
    //    blocks of this wave (block % NW == w) whose box some lane needs.
    for (int s = 0; s < nsb; ++s) {
        const float* so = sbx + (size_t)s * 8;
        if (ballot(f2u(box_bound(so, q.x, q.y, q.z)) + 1u <= lim) == 0) continue;
        const int first = s * kWave, end = min(nblk, first + kWave);
        for (int blk = first + (w - first % NW + NW) % NW; blk < end; blk += NW) {
            if (blk >= s0 && blk < seed_end) continue;
            const float* o = bx + (size_t)blk * 8;
            if (ballot(f2u(box_bound(o, q.x, q.y, q.z)) + 1u <= lim) == 0) continue;
            scan_block(blk);
            refresh();
        }
    }

    // 3. Merge the NW lists (tree over LDS rows), then write rows in query order.
    if (NW > 1) {
#pragma unroll
        for (int p = 0; p < KCAP; ++p)
            buf[p * kWave + lane] = make_uint2((uint32_t)top.key[p], (uint32_t)(top.key[p] >> 32));
#pragma unroll
        for (int d = 1; d < NW; d *= 2) {
            __syncthreads();
            if (w % (2 * d) == 0) {
                const uint2* other = lds + (size_t)(w + d) * ROWS * kWave;
#pragma unroll 1
                for (int p = 0; p < KCAP; ++p) {
                    const uint2 c = other[p * kWave + lane];
                    const uint64_t kk = ((uint64_t)c.y << 32) | c.x;
                    top.insert(kk != 0ull ? kk : ~0ull);  // front sentinels insert nothing
                }
                if (2 * d < NW) {
#pragma unroll
                    for (int p = 0; p < KCAP; ++p)
                        buf[p * kWave + lane] =
                            make_uint2((uint32_t)top.key[p], (uint32_t)(top.key[p] >> 32));
                }
            }
        }
        if (w != 0) return;
    }
    if (!qvalid) return;
    const int64_t row = (int64_t)b * Q + __float_as_int(q.w);
    float* od = out_dist + row * k;
    int64_t* oi = out_idx + row * k;
    const int front = KCAP - k;
#pragma unroll
    for (int p = 0; p < KCAP; ++p) {
        if (p >= front) {
            od[p - front] = sqrtf(u2f((uint32_t)(top.key[p] >> 32) - 1u));
            oi[p - front] = (int64_t)(uint32_t)top.key[p];
        }
    }
}

// ------------------------------------------------------------------ host side

int knn_grid_level(int64_t P) {
    // about four references per cell, 2..7 bits per axis
    int L = 2;
    while (L < 7 && ((int64_t)1 << (3 * (L + 1))) * 4 <= P) ++L;
    return L;
}

struct GridLayout {
    size_t params, ref_cnt, ref_fill, q_cnt, q_fill, sref, squery, box, sbox, total;
};

static size_t al(size_t n) { return (n + 255) / 256 * 256; }

static GridLayout grid_layout(int64_t B, int64_t Q, int64_t P) {
    const int L = knn_grid_level(P);
    const size_t C = (size_t)1 << (3 * L);
    const int64_t nblk = (P + kWave - 1) / kWave, nsb = (nblk + kWave - 1) / kWave;
    GridLayout g;
    size_t o = 0;
    g.params = o; o += al(B * sizeof(GridParams));
    g.ref_cnt = o; o += al(B * C * 4);
    g.ref_fill = o; o += al(B * C * 4);
    g.q_cnt = o; o += al(B * C * 4);
    g.q_fill = o; o += al(B * C * 4);
    g.sref = o; o += al(B * P * sizeof(float4));
    g.squery = o; o += al(B * Q * sizeof(float4));
    g.box = o; o += al(B * nblk * 8 * sizeof(float));
    g.sbox = o; o += al(B * nsb * 8 * sizeof(float));
    g.total = o;
    return g;
}

size_t knn_grid_workspace_bytes(int64_t B, int64_t Q, int64_t P) {
    return grid_layout(B, Q, P).total;
}

static unsigned grid_blocks(int64_t n) {
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 8192));
}

hipError_t launch_knn_grid(const float* query, const float* ref, int64_t B, int64_t Q, int64_t P,
                           int64_t k, float* out_dist, int64_t* out_idx, int kcap, int nw,
                           void* workspace, hipStream_t stream) {
    const int L = knn_grid_level(P);
    const int64_t C = (int64_t)1 << (3 * L);
    const int nblk = (int)((P + kWave - 1) / kWave), nsb = (nblk + kWave - 1) / kWave;
    const GridLayout g = grid_layout(B, Q, P);
    char* ws = (char*)workspace;
    GridParams* gp = (GridParams*)(ws + g.params);
    uint32_t* rcnt = (uint32_t*)(ws + g.ref_cnt);
    uint32_t* rfill = (uint32_t*)(ws + g.ref_fill);
    uint32_t* qcnt = (uint32_t*)(ws + g.q_cnt);
    uint32_t* qfill = (uint32_t*)(ws + g.q_fill);
    float4* sref = (float4*)(ws + g.sref);
    float4* squery = (float4*)(ws + g.squery);
    float* box = (float*)(ws + g.box);
    float* sbox = (float*)(ws + g.sbox);
    hipError_t e;
#define POINTOPS_CHECK(x) \
    do {                   \
        x;                 \
        e = hipGetLastError(); \
        if (e != hipSuccess) return e; \
    } while (0)
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_bounds_kernel, dim3((unsigned)B), dim3(256), 0, stream,
                                      ref, (int)P, L, gp));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_zero_kernel, dim3(grid_blocks(B * C)), dim3(256), 0,
                                      stream, rcnt, (size_t)(B * C)));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_zero_kernel, dim3(grid_blocks(B * C)), dim3(256), 0,
                                      stream, qcnt, (size_t)(B * C)));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_count_kernel, dim3(grid_blocks(B * P)), dim3(256), 0,
                                      stream, ref, B, (int)P, L, gp, rcnt));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_count_kernel, dim3(grid_blocks(B * Q)), dim3(256), 0,
                                      stream, query, B, (int)Q, L, gp, qcnt));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_scan_kernel, dim3((unsigned)B), dim3(1024), 0, stream,
                                      rcnt, rfill, L));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_scan_kernel, dim3((unsigned)B), dim3(1024), 0, stream,
                                      qcnt, qfill, L));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_scatter_kernel, dim3(grid_blocks(B * P)), dim3(256), 0,
                                      stream, ref, B, (int)P, L, gp, rcnt, rfill, sref));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_scatter_kernel, dim3(grid_blocks(B * Q)), dim3(256), 0,
                                      stream, query, B, (int)Q, L, gp, qcnt, qfill, squery));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_boxes_kernel, dim3((unsigned)((B * nblk + 3) / 4)),
                                      dim3(256), 0, stream, sref, B, (int)P, nblk, box));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_superboxes_kernel, dim3((unsigned)((B * nsb + 3) / 4)),
                                      dim3(256), 0, stream, box, B, nblk, nsb, sbox));
    dim3 grid((unsigned)((Q + kWave - 1) / kWave), (unsigned)B);
#define POINTOPS_GRID_CASE(KC, W)                                                              \
    if (kcap == KC && nw == W) {                                                               \
        constexpr int rows = kGridBuf > KC ? kGridBuf : KC;                                    \
        const size_t lds = (size_t)W * rows * kWave * sizeof(uint2);                           \
        if (lds > 65536) {                                                                     \
            e = hipFuncSetAttribute((const void*)knn_grid_kernel<KC, W>,                       \
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);     \
            if (e != hipSuccess) return e;                                                     \
        }                                                                                      \
        POINTOPS_CHECK(hipLaunchKernelGGL((knn_grid_kernel<KC, W>), grid, dim3(W * kWave), lds, \
                                          stream, squery, sref, (int)Q, (int)P, (int)k, box,   \
                                          sbox, nblk, nsb, rcnt, gp, L, out_dist, out_idx));   \
        return hipSuccess;                                                                     \
    }
    POINTOPS_GRID_CASE(1, 4) POINTOPS_GRID_CASE(2, 4) POINTOPS_GRID_CASE(4, 4)
    POINTOPS_GRID_CASE(8, 4) POINTOPS_GRID_CASE(16, 4) POINTOPS_GRID_CASE(32, 4)
    POINTOPS_GRID_CASE(64, 2)
#undef POINTOPS_GRID_CASE
#undef POINTOPS_CHECK
    return hipErrorInvalidValue;
}

}  // namespace pointops
