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
// 2. Boxes. Every 16 consecutive sorted references form a block with its
//    bounding box, every 64 blocks a superblock with the union box.
//    (Steps 1 and 2 are launch_grid_build, shared with the Ball Query grid
//    pass; grid.h holds the helpers both searches use.)
// 3. Search. A workgroup holds 64 sorted queries (one per lane) and NW waves.
//    Wave 0 first inserts, for every lane, the 64 references around the
//    lane's own grid position in sorted order (most of its k nearest are
//    there), so each lane's limit is tight before any box is tested. The
//    waves then test every superblock and,
//    inside a surviving one, every block: a lane needs a box only if the
//    box's lower bound of s32 does not exceed the lane's current k-th
//    distance. The bound is computed from the per-axis gaps with the
//    float32 operations of s32; rounding is monotone, so it never exceeds the
//    s32 of any point in the box, and a box is skipped only when no point in
//    it could enter the final list. Keys are 64-bit, (bits(s) + 1) << 32 |
//    original index, so any visiting order gives the (s, j) order. The waves
//    share their lanes' k-th keys through LDS (the smallest of them bounds the
//    final k-th key too), then merge their lists.
#include <algorithm>

#include "common.h"
#include "grid.h"
#include "wave_list.h"

namespace pointops {

constexpr int kGridBuf = 16;    // candidate slots per lane; at most 8 in use between groups of 8
constexpr int kGridLocal = 64;  // references around each query's own position, scanned first

// ------------------------------------------------------------------ grid build

// The references' bounding box: many workgroups fold their points in with
// integer atomics on an order-preserving encoding of the floats; the last
// workgroup of a cloud to finish turns the box into the cell mapping.
constexpr int kEncWords = 8;  // per cloud: 3 minima, 3 maxima, a finish counter, unused

__device__ __forceinline__ uint32_t ord_enc(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // unsigned order = float order
}

__device__ __forceinline__ float ord_dec(uint32_t e) {
    return __uint_as_float((e & 0x80000000u) ? (e & 0x7FFFFFFFu) : ~e);
}

// Clears the histograms (n words from `zero`) and sets every cloud's box
// slots to the empty box and its counter to 0.
__global__ void grid_init_kernel(uint32_t* __restrict__ enc, int64_t B,
                                 uint32_t* __restrict__ zero, size_t n,
                                 const uint32_t* __restrict__ gate) {
    if (gate && *gate == 0) return;  // the grid is not needed
    const size_t i0 = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    if (i0 < (size_t)B * kEncWords) {
        const int r = (int)(i0 % kEncWords);
        enc[i0] = r < 3 ? 0xFFFFFFFFu : 0u;  // min slots high, max slots and counter 0
    }
    for (size_t i = i0; i < n; i += (size_t)gridDim.x * blockDim.x) zero[i] = 0;
}

__global__ __launch_bounds__(256) void grid_bounds_kernel(const float* __restrict__ ref, int64_t B,
                                                          int P, int L, uint32_t* __restrict__ enc,
                                                          GridParams* __restrict__ gp,
                                                          const uint32_t* __restrict__ gate,
                                                          const int64_t* __restrict__ clouds) {
    if (gate && *gate == 0) return;  // the grid is not needed
    __shared__ uint32_t sh[6];
    __shared__ bool last;
    const int b = blockIdx.y;
    const float* xb = ref + (clouds ? clouds[kGcWords * b + kGcROff] : (int64_t)b * P) * 3;
    if (clouds) P = (int)clouds[kGcWords * b + kGcRCnt];
    uint32_t* e = enc + (size_t)b * kEncWords;
    if (threadIdx.x < 6) sh[threadIdx.x] = threadIdx.x < 3 ? 0xFFFFFFFFu : 0u;
    __syncthreads();
    uint32_t mn[3] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu}, mx[3] = {0u, 0u, 0u};
    for (int j = blockIdx.x * 256 + threadIdx.x; j < P; j += gridDim.x * 256)
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            const uint32_t v = ord_enc(xb[(size_t)3 * j + d]);
            mn[d] = min(mn[d], v);
            mx[d] = max(mx[d], v);
        }
    // wave reductions first (DPP), then one LDS atomic per wave and value
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        mn[d] = ~wave_max_u32(~mn[d]);
        mx[d] = wave_max_u32(mx[d]);
    }
    if (threadIdx.x % kWave == 0) {
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            atomicMin(&sh[d], mn[d]);
            atomicMax(&sh[3 + d], mx[d]);
        }
    }
    __syncthreads();
    if (threadIdx.x < 3) atomicMin(&e[threadIdx.x], sh[threadIdx.x]);
    else if (threadIdx.x < 6) atomicMax(&e[threadIdx.x], sh[threadIdx.x]);
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();  // this workgroup's box atomics before its count
        last = atomicAdd(&e[6], 1u) == gridDim.x - 1;
    }
    __syncthreads();
    if (last && threadIdx.x == 0) {
        __threadfence();
        GridParams g{};
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            // atomic reads: the other workgroups' updates are in the device-scope values
            const float lo = ord_dec(atomicOr(&e[d], 0u));
            const float hi = ord_dec(atomicOr(&e[3 + d], 0u));
            const float ext = hi - lo;
            g.lo[d] = lo;
            g.inv[d] = ext > 0.0f ? (float)(1 << L) / ext : 0.0f;
        }
        gp[b] = g;
    }
}

// Histograms of cell codes, references then queries: cnt[b * C + code]++.
__global__ void grid_count_kernel(const float* __restrict__ ref, const float* __restrict__ query,
                                  int64_t B, int P, int Q, int L,
                                  const GridParams* __restrict__ gp, uint32_t* __restrict__ rcnt,
                                  uint32_t* __restrict__ qcnt, const uint32_t* __restrict__ gate,
                                  const int64_t* __restrict__ clouds) {
    if (gate && *gate == 0) return;  // the grid is not needed
    const int64_t C = (int64_t)1 << (3 * L);
    const int64_t nr = B * P;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < nr + B * Q;
         e += (int64_t)gridDim.x * blockDim.x) {
        const bool is_ref = e < nr;
        const int64_t i = is_ref ? e : e - nr;
        const int64_t n = is_ref ? P : Q;
        const int64_t b = i / n;
        int64_t row = i;
        if (clouds) {  // slot i - b * n of cloud b, if the cloud has that many points
            const int64_t loc = i - b * n;
            if (loc >= clouds[kGcWords * b + (is_ref ? kGcRCnt : kGcQCnt)]) continue;
            row = clouds[kGcWords * b + (is_ref ? kGcROff : kGcQOff)] + loc;
        }
        const float* p = (is_ref ? ref : query) + row * 3;
        atomicAdd(&(is_ref ? rcnt : qcnt)[b * C + cell_code(gp[b], p[0], p[1], p[2], L)], 1u);
    }
}

// Exclusive scan of each cloud's C counts in place, in chunks of 1024 bins:
// first the sum of every chunk, then each chunk adds the sums before it to
// its own scan. `fill` (the scatter cursors) is cleared on the way.
constexpr int kScanChunk = 1024;

// blockIdx.z: 0 references, 1 queries (each side its own counts and sums).
__global__ __launch_bounds__(256) void grid_chunk_sums_kernel(const uint32_t* __restrict__ rcnt,
                                                              const uint32_t* __restrict__ qcnt,
                                                              int L, uint32_t* __restrict__ sums2,
                                                              const uint32_t* __restrict__ gate) {
    if (gate && *gate == 0) return;  // the grid is not needed
    __shared__ uint32_t sh[256];
    const int64_t C = (int64_t)1 << (3 * L);
    const uint32_t* cnt = blockIdx.z ? qcnt : rcnt;
    uint32_t* sums = sums2 + (size_t)blockIdx.z * gridDim.y * gridDim.x;
    const int64_t base = (int64_t)blockIdx.y * C + (int64_t)blockIdx.x * kScanChunk;
    uint32_t v = 0;
    for (int i = threadIdx.x; i < kScanChunk && blockIdx.x * (int64_t)kScanChunk + i < C; i += 256)
        v += cnt[base + i];
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int o = 128; o >= 1; o /= 2) {
        if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) sums[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = sh[0];
}

__global__ __launch_bounds__(256) void grid_chunk_scan_kernel(
    uint32_t* __restrict__ rcnt, uint32_t* __restrict__ rfill, uint32_t* __restrict__ qcnt,
    uint32_t* __restrict__ qfill, int L, const uint32_t* __restrict__ sums2,
    const uint32_t* __restrict__ gate) {
    if (gate && *gate == 0) return;  // the grid is not needed
    __shared__ uint32_t sh[256];
    const int64_t C = (int64_t)1 << (3 * L);
    uint32_t* cnt = blockIdx.z ? qcnt : rcnt;
    uint32_t* fill = blockIdx.z ? qfill : rfill;
    const uint32_t* sums = sums2 + (size_t)blockIdx.z * gridDim.y * gridDim.x;
    const int64_t base = (int64_t)blockIdx.y * C + (int64_t)blockIdx.x * kScanChunk;
    // offset of this chunk: the sum of the chunks before it
    uint32_t off = 0;
    for (int i = threadIdx.x; i < (int)blockIdx.x; i += 256)
        off += sums[(int64_t)blockIdx.y * gridDim.x + i];
    sh[threadIdx.x] = off;
    __syncthreads();
    for (int o = 128; o >= 1; o /= 2) {
        if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
        __syncthreads();
    }
    off = sh[0];
    __syncthreads();
    // four consecutive bins per thread
    const int i0 = threadIdx.x * 4;
    uint32_t v[4], t = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool in = blockIdx.x * (int64_t)kScanChunk + i0 + r < C;
        v[r] = in ? cnt[base + i0 + r] : 0u;
        t += v[r];
    }
    sh[threadIdx.x] = t;
    __syncthreads();
    for (int o = 1; o < 256; o *= 2) {  // inclusive scan of the thread sums
        const uint32_t a = (int)threadIdx.x >= o ? sh[threadIdx.x - o] : 0u;
        __syncthreads();
        sh[threadIdx.x] += a;
        __syncthreads();
    }
    uint32_t run = off + sh[threadIdx.x] - t;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (blockIdx.x * (int64_t)kScanChunk + i0 + r < C) {
            cnt[base + i0 + r] = run;
            fill[base + i0 + r] = 0;
            run += v[r];
        }
    }
}

// Sorted copies, references then queries:
// out[b * n + start[code] + k] = (x, y, z, original index).
__global__ void grid_scatter_kernel(const float* __restrict__ ref, const float* __restrict__ query,
                                    int64_t B, int P, int Q, int L,
                                    const GridParams* __restrict__ gp,
                                    const uint32_t* __restrict__ rstart, uint32_t* __restrict__ rfill,
                                    const uint32_t* __restrict__ qstart, uint32_t* __restrict__ qfill,
                                    float4* __restrict__ rout, float4* __restrict__ qout,
                                    const uint32_t* __restrict__ gate,
                                    const int64_t* __restrict__ clouds) {
    if (gate && *gate == 0) return;  // the grid is not needed
    const int64_t C = (int64_t)1 << (3 * L);
    const int64_t nr = B * P;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < nr + B * Q;
         e += (int64_t)gridDim.x * blockDim.x) {
        const bool is_ref = e < nr;
        const int64_t i = is_ref ? e : e - nr;
        const int n = is_ref ? P : Q;
        const int64_t b = i / n;
        const int j = (int)(i - b * n);
        int64_t row = i;
        if (clouds) {
            if (j >= clouds[kGcWords * b + (is_ref ? kGcRCnt : kGcQCnt)]) continue;
            row = clouds[kGcWords * b + (is_ref ? kGcROff : kGcQOff)] + j;
        }
        const float* p = (is_ref ? ref : query) + row * 3;
        const uint32_t code = cell_code(gp[b], p[0], p[1], p[2], L);
        const uint32_t pos = (is_ref ? rstart : qstart)[b * C + code] +
                             atomicAdd(&(is_ref ? rfill : qfill)[b * C + code], 1u);
        (is_ref ? rout : qout)[b * n + pos] = make_float4(p[0], p[1], p[2], __int_as_float(j));
    }
}

// One 1024-thread workgroup per superblock (64 blocks of 16 sorted
// references): every block's box, box[(b * nblk + k) * 8 + 0..5], then the
// superblock's, sbox[(b * nsb + s) * 8 + 0..5]. Words 6 and 7 of each hold
// the smallest and largest original index of its references (int32 bits;
// 0x7FFFFFFF and -1 for an empty box), which Ball Query's grid pass tests
// against its index window.
__global__ __launch_bounds__(1024) void grid_boxes_kernel(const float4* __restrict__ sr,
                                                          int64_t B, int P, int nblk, int nsb,
                                                          float* __restrict__ box,
                                                          float* __restrict__ sbox,
                                                          const uint32_t* __restrict__ gate,
                                                          const int64_t* __restrict__ clouds) {
    if (gate && *gate == 0) return;  // the grid is not needed
    __shared__ float sh[kWave][8];
    const int64_t b = blockIdx.y;
    const int Pb = clouds ? (int)clouds[kGcWords * b + kGcRCnt] : P;  // real points of this cloud
    const int sb = blockIdx.x;
    const int t = threadIdx.x;
    const int j = sb * kWave * kGridBlk + t;
    const int k = sb * kWave + t / kGridBlk;  // this thread's block
    const float inf = __builtin_inff();
    float v[6] = {inf, inf, inf, -inf, -inf, -inf};
    int ilo = 0x7FFFFFFF, ihi = -1;
    if (j < Pb) {
        const float4 p = sr[b * P + j];
        v[0] = v[3] = p.x;
        v[1] = v[4] = p.y;
        v[2] = v[5] = p.z;
        ilo = ihi = __float_as_int(p.w);
    }
    auto fold = [&](int o) {
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            v[d] = fminf(v[d], __shfl_xor(v[d], o));
            v[3 + d] = fmaxf(v[3 + d], __shfl_xor(v[3 + d], o));
        }
        ilo = min(ilo, __shfl_xor(ilo, o));
        ihi = max(ihi, __shfl_xor(ihi, o));
    };
#pragma unroll
    for (int o = kGridBlk / 2; o >= 1; o /= 2) fold(o);
    if (t % kGridBlk == 0) {
#pragma unroll
        for (int d = 0; d < 6; ++d) sh[t / kGridBlk][d] = v[d];
        sh[t / kGridBlk][6] = __int_as_float(ilo);
        sh[t / kGridBlk][7] = __int_as_float(ihi);
        if (k < nblk) {
            float* o = box + ((size_t)b * nblk + k) * 8;
#pragma unroll
            for (int d = 0; d < 8; ++d) o[d] = sh[t / kGridBlk][d];
        }
    }
    __syncthreads();
    if (t < kWave) {
#pragma unroll
        for (int d = 0; d < 6; ++d) v[d] = sh[t][d];  // empty boxes past the end
        ilo = __float_as_int(sh[t][6]);
        ihi = __float_as_int(sh[t][7]);
#pragma unroll
        for (int o = kWave / 2; o >= 1; o /= 2) fold(o);
        if (t == 0) {
            float* o = sbox + ((size_t)b * nsb + sb) * 8;
#pragma unroll
            for (int d = 0; d < 6; ++d) o[d] = v[d];
            o[6] = __int_as_float(ilo);
            o[7] = __int_as_float(ihi);
        }
    }
}

// ------------------------------------------------------------------ search

template <int KCAP, int NW>
__global__ __launch_bounds__(NW* kWave) void knn_grid_kernel(
    const float4* __restrict__ sq, const float4* __restrict__ sr, int Q, int P, int k,
    const float* __restrict__ box, const float* __restrict__ sbox, int nblk, int nsb,
    const uint32_t* __restrict__ ref_start, const GridParams* __restrict__ gp, int L,
    float* __restrict__ out_dist, int64_t* __restrict__ out_idx, int squared,
    const int64_t* __restrict__ clouds) {
    constexpr int ROWS = kGridBuf > KCAP ? kGridBuf : KCAP;
    extern __shared__ uint2 lds[];             // per wave ROWS x 64 entries
    __shared__ uint32_t thr[NW][kWave];        // each wave's lanes' k-th key (high half)

    const int b = blockIdx.y;
    // This cloud's counts (a ragged batch: its own; the slots keep the
    // strides Q, P, nblk and nsb), first output row and index base.
    int Qb = Q, Pb = P, nbb = nblk, nsbb = nsb;
    int64_t orow0 = (int64_t)b * Q, ibase = 0;
    if (clouds) {
        const int64_t* c = clouds + (size_t)b * kGcWords;
        Qb = (int)c[kGcQCnt];
        Pb = (int)c[kGcRCnt];
        nbb = (Pb + kGridBlk - 1) / kGridBlk;
        nsbb = (nbb + kWave - 1) / kWave;
        orow0 = c[kGcQOff];
        ibase = c[kGcIdxBase];
    }
    if ((int)blockIdx.x * kWave >= Qb) return;  // the whole workgroup: no query of its cloud
    const int lane = threadIdx.x % kWave;
    const int w = uniform((int)(threadIdx.x / kWave));
    const int qi = blockIdx.x * kWave + lane;
    const bool qvalid = qi < Qb;
    const float4 q = sq[(size_t)b * Q + (qvalid ? qi : Qb - 1)];
    const float4* rb = sr + (size_t)b * P;
    const float* bx = box + (size_t)b * nblk * 8;
    const float* sbx = sbox + (size_t)b * nsb * 8;
    uint2* buf = lds + (size_t)w * ROWS * kWave;

    TopK64<KCAP> top;
    top.init(k);
    // Accept a key whose high half u <= lim; none without a query. Real keys
    // have u <= bits(+inf) + 1, so the start 0xFFFFFFFE admits them all but
    // never the marker 0xFFFFFFFF of the local pass's references (which a
    // cloud with fewer than k references would otherwise take twice).
    uint32_t lim = qvalid ? 0xFFFFFFFEu : 0u;
    thr[w][lane] = lim;
    int cnt = 0;

    // Each lane's own neighbourhood in sorted order: the kGridLocal references
    // around the first reference of its grid cell.
    const int nloc = min(Pb, kGridLocal);
    int loc0;
    {
        const int64_t C = (int64_t)1 << (3 * L);
        const uint32_t code = cell_code(gp[b], q.x, q.y, q.z, L);
        const int pos = (int)ref_start[(int64_t)b * C + code];
        loc0 = max(0, min(pos - nloc / 2, Pb - nloc));
    }

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
    // Candidates of 8 keys u[] at sorted positions j..j+7 (per lane `jl` when
    // the positions differ between lanes).
    auto take8 = [&](const uint32_t (&u)[8], const int (&jl)[8]) {
        uint32_t mn = u[0];
#pragma unroll
        for (int r = 1; r < 8; ++r) mn = min(mn, u[r]);
        if (ballot(mn <= lim)) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (u[r] <= lim) {
                    buf[cnt * kWave + lane] =
                        make_uint2(u[r], (uint32_t)__float_as_int(rb[jl[r]].w));
                    ++cnt;
                }
            }
            if (ballot(cnt > kGridBuf - 8)) flush();
        }
    };
    // Every wave skips, in later blocks, the references of its lane's local
    // pass: they are in wave 0's list already.
    auto scan_block = [&](int blk) {
        const int j0 = blk * kGridBlk, j1 = min(Pb, j0 + kGridBlk);
        int j = j0;
        for (; j + 8 <= j1; j += 8) {
            uint32_t u[8];
            int jl[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float4 p = rb[j + r];
                u[r] = f2u(s32(q.x, q.y, q.z, p.x, p.y, p.z)) + 1u;
                if ((uint32_t)(j + r - loc0) < (uint32_t)nloc) u[r] = 0xFFFFFFFFu;
                jl[r] = j + r;
            }
            take8(u, jl);
        }
        for (; j < j1; ++j) {
            const float4 p = rb[j];
            uint32_t u = f2u(s32(q.x, q.y, q.z, p.x, p.y, p.z)) + 1u;
            if ((uint32_t)(j - loc0) < (uint32_t)nloc) u = 0xFFFFFFFFu;
            if (u <= lim) {
                buf[cnt * kWave + lane] = make_uint2(u, (uint32_t)__float_as_int(p.w));
                ++cnt;
            }
            if (ballot(cnt > kGridBuf - 8)) flush();  // keep room for 8
        }
        // no flush here: candidates are rare once the limits are tight, and a
        // flush costs as many insertions as the fullest lane's buffer
    };

    // 1. Local pass (wave 0): every lane's own kGridLocal references, which
    //    hold most of its k nearest, so the limits are tight from the start.
    if (w == 0) {
        int r = 0;
        for (; r + 8 <= nloc; r += 8) {
            uint32_t u[8];
            int jl[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                jl[t] = loc0 + r + t;
                const float4 p = rb[jl[t]];
                u[t] = f2u(s32(q.x, q.y, q.z, p.x, p.y, p.z)) + 1u;
            }
            take8(u, jl);
        }
        for (; r < nloc; ++r) {
            const float4 p = rb[loc0 + r];
            const uint32_t u = f2u(s32(q.x, q.y, q.z, p.x, p.y, p.z)) + 1u;
            if (u <= lim) {
                buf[cnt * kWave + lane] = make_uint2(u, (uint32_t)__float_as_int(p.w));
                ++cnt;
            }
            if (ballot(cnt > kGridBuf - 8)) flush();  // keep room for 8
        }
        flush();
    }
    __syncthreads();  // every wave's limits, wave 0's local ones included, are in LDS
    refresh();

    // 2. Candidates first for the whole group at once, one box per lane: the
    //    bound between a box and the box of the group's queries (no larger than
    //    any query's bound) against the largest limit of the lanes; then each
    //    candidate per lane. Superblocks, then the blocks of a surviving
    //    superblock that belong to this wave (block % NW == w).
    float gl[3] = {q.x, q.y, q.z}, gh[3] = {q.x, q.y, q.z};
#pragma unroll
    for (int o = kWave / 2; o >= 1; o /= 2)
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            gl[d] = fminf(gl[d], __shfl_xor(gl[d], o));
            gh[d] = fmaxf(gh[d], __shfl_xor(gh[d], o));
        }
    auto group_bound = [&](const float* __restrict__ o) {
        const float gx = fmaxf(fmaxf(o[0] - gh[0], gl[0] - o[3]), 0.0f);
        const float gy = fmaxf(fmaxf(o[1] - gh[1], gl[1] - o[4]), 0.0f);
        const float gz = fmaxf(fmaxf(o[2] - gh[2], gl[2] - o[5]), 0.0f);
        return (gx * gx + gy * gy) + gz * gz;
    };
    for (int sb0 = 0; sb0 < nsbb; sb0 += kWave) {
        uint32_t mlim = wave_max_u32(lim);
        const int my_sb = sb0 + lane;
        uint64_t cs = ballot(my_sb < nsbb &&
                             f2u(group_bound(sbx + (size_t)min(my_sb, nsbb - 1) * 8)) + 1u <= mlim);
        while (cs) {
            const int s = sb0 + __builtin_ctzll(cs);
            cs &= cs - 1;
            if (ballot(f2u(box_bound(sbx + (size_t)s * 8, q.x, q.y, q.z)) + 1u <= lim) == 0)
                continue;
            mlim = wave_max_u32(lim);
            const int my_blk = s * kWave + lane;
            const bool mine = my_blk < nbb && my_blk % NW == w;
            uint64_t cb = ballot(mine && f2u(group_bound(bx + (size_t)min(my_blk, nbb - 1) * 8)) +
                                             1u <= mlim);
            while (cb) {
                const int blk = s * kWave + __builtin_ctzll(cb);
                cb &= cb - 1;
                if (ballot(f2u(box_bound(bx + (size_t)blk * 8, q.x, q.y, q.z)) + 1u <= lim) == 0)
                    continue;
                scan_block(blk);
                refresh();
            }
        }
    }

    flush();

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
                    // front sentinels insert nothing, nor does a reference that
                    // two waves both hold (the local pass and a later block)
                    top.insert(kk != 0ull && !top.contains(kk) ? kk : ~0ull);
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
    const int64_t row = orow0 + __float_as_int(q.w);
    float* od = out_dist + row * k;
    int64_t* oi = out_idx + row * k;
    const int front = KCAP - k;
#pragma unroll
    for (int p = 0; p < KCAP; ++p) {
        if (p >= front) {
            // an empty slot only in a cloud with fewer than k references:
            // (+inf, -1), or (0, -1) for squared distances
            const bool empty = top.key[p] == ~0ull;
            const float sv = u2f((uint32_t)(top.key[p] >> 32) - 1u);
            od[p - front] = empty ? (squared ? 0.0f : __builtin_inff()) : squared ? sv : sqrtf(sv);
            oi[p - front] = empty ? (int64_t)-1 : ibase + (int64_t)(uint32_t)top.key[p];
        }
    }
}

// One or two (QW) queries per wave (k <= 32). A workgroup holds kKgwWaves
// waves of consecutive queries in grid order; with QW = 2 a wave's two
// neighbouring queries share every box test (a box is opened for either)
// and every reference load. The wave first sorts the 64
// references around its query's grid position into its list (wave_list.h,
// keys (bits(s) << 32) | index) and takes the k-th key's high word as its
// bound; then its lanes test 64 superblock boxes at a time and, in a
// surviving superblock, 64 block boxes, and test the references of up to four
// surviving blocks at a time, one per lane. A box is visited when its lower
// bound's bits do not exceed the bound (a point with equal bits may still
// enter by a smaller index), and a reference is offered under the same
// inclusive test; the merges keep the 32 smallest keys, so any visiting order
// gives the (s, j) order. No barriers: the waves of a workgroup are
// independent.
constexpr int kKgwWaves = 4;

template <int QW, int KL>
__global__ __launch_bounds__(kKgwWaves* kWave) void knn_grid_wave_kernel(
    const float4* __restrict__ sq, const float4* __restrict__ sr, int Q, int P, int k,
    const float* __restrict__ box, const float* __restrict__ sbox, int nblk, int nsb,
    const uint32_t* __restrict__ ref_start, const GridParams* __restrict__ gp, int L,
    float* __restrict__ out_dist, int64_t* __restrict__ out_idx, int squared,
    const int64_t* __restrict__ clouds) {
    __shared__ uint64_t cbuf[kKgwWaves][QW][kWave - KL];
    const int b = blockIdx.y;
    int Qb = Q, Pb = P, nbb = nblk, nsbb = nsb;
    int64_t orow0 = (int64_t)b * Q, ibase = 0;
    if (clouds) {
        const int64_t* c = clouds + (size_t)b * kGcWords;
        Qb = (int)c[kGcQCnt];
        Pb = (int)c[kGcRCnt];
        nbb = (Pb + kGridBlk - 1) / kGridBlk;
        nsbb = (nbb + kWave - 1) / kWave;
        orow0 = c[kGcQOff];
        ibase = c[kGcIdxBase];
    }
    const int lane = lane_id();
    const int w = uniform((int)(threadIdx.x / kWave));
    const int q0 = ((int)blockIdx.x * kKgwWaves + w) * QW;  // this wave's first query
    if (q0 >= Qb) return;  // whole waves
    const float4* rb = sr + (size_t)b * P;
    const float* bx = box + (size_t)b * nblk * 8;
    const float* sbx = sbox + (size_t)b * nsb * 8;
    const int nloc = min(Pb, kWave);
    const int64_t C = (int64_t)1 << (3 * L);

    // 1. Per query, the kWave references around its own grid position. A
    //    query slot past the cloud's last (QW > 1, odd count) repeats the
    //    first query; it opens no box and takes no candidate.
    float4 q[QW];
    int loc0[QW];
    bool real[QW];
    KwQuery st[QW];
#pragma unroll
    for (int h = 0; h < QW; ++h) {
        const bool valid = q0 + h < Qb;
        real[h] = valid;
        q[h] = sq[(size_t)b * Q + (valid ? q0 + h : q0)];
        const uint32_t code = cell_code(gp[b], q[h].x, q[h].y, q[h].z, L);
        const int pos = (int)ref_start[(int64_t)b * C + code];
        loc0[h] = max(0, min(pos - nloc / 2, Pb - nloc));
        uint64_t key = kKwEmpty;
        if (lane < nloc) {
            const float4 p = rb[loc0[h] + lane];
            key = ((uint64_t)f2u(s32(q[h].x, q[h].y, q[h].z, p.x, p.y, p.z)) << 32) |
                  (uint32_t)__float_as_int(p.w);
        }
        st[h] = KwQuery{kw_sort_merge(key, lane), 0u, 0, cbuf[w][h]};
        st[h].bound = valid ? lane_value((uint32_t)(st[h].list >> 32), k - 1) : 0u;
    }
    auto open = [&](const float* o) {  // the box may hold a reference some query takes
        bool any = false;
#pragma unroll
        for (int h = 0; h < QW; ++h)
            any |= real[h] && f2u(box_bound(o, q[h].x, q[h].y, q[h].z)) <= st[h].bound;
        return any;
    };

    // 2. Superblocks, then the blocks of a surviving one, then the references
    //    of up to four surviving blocks at a time (16 lanes each), each read
    //    once for the QW queries; a query's local references are in its list.
    for (int sb0 = 0; sb0 < nsbb; sb0 += kWave) {
        const int my_sb = sb0 + lane;
        uint64_t ms = ballot(my_sb < nsbb && open(sbx + (size_t)min(my_sb, nsbb - 1) * 8));
        while (ms) {
            const int s = sb0 + __builtin_ctzll(ms);
            ms &= ms - 1;
            const int my_blk = s * kWave + lane;
            uint64_t mb = ballot(my_blk < nbb && open(bx + (size_t)min(my_blk, nbb - 1) * 8));
            while (mb) {
                int blk[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    blk[r] = mb ? s * kWave + __builtin_ctzll(mb) : -1;
                    mb &= mb - 1;  // no-op once empty
                }
                const int g = lane >> 4;
                const int mine = g == 0 ? blk[0] : g == 1 ? blk[1] : g == 2 ? blk[2] : blk[3];
                const int j = mine * kGridBlk + (lane & (kGridBlk - 1));
                const bool in = mine >= 0 && j < Pb;
                const float4 p = in ? rb[j] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
                for (int h = 0; h < QW; ++h) {
                    bool cand = false;
                    uint32_t u = 0u;
                    if (real[h] && in && (uint32_t)(j - loc0[h]) >= (uint32_t)nloc) {
                        u = f2u(s32(q[h].x, q[h].y, q[h].z, p.x, p.y, p.z));
                        cand = u <= st[h].bound;
                    }
                    kw_offer<true, KL>(st[h], cand, u, __float_as_int(p.w), lane, k);
                }
            }
        }
    }

    // 3. Lane n < k writes the n-th key of each query; empty only in a cloud
    //    with fewer than k references.
#pragma unroll
    for (int h = 0; h < QW; ++h) {
        if (q0 + h >= Qb) break;
        if (st[h].cnt > 0) kw_merge<KL>(st[h], lane, k);
        if (lane < k) {
            const uint64_t e = st[h].list;
            const bool empty = e == kKwEmpty;
            const float sv = u2f((uint32_t)(e >> 32));
            const int64_t o = (orow0 + __float_as_int(q[h].w)) * k + lane;
            out_dist[o] = empty ? (squared ? 0.0f : __builtin_inff()) : squared ? sv : sqrtf(sv);
            out_idx[o] = empty ? (int64_t)-1 : ibase + (int64_t)(uint32_t)e;
        }
    }
}

// ------------------------------------------------------------------ host side

int knn_grid_level(int64_t P) {
    // two to sixteen references per cell, 2..7 bits per axis (a CPU model of
    // the scanned references at 100k uniform points favoured about 3 per cell)
    int L = 2;
    while (L < 7 && ((int64_t)1 << (3 * (L + 1))) * 2 <= P) ++L;
    return L;
}

struct GridLayout {
    size_t params, enc, sums, ref_cnt, ref_fill, q_cnt, q_fill, sref, squery, box, sbox, total;
};

static size_t al(size_t n) { return (n + 255) / 256 * 256; }

static GridLayout grid_layout(int64_t B, int64_t Q, int64_t P, int L) {
    const size_t C = (size_t)1 << (3 * L);
    const int64_t nblk = (P + kGridBlk - 1) / kGridBlk, nsb = (nblk + kWave - 1) / kWave;
    GridLayout g;
    size_t o = 0;
    g.params = o; o += al(B * sizeof(GridParams));
    g.enc = o; o += al(B * kEncWords * sizeof(uint32_t));
    g.sums = o; o += al(2 * B * ((C + 1023) / 1024) * sizeof(uint32_t));
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

size_t grid_workspace_bytes(int64_t B, int64_t Q, int64_t P, int L) {
    return grid_layout(B, Q, P, L).total;
}

size_t knn_grid_workspace_bytes(int64_t B, int64_t Q, int64_t P) {
    return grid_workspace_bytes(B, Q, P, knn_grid_level(P));
}

static unsigned grid_blocks(int64_t n) {
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 8192));
}

hipError_t launch_grid_build(const float* query, const float* ref, int64_t B, int64_t Q,
                             int64_t P, int L, void* workspace, const uint32_t* gate,
                             const int64_t* clouds, hipStream_t stream, GridView* view) {
    const int64_t C = (int64_t)1 << (3 * L);
    const int nblk = (int)((P + kGridBlk - 1) / kGridBlk), nsb = (nblk + kWave - 1) / kWave;
    const GridLayout g = grid_layout(B, Q, P, L);
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
    *view = GridView{gp, rcnt, sref, squery, box, sbox, L, nblk, nsb};
    hipError_t e;
#define POINTOPS_CHECK(x) \
    do {                   \
        x;                 \
        e = hipGetLastError(); \
        if (e != hipSuccess) return e; \
    } while (0)
    uint32_t* enc = (uint32_t*)(ws + g.enc);
    // the four histogram arrays are contiguous: cleared together
    const size_t nzero = (g.sref - g.ref_cnt) / sizeof(uint32_t);
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_init_kernel,
                                      dim3(std::max(grid_blocks((int64_t)nzero),
                                                    grid_blocks(B * kEncWords))),
                                      dim3(256), 0, stream, enc, B, rcnt, nzero, gate));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_bounds_kernel,
                                      dim3((unsigned)std::min<int64_t>((P + 1023) / 1024, 256),
                                           (unsigned)B),
                                      dim3(256), 0, stream, ref, B, (int)P, L, enc, gp, gate, clouds));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_count_kernel, dim3(grid_blocks(B * (P + Q))), dim3(256),
                                      0, stream, ref, query, B, (int)P, (int)Q, L, gp, rcnt, qcnt,
                                      gate, clouds));
    const unsigned nchunk = (unsigned)((C + kScanChunk - 1) / kScanChunk);
    uint32_t* sums = (uint32_t*)(ws + g.sums);
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_chunk_sums_kernel, dim3(nchunk, (unsigned)B, 2),
                                      dim3(256), 0, stream, rcnt, qcnt, L, sums, gate));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_chunk_scan_kernel, dim3(nchunk, (unsigned)B, 2),
                                      dim3(256), 0, stream, rcnt, rfill, qcnt, qfill, L, sums,
                                      gate));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_scatter_kernel, dim3(grid_blocks(B * (P + Q))),
                                      dim3(256), 0, stream, ref, query, B, (int)P, (int)Q, L, gp,
                                      rcnt, rfill, qcnt, qfill, sref, squery, gate, clouds));
    POINTOPS_CHECK(hipLaunchKernelGGL(grid_boxes_kernel, dim3((unsigned)nsb, (unsigned)B),
                                      dim3(1024), 0, stream, sref, B, (int)P, nblk, nsb, box,
                                      sbox, gate, clouds));
#undef POINTOPS_CHECK
    return hipSuccess;
}

// squared != 0: out_dist holds s itself (the Chamfer distance's nearest points).
// With `clouds` (device memory, B records; see GridCloud) P and Q are the
// largest counts of the ragged batch.
// nw == 0 / -2: one / two queries per wave (knn_grid_wave_kernel, k <= 32);
// otherwise one query per lane with nw waves per workgroup.
hipError_t launch_knn_grid(const float* query, const float* ref, int64_t B, int64_t Q, int64_t P,
                           int64_t k, float* out_dist, int64_t* out_idx, int kcap, int nw,
                           void* workspace, int squared, const int64_t* clouds,
                           hipStream_t stream) {
    if (nw <= 0 && (k < 1 || k > kKwBuf)) return hipErrorInvalidValue;
    GridView v;
    hipError_t e = launch_grid_build(query, ref, B, Q, P, knn_grid_level(P), workspace, nullptr,
                                     clouds, stream, &v);
    if (e != hipSuccess) return e;
    if (nw <= 0) {  // 0: one query per wave, -2: two
        const int qw = nw == -2 ? 2 : 1;
        const dim3 grid((unsigned)((Q + kKgwWaves * qw - 1) / (kKgwWaves * qw)), (unsigned)B);
        // k <= 16: a 16-lane list and 48 buffered candidates per merge
#define POINTOPS_KGW(QWV, KLV)                                                                \
    hipLaunchKernelGGL((knn_grid_wave_kernel<QWV, KLV>), grid, dim3(kKgwWaves * kWave), 0,     \
                       stream, v.squery, v.sref, (int)Q, (int)P, (int)k, v.box, v.sbox, v.nblk, \
                       v.nsb, v.ref_start, v.gp, v.L, out_dist, out_idx, squared, clouds)
        if (qw == 2) {
            if (k <= 16) POINTOPS_KGW(2, 16); else POINTOPS_KGW(2, 32);
        } else {
            if (k <= 16) POINTOPS_KGW(1, 16); else POINTOPS_KGW(1, 32);
        }
#undef POINTOPS_KGW
        return hipGetLastError();
    }
#define POINTOPS_CHECK(x) \
    do {                   \
        x;                 \
        e = hipGetLastError(); \
        if (e != hipSuccess) return e; \
    } while (0)
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
                                          stream, v.squery, v.sref, (int)Q, (int)P, (int)k,    \
                                          v.box, v.sbox, v.nblk, v.nsb, v.ref_start, v.gp, v.L,\
                                          out_dist, out_idx, squared, clouds));                \
        return hipSuccess;                                                                     \
    }
    POINTOPS_GRID_CASE(1, 2) POINTOPS_GRID_CASE(2, 2) POINTOPS_GRID_CASE(4, 2)
    POINTOPS_GRID_CASE(8, 2) POINTOPS_GRID_CASE(16, 2) POINTOPS_GRID_CASE(32, 2)
    POINTOPS_GRID_CASE(64, 2)
    POINTOPS_GRID_CASE(16, 1) POINTOPS_GRID_CASE(16, 4) POINTOPS_GRID_CASE(16, 8)
#undef POINTOPS_GRID_CASE
#undef POINTOPS_CHECK
    return hipErrorInvalidValue;
}

}  // namespace pointops
