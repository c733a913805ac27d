// Farthest point sampling for gfx950: one persistent launch for all steps.
//
// Contract: project page "mps-pointops", section "The operators in equations",
// "Farthest point sampling" (c_0 = start_idx; m_j is the smallest squared
// distance from x_j to a chosen centre; the next centre is the smallest index
// holding the largest m) and section "Contracts" (the start index; the
// remaining slots repeat index 0 once every point is taken).
//
// Mapping. Each cloud is split into G contiguous slices, one workgroup per
// slice; all G workgroups of a cloud run together for the whole launch (the
// host keeps the grid within what the device holds at once). Thread t of a
// workgroup keeps the PPT consecutive points at slice positions t*PPT .. t*PPT
// + PPT - 1 in registers with their running minimum m, so position order is
// index order across (wave, lane, register) and a step reads no global memory.
//
// m is kept as the bits of the float: m >= +0, so unsigned order is value
// order, and min_u32(m, bits(d)) equals the contract's "d < m ? d : m" for
// every d >= +0 and leaves m unchanged for a NaN d. Positions past the end of
// the slice hold m = +0: they can only tie with a maximum of 0, and then the
// slice's first point (position 0, a real point with m = 0) comes first.
//
// A step: fold the last centre into m and keep each thread's first maximum
// (3 integer ops per point on top of the 9 of s32 and the min); the wave
// maximum by DPP lane exchanges; the first lane holding it (ballot + find
// first set) gives the smallest position, hence the smallest index; the
// workgroup does the same over its waves' winners through LDS. With G > 1 the
// workgroups then exchange their winners through device memory: each writes
// five 64-bit words (m, index, x, y, z), each carrying the step number in its
// low half, with relaxed device-scope atomic stores, and polls all G slots
// with relaxed device-scope atomic loads until every word shows the step. A
// word is never read torn and validates itself, so no release/acquire fences
// (cache write-back / invalidate) are needed. Two slot sets alternate by step
// parity: a workgroup can only write set (t & 1) again at step t + 2 after
// every workgroup has published step t + 1, which each does only after it has
// read all of step t. The winner's coordinates travel with it (read from an
// LDS copy of the slice), so no step waits on a load of the new centre.
//
// Compared with the project page's design (one threadgroup per cloud running
// every step, and for one large cloud a second dispatch per step to reduce the
// chunk maxima), the reduction here never leaves the launch.
//
// Termination: every poll loop is bounded. A workgroup that waits longer than
// `spin_limit` polls raises the status word and stops; the others then stop on
// their own bound; output slots not reached are -1.
//
// Ragged batches (a cloud table, see segments.h; the project page's flat FPS
// and its planned multi-workgroup FPS over uneven batches): each cloud gets
// its own number of workgroups, numbered cloud after cloud, with its own
// points, outputs, start index and exchange words. Clouds never interact; the
// argmax of each step is taken over that cloud's workgroups only.
#include <algorithm>
#include <cstdlib>
#include <tuple>
#include <type_traits>
#include <utility>

#include "api_internal.h"
#include "common.h"
#include "segments.h"

namespace pointops {

struct alignas(64) FpsSlot {
    uint64_t w[5];  // (payload << 32) | step: m bits, index, x, y, z
    uint64_t pad[3];
};

__device__ __forceinline__ uint64_t tagged(uint32_t payload, uint32_t step) {
    return ((uint64_t)payload << 32) | step;
}

template <int PPT, int BLOCK>
__global__ __launch_bounds__(BLOCK) void fps_kernel(
    const float* __restrict__ xyz, int N, int M, int start_idx, int G, int slice,
    int64_t* __restrict__ out_idx, float* __restrict__ out_xyz, FpsSlot* __restrict__ slots,
    uint32_t* __restrict__ status, uint32_t spin_limit, const int64_t* __restrict__ seg,
    int nseg) {
    constexpr int NWAVE = BLOCK / kWave;
    extern __shared__ float lds_xyz[];  // the slice's coordinates, AoS
    __shared__ uint32_t wave_m[2][NWAVE];
    __shared__ uint32_t wave_j[2][NWAVE];
    __shared__ uint32_t result[2][6];    // m, index, x, y, z, abort

    // this workgroup's cloud; ragged launches give every cloud one workgroup
    int g;
    int64_t xrow0, orow0, jbase;
    FpsSlot* cs;
    if (seg) {
        const int b = seg_find(seg, nseg, blockIdx.x);
        const int64_t* rec = seg_record(seg, nseg, b);
        g = 0;
        G = 1;
        N = (int)rec[kFrXCnt];
        slice = N;
        M = (int)rec[kFrOCnt];
        start_idx = (int)rec[kFrStart];
        xrow0 = rec[kFrXOff];
        orow0 = rec[kFrOOff];
        jbase = rec[kFrIdxBase];
        cs = slots;
    } else {
        const int b = blockIdx.x / G;
        g = blockIdx.x - b * G;
        xrow0 = (int64_t)b * N;
        orow0 = (int64_t)b * M;
        jbase = 0;
        cs = slots + (size_t)b * 2 * G;
    }
    const int tid = threadIdx.x;
    const int wave = uniform(tid / kWave);
    const int lane = tid % kWave;
    const float* xb = xyz + xrow0 * 3;
    const int lo = g * slice;
    const int cnt = min(N, lo + slice) - lo;  // >= 1: the host never makes empty slices

    for (int i = tid; i < 3 * cnt; i += BLOCK) lds_xyz[i] = xb[(size_t)3 * lo + i];

    float px[PPT], py[PPT], pz[PPT];
    uint32_t pm[PPT];
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
        const int r = tid * PPT + p;
        const bool real = r < cnt;
        const size_t j = (size_t)lo + (real ? r : 0);
        px[p] = xb[3 * j + 0];
        py[p] = xb[3 * j + 1];
        pz[p] = xb[3 * j + 2];
        pm[p] = real ? 0x7F800000u : 0u;  // +inf for points, +0 for padding
    }

    int c = start_idx;
    float cx = xb[(size_t)3 * c + 0], cy = xb[(size_t)3 * c + 1], cz = xb[(size_t)3 * c + 2];
    int64_t* ob = out_idx + orow0;
    float* oxb = out_xyz ? out_xyz + orow0 * 3 : nullptr;
    if (g == 0 && tid == 0) {
        ob[0] = jbase + c;
        if (oxb) { oxb[0] = cx; oxb[1] = cy; oxb[2] = cz; }
    }
    __syncthreads();  // lds_xyz is complete

    for (int t = 1; t < M; ++t) {
        const int par = t & 1;
        // 1. fold centre c_{t-1} in; first maximum of this thread's points
        uint32_t bm = 0;
        int bp = 0;
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            pm[p] = min(pm[p], f2u(s32(cx, cy, cz, px[p], py[p], pz[p])));
            bp = pm[p] > bm ? p : bp;
            bm = max(bm, pm[p]);
        }
        // 2. wave: maximum, then the first lane holding it
        {
            const uint32_t wm = wave_max_u32(bm);
            const int l = __builtin_ctzll(ballot(bm == wm));
            const int wj = lo + (wave * kWave + l) * PPT + (int)lane_value((uint32_t)bp, l);
            if (lane == 0) {
                wave_m[par][wave] = wm;
                wave_j[par][wave] = (uint32_t)wj;
            }
        }
        __syncthreads();
        // 3. workgroup: the same over the waves' winners (every wave when G == 1)
        uint32_t rm = 0, rj = 0, rx = 0, ry = 0, rz = 0, abort = 0;
        if (G == 1 || wave == 0) {
            const uint32_t em = lane < NWAVE ? wave_m[par][lane] : 0u;
            const uint32_t ej = lane < NWAVE ? wave_j[par][lane] : 0u;
            rm = wave_max_u32(em);
            const int l = __builtin_ctzll(ballot(em == rm));
            rj = lane_value(ej, l);
            const int r = (int)rj - lo;  // the winner is a real point of the slice
            rx = f2u(lds_xyz[3 * r + 0]);
            ry = f2u(lds_xyz[3 * r + 1]);
            rz = f2u(lds_xyz[3 * r + 2]);
        }
        if (G > 1) {
            if (wave == 0) {
                // 4. cloud: publish this slice's winner, gather all G of step t
                FpsSlot* set = cs + (size_t)par * G;
                const uint32_t tag = (uint32_t)t;
                if (lane < 5) {
                    const uint32_t v = lane == 0 ? rm : lane == 1 ? rj : lane == 2 ? rx
                                     : lane == 3 ? ry : rz;
                    __hip_atomic_store(&set[g].w[lane], tagged(v, tag), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
                uint32_t bestm = 0, bestj = 0, bestx = 0, besty = 0, bestz = 0;
                bool have = false;
                for (int base = 0; base < G && !abort; base += kWave) {
                    const int s = base + lane;
                    const bool mine = s < G;
                    uint64_t w0 = 0, w1 = 0, w2 = 0, w3 = 0, w4 = 0;
                    uint32_t spins = 0;
                    while (true) {
                        if (mine) {
                            w0 = __hip_atomic_load(&set[s].w[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            w1 = __hip_atomic_load(&set[s].w[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            w2 = __hip_atomic_load(&set[s].w[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            w3 = __hip_atomic_load(&set[s].w[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            w4 = __hip_atomic_load(&set[s].w[4], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        }
                        const bool ready = !mine || ((uint32_t)w0 == tag && (uint32_t)w1 == tag &&
                                                     (uint32_t)w2 == tag && (uint32_t)w3 == tag &&
                                                     (uint32_t)w4 == tag);
                        if (ballot(!ready) == 0) break;
                        if (++spins > spin_limit) { abort = 1; break; }
                        __builtin_amdgcn_s_sleep(1);
                    }
                    if (abort) break;
                    // slots of this chunk in index order by lane; an earlier chunk
                    // keeps its winner on a tie
                    const uint32_t sm = mine ? (uint32_t)(w0 >> 32) : 0u;
                    const uint32_t cm = wave_max_u32(sm);
                    const int l = __builtin_ctzll(ballot(mine && sm == cm));
                    if (!have || cm > bestm) {
                        have = true;
                        bestm = cm;
                        bestj = lane_value((uint32_t)(w1 >> 32), l);
                        bestx = lane_value((uint32_t)(w2 >> 32), l);
                        besty = lane_value((uint32_t)(w3 >> 32), l);
                        bestz = lane_value((uint32_t)(w4 >> 32), l);
                    }
                }
                if (lane == 0) {
                    uint32_t* o = result[par];
                    o[0] = bestm; o[1] = bestj; o[2] = bestx; o[3] = besty; o[4] = bestz;
                    o[5] = abort;
                }
            }
            __syncthreads();
            // result[par] is next written at step t + 2, after step t + 1's barriers
            const uint32_t* o = result[par];
            rj = o[1]; rx = o[2]; ry = o[3]; rz = o[4]; abort = o[5];
        }
        if (abort) {
            if (tid == 0) {
                atomicOr(status, 1u);
                if (g == 0)
                    for (int u = t; u < M; ++u) ob[u] = -1;
            }
            return;
        }
        c = (int)rj;
        cx = u2f(rx);
        cy = u2f(ry);
        cz = u2f(rz);
        if (g == 0 && tid == 0) {
            ob[t] = jbase + c;
            if (oxb) { oxb[3 * t + 0] = cx; oxb[3 * t + 1] = cy; oxb[3 * t + 2] = cz; }
        }
    }
    // header word 1: the exchanges of the launch's first cloud (one per step)
    if (blockIdx.x == 0 && tid == 0) status[1] = G > 1 && M > 1 ? (uint32_t)(M - 1) : 0u;
}

// ---------------------------------------------------------------- batched FPS
//
// The same selection, with far fewer cross-workgroup exchanges. Wave 0 of every
// workgroup certifies; the other waves hold the slice. At an exchange each
// point wave reports its two largest keys (m, -index) with their coordinates,
// and a bound: its third largest key. Each workgroup publishes its RG best
// reports and its own bound, the largest of its wave bounds and unpublished
// reports. Every workgroup of the cloud receives the same candidate set C and
// the largest bound beta, and wave 0 of each workgroup then runs FPS steps on
// C alone: it takes the largest key K* in C and folds the new centre into the
// m of every candidate. Every point outside C has a key at most beta, and
// keys only decrease as centres are added, so whenever K* > beta the candidate
// is the true next centre of the whole cloud; the first step after an
// exchange always qualifies (the cloud's largest key is a report that its
// workgroup publishes). When a step does not qualify, or the batch is full,
// the batch ends. While wave 0 certifies centres, the point waves fold each
// new centre (read from an LDS list) into their points' m; at the end of the
// batch every point is up to date and the next exchange starts. All decisions
// are the ones the plain definition makes, in the same order; only the
// communication is batched.

constexpr int kFpsMaxBatch = 256;  // centres certified per batch at most
constexpr int kCertBlock = 4;       // certification steps between exit tests
constexpr uint32_t kNone = 0xFFFFFFFFu;

// Key order: larger m first, then smaller index.
__device__ __forceinline__ bool key_gt(uint32_t ma, uint32_t ja, uint32_t mb, uint32_t jb) {
    return ma > mb || (ma == mb && ja < jb);
}

// Exchange words of the batched kernel: an 8-bit batch tag in the low byte and
// 56 payload bits above it. A candidate's five 32-bit fields (m, index, x, y,
// z: 160 bits) travel in three words; a bound's m and index in two.
__device__ __forceinline__ uint64_t tag8(uint64_t payload, uint32_t tag) {
    return (payload << 8) | (tag & 0xFFu);
}

__device__ __forceinline__ void pack_candidate(uint32_t m, uint32_t j, uint32_t x, uint32_t y,
                                               uint32_t z, uint64_t& w0, uint64_t& w1,
                                               uint64_t& w2) {
    const uint64_t a = (uint64_t)m | ((uint64_t)j << 32);
    const uint64_t b = (uint64_t)x | ((uint64_t)y << 32);
    w0 = a & ((1ull << 56) - 1);                       // a bits 0..55
    w1 = ((a >> 56) | (b << 8)) & ((1ull << 56) - 1);  // a bits 56..63, b bits 0..47
    w2 = (b >> 48) | ((uint64_t)z << 16);              // b bits 48..63, z
}

__device__ __forceinline__ void unpack_candidate(uint64_t w0, uint64_t w1, uint64_t w2,
                                                 uint32_t& m, uint32_t& j, uint32_t& x,
                                                 uint32_t& y, uint32_t& z) {
    const uint64_t a = w0 | (w1 << 56);
    const uint64_t b = (w1 >> 8) | (w2 << 48);
    m = (uint32_t)a;
    j = (uint32_t)(a >> 32);
    x = (uint32_t)b;
    y = (uint32_t)(b >> 32);
    z = (uint32_t)(w2 >> 16);
}

// Largest key over the lanes of a wave whose `use` flag is set. Lanes must be
// in increasing index order (the first lane holding the largest m has the
// smallest index). Returns (m, index) of the winner, (0, kNone) when no lane
// takes part.
__device__ __forceinline__ void wave_max_key(uint32_t m, uint32_t j, bool use, uint32_t& om,
                                             uint32_t& oj, int& olane) {
    const uint32_t mx = wave_max_u32(use ? m : 0u);
    const uint64_t mask = ballot(use && m == mx);
    if (mask == 0) {
        om = 0;
        oj = kNone;
        olane = -1;
        return;
    }
    olane = __builtin_ctzll(mask);
    om = mx;
    oj = lane_value(j, olane);
}

// Like wave_max_key, for lanes in any index order: among the lanes holding the
// largest m, the one with the smallest index (rare: an extra reduction).
__device__ __forceinline__ void wave_max_key_any(uint32_t m, uint32_t j, bool use, uint32_t& om,
                                                 uint32_t& oj, int& olane) {
    const uint32_t mx = wave_max_u32(use ? m : 0u);
    uint64_t mask = ballot(use && m == mx);
    if (mask == 0) {
        om = 0;
        oj = kNone;
        olane = -1;
        return;
    }
    if (mask & (mask - 1)) {
        const bool in = (mask >> lane_id()) & 1ull;
        const uint32_t jm = ~wave_max_u32(in ? ~j : 0u);
        mask &= ballot(j == jm);
    }
    olane = __builtin_ctzll(mask);
    om = mx;
    oj = lane_value(j, olane);
}

// ------------------------------------------------------- grouping of the slices
//
// For the batched kernel on clouds where a centre's fold over a workgroup's
// points outweighs its certification (several points per thread), each slice
// is first reordered so that every point wave holds a spatially compact group:
// the slice's points in the Morton order of their cells in the slice's
// bounding box, cut into runs of one wave's capacity. Position order is then
// not index order, so wherever the plain kernel lets the first lane or the
// earlier register win a tie (a thread's best points, a wave's reports, the
// certifying wave's choice among the waves' reports, the workgroup bound, the
// order of the published candidates), the grouped kernel compares indices
// explicitly; padding positions carry no index and lose every tie. A point
// wave then folds a centre only if the centre's lower bound to the wave's box
// is below the largest m in the wave. The result is unchanged: a skipped fold
// leaves every m of the wave as it was.

constexpr int kGroupMaxSlice = kFpsGroupMaxSlice;

// 4-bit coordinate cell in [lo, lo + 16 / scale) (0 for NaN), spread to every
// third bit: 4096 cells of the slice's box in Morton order.
__device__ __forceinline__ uint32_t morton4(float v, float lo, float scale) {
    const float t = (v - lo) * scale;
    uint32_t q = t >= 15.f ? 15u : (t >= 0.f ? (uint32_t)t : 0u);
    q = (q | (q << 4)) & 0x0C3u;
    q = (q | (q << 2)) & 0x249u;
    return q;
}

// One workgroup per slice: a counting sort of the slice's points by their
// Morton cell (4096 cells of the slice's bounding box; the order inside a
// cell is whichever the LDS counters hand out), written as (x, y, z, cloud
// index) to `grouped` (B x N float4, slice positions in place). Runs of one
// wave's capacity of this order are the point waves' groups.
template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void fps_group_kernel(const float* __restrict__ xyz, int N,
                                                          int G, int slice,
                                                          float4* __restrict__ grouped) {
    constexpr int kCells = 4096, kPer = kGroupMaxSlice / BLOCK, kNW = BLOCK / kWave;
    __shared__ uint32_t cell_start[kCells];
    __shared__ float red[6][kNW];
    __shared__ uint32_t wsum[kNW];
    const int b = blockIdx.x / G, g = blockIdx.x - b * G;
    const int lo = g * slice;
    const int cnt = min(N, lo + slice) - lo;
    const float* xb = xyz + ((int64_t)b * N + lo) * 3;
    float4* ob = grouped + (int64_t)b * N + lo;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    for (int c = tid; c < kCells; c += BLOCK) cell_start[c] = 0;
    // the slice's bounding box (NaN coordinates take no part: fminf/fmaxf)
    float mn[3] = {INFINITY, INFINITY, INFINITY}, mx[3] = {-INFINITY, -INFINITY, -INFINITY};
    for (int i = tid; i < cnt; i += BLOCK)
        for (int a = 0; a < 3; ++a) {
            mn[a] = fminf(mn[a], xb[3 * i + a]);
            mx[a] = fmaxf(mx[a], xb[3 * i + a]);
        }
    for (int a = 0; a < 3; ++a)
        for (int off = 32; off >= 1; off >>= 1) {
            mn[a] = fminf(mn[a], __shfl_xor(mn[a], off, kWave));
            mx[a] = fmaxf(mx[a], __shfl_xor(mx[a], off, kWave));
        }
    if (lane == 0)
        for (int a = 0; a < 3; ++a) {
            red[a][wave] = mn[a];
            red[3 + a][wave] = mx[a];
        }
    __syncthreads();
    float sc[3];
    for (int a = 0; a < 3; ++a) {
        mn[a] = red[a][0];
        mx[a] = red[3 + a][0];
        for (int w = 1; w < kNW; ++w) {
            mn[a] = fminf(mn[a], red[a][w]);
            mx[a] = fmaxf(mx[a], red[3 + a][w]);
        }
        const float ext = mx[a] - mn[a];
        sc[a] = ext > 0.f && ext < INFINITY ? 16.f / ext : 0.f;
        if (!(mn[a] > -INFINITY)) mn[a] = 0.f;
    }
    // each thread's points: i = tid + r * BLOCK; their cells and order inside
    uint32_t cell[kPer], within[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int i = tid + r * BLOCK;
        if (i < cnt) {
            cell[r] = morton4(xb[3 * i + 0], mn[0], sc[0]) |
                      (morton4(xb[3 * i + 1], mn[1], sc[1]) << 1) |
                      (morton4(xb[3 * i + 2], mn[2], sc[2]) << 2);
            within[r] = atomicAdd(&cell_start[cell[r]], 1u);
        }
    }
    __syncthreads();
    // exclusive scan of the cell counts: kCells / BLOCK consecutive cells per thread
    constexpr int kCpt = kCells / BLOCK;
    uint32_t c_[kCpt], run = 0;
#pragma unroll
    for (int c = 0; c < kCpt; ++c) {
        c_[c] = cell_start[tid * kCpt + c];
        run += c_[c];
    }
    uint32_t incl = run;  // inclusive scan over the wave's lanes
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)incl, off, kWave);
        if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    uint32_t base = incl - run;
    for (int w = 0; w < wave; ++w) base += wsum[w];
#pragma unroll
    for (int c = 0; c < kCpt; ++c) {
        cell_start[tid * kCpt + c] = base;
        base += c_[c];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int i = tid + r * BLOCK;
        if (i < cnt) {
            const uint32_t pos = cell_start[cell[r]] + within[r];
            ob[pos] = make_float4(xb[3 * i + 0], xb[3 * i + 1], xb[3 * i + 2],
                                  __uint_as_float((uint32_t)(lo + i)));
        }
    }
}

// The exchange words of one cloud and batch parity: three for each of the
// G * rg candidates and two for each of the G bounds, both counts rounded up to
// a multiple of 64 (a gather's lanes past the end read within the set).
__host__ __device__ __forceinline__ int pad64(int n) { return (n + 63) & ~63; }
__host__ __device__ __forceinline__ int fps_set_words(int G, int rg) {
    return 3 * pad64(G * rg) + 2 * pad64(G);
}

// STAGED: the exchange words go through LDS (clouds of more than 64
// workgroups or 128 candidates); otherwise straight into registers. GROUPED:
// the points come from the grouped slices (`grouped`) and folds are culled by
// each wave's box. Each combination is its own kernel, so that none carries
// another's registers.
// LDS position of published word w of a set of Q candidates (three words
// each, candidate-major) and its bounds: word i of candidate q goes to
// i * (Q + kStagePad) + q; the bounds keep their order after the three
// arrays. The pad moves the arrays' starts to different LDS banks whatever Q.
constexpr int kStagePad = 8;
__device__ __forceinline__ int stage_pos(int w, int Q) {
    return w < 3 * Q ? (w % 3) * (Q + kStagePad) + w / 3 : w + 2 * kStagePad;
}

template <int PPT, int BLOCK, int CPL, bool STAGED, bool GROUPED>
__global__ __launch_bounds__(BLOCK) void fps_batch_kernel(
    const float* __restrict__ xyz, const float4* __restrict__ grouped, int N, int M,
    int start_idx, int G, int slice, int RG,
    int64_t* __restrict__ out_idx, float* __restrict__ out_xyz, uint64_t* __restrict__ words,
    uint32_t* __restrict__ status, uint32_t spin_limit,
    const int64_t* __restrict__ seg, int nseg) {
    constexpr int NW = BLOCK / kWave;
    // Wave 0 certifies; the others hold points. Waves go round-robin over the
    // 4 SIMDs of a CU, so wave 0 shares its SIMD with waves 4, 8, 12, which
    // hold points too; wave 0 runs at the highest priority, the point waves
    // one below it, above the waves of other kernels sharing the CU (about
    // 0.5% on the 100k-point cloud). (Leaving those three waves without
    // points, so nothing else issues on wave 0's SIMD, measured slower: 1.23
    // against 1.17 ms on the 100k-point cloud).
    static_assert(NW % 4 == 0 && 2 * (NW - 1) <= kWave, "wave count");
    // Certified centres of the batch: x, y, z bits and the point's index. An
    // entry is written before the count that includes it (LDS performs one
    // wave's operations in issue order), and readers load the count first.
    __shared__ uint4 cen[kFpsMaxBatch];
    __shared__ uint4 sink_rec[kWave];  // stores of the certifying wave's other lanes
    __shared__ int sink_cnt[kWave];
    __shared__ int cen_count, cen_done, sh_t, sh_abort, sh_gather_abort, sh_pub;
    // reports of the point waves (m, index, x, y; z) and each wave's bound
    // (m, index), one entry per lane of the reading wave: the entries past the
    // last report or wave stay empty
    __shared__ uint4 rep[kWave];
    __shared__ uint32_t rep_z[kWave];
    __shared__ uint2 bnd[kWave];
    __shared__ uint4 live_a[kWave * CPL];  // compacted live candidates: m, index, x, y
    __shared__ uint32_t live_z[kWave * CPL];  // and z
    // the gathered words (STAGED), then the bounds as published. With fewer
    // than eight slots per lane the candidates' three words go to three
    // arrays (stage_pos), so reading them back by candidate is a contiguous
    // load per word (100k points: 0.998 -> 0.966 ms); the eight-slot kernels,
    // whose point waves gather the set, keep the published order (2^20
    // points: 4.93 -> 5.18 ms with the arrays, 5.07 without the pad).
    constexpr bool kSoA = CPL < 8;
    extern __shared__ uint64_t stage[];
    // loads per lane in flight per poll of a staged gather (32 spill registers)
    constexpr int kPoll = 16;

    // this workgroup's cloud
    int g;
    int64_t xrow0, orow0, jbase;
    uint64_t* cw;  // the cloud's exchange words
    if (seg) {
        const int b = seg_find(seg, nseg, blockIdx.x);
        const int64_t* rec = seg_record(seg, nseg, b);
        G = (int)(seg[b + 1] - seg[b]);
        g = (int)(blockIdx.x - seg[b]);
        N = (int)rec[kFrXCnt];
        slice = (N + G - 1) / G;
        M = (int)rec[kFrOCnt];
        start_idx = (int)rec[kFrStart];
        RG = (int)rec[kFrRG];
        xrow0 = rec[kFrXOff];
        orow0 = rec[kFrOOff];
        jbase = rec[kFrIdxBase];
        cw = words + rec[kFrWOff];
    } else {
        const int b = blockIdx.x / G;
        g = blockIdx.x - b * G;
        xrow0 = (int64_t)b * N;
        orow0 = (int64_t)b * M;
        jbase = 0;
        cw = words + (size_t)b * 2 * fps_set_words(G, RG);
    }
    const int tid = threadIdx.x;
    const int wave = uniform(tid / kWave);
    const int lane = tid % kWave;
    const float* xb = xyz + xrow0 * 3;
    const int lo = g * slice;
    const int cnt = min(N, lo + slice) - lo;  // >= 1
    const int NPW = NW - 1;
    const bool point_wave = wave != 0;
    const int pw = wave - 1;  // index among the point waves
    const int u = pw * kWave + lane;          // point-thread id
    const int wbase = pw * kWave * PPT;       // first slice position of this wave

    float px[PPT], py[PPT], pz[PPT];
    uint32_t pm[PPT], pj[PPT];  // pj: the points' indices (GROUPED)
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
        const int r = u * PPT + p;
        const bool real = point_wave && r < cnt;
        const size_t j = (size_t)lo + (real ? r : 0);
        if constexpr (GROUPED) {
            const float4 e = grouped[xrow0 + (int64_t)j];
            px[p] = e.x;
            py[p] = e.y;
            pz[p] = e.z;
            pj[p] = real ? f2u(e.w) : kNone;  // padding loses every tie
        } else {
            px[p] = xb[3 * j + 0];
            py[p] = xb[3 * j + 1];
            pz[p] = xb[3 * j + 2];
        }
        pm[p] = real ? 0x7F800000u : 0u;  // +inf for points, +0 for padding
    }
    // GROUPED: the wave's box over its real points, and the largest m of the
    // wave as of the last exchange (keys only decrease, so it stays an upper
    // bound until the next); a wave with no real point never folds
    float bx0 = 0.f, by0 = 0.f, bz0 = 0.f, bx1 = 0.f, by1 = 0.f, bz1 = 0.f;
    uint32_t wmax = 0x7F800000u;
    bool wave_real = false;
    if constexpr (GROUPED) {
        float l[3] = {INFINITY, INFINITY, INFINITY}, h[3] = {-INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            if (point_wave && u * PPT + p < cnt) {
                l[0] = fminf(l[0], px[p]);
                l[1] = fminf(l[1], py[p]);
                l[2] = fminf(l[2], pz[p]);
                h[0] = fmaxf(h[0], px[p]);
                h[1] = fmaxf(h[1], py[p]);
                h[2] = fmaxf(h[2], pz[p]);
            }
        }
        // a NaN coordinate: no box (the wave always folds)
        bool nan_pt = false;
#pragma unroll
        for (int p = 0; p < PPT; ++p)
            nan_pt |= point_wave && u * PPT + p < cnt && (px[p] != px[p] || py[p] != py[p] || pz[p] != pz[p]);
#pragma unroll
        for (int a = 0; a < 3; ++a)
            for (int off = 32; off >= 1; off >>= 1) {
                l[a] = fminf(l[a], __shfl_xor(l[a], off, kWave));
                h[a] = fmaxf(h[a], __shfl_xor(h[a], off, kWave));
            }
        // (the lane read takes 32-bit integers: pass the bits)
        bx0 = u2f(uniform(f2u(l[0])));
        by0 = u2f(uniform(f2u(l[1])));
        bz0 = u2f(uniform(f2u(l[2])));
        bx1 = u2f(uniform(f2u(h[0])));
        by1 = u2f(uniform(f2u(h[1])));
        bz1 = u2f(uniform(f2u(h[2])));
        wave_real = point_wave && cnt > wbase;
        if (ballot(nan_pt) != 0) {
            bx0 = by0 = bz0 = -INFINITY;
            bx1 = by1 = bz1 = INFINITY;
        }
    }

    int64_t* ob = out_idx + orow0;
    float* oxb = out_xyz ? out_xyz + orow0 * 3 : nullptr;
    if (tid == 0) {
        const float sx = xb[(size_t)3 * start_idx + 0], sy = xb[(size_t)3 * start_idx + 1],
                    sz = xb[(size_t)3 * start_idx + 2];
        cen[0] = make_uint4(f2u(sx), f2u(sy), f2u(sz), (uint32_t)start_idx);
        cen_count = 1;
        cen_done = 1;
        sh_t = 1;
        sh_abort = 0;
        sh_gather_abort = 0;
        sh_pub = 0;
        if (g == 0) {
            ob[0] = jbase + start_idx;
            if (oxb) { oxb[0] = sx; oxb[1] = sy; oxb[2] = sz; }
        }
    }
    if (wave == 0) {
        rep[lane] = make_uint4(0u, kNone, 0u, 0u);
        rep_z[lane] = 0u;
        bnd[lane] = make_uint2(0u, kNone);
        __builtin_amdgcn_s_setprio(3);
    } else {
        __builtin_amdgcn_s_setprio(2);
    }
    __syncthreads();

    uint32_t batch = 0;
    int out_t0 = 0;  // output slot of the current batch's first centre (0: c_0, written above)
    while (true) {
        // ---- point waves: fold in the centres of the current batch as they come
        if (point_wave) {
            // outputs are written here, not by the certifying wave, so that
            // wave never waits on a global store
            const bool writer = g == 0 && pw == 0 && out_t0 >= 1;
            int a = 0;
            while (true) {
                const int d = __hip_atomic_load(&cen_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                __asm__ __volatile__("" ::: "memory");
                const int n = __hip_atomic_load(&cen_count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                __asm__ __volatile__("" ::: "memory");
                if (writer) {
                    for (int i = a + lane; i < n; i += kWave) {
                        const uint4 c = cen[i];
                        ob[out_t0 + i] = jbase + c.w;
                        if (oxb) {
                            oxb[3 * (out_t0 + i) + 0] = u2f(c.x);
                            oxb[3 * (out_t0 + i) + 1] = u2f(c.y);
                            oxb[3 * (out_t0 + i) + 2] = u2f(c.z);
                        }
                    }
                }
                if constexpr (!GROUPED) {
                    // the next entry's load goes out while this one folds
                    if (a < n) {
                        uint4 c = cen[a];
                        for (; a < n; ++a) {
                            const uint4 nx = cen[a + 1 < n ? a + 1 : a];
#pragma unroll
                            for (int p = 0; p < PPT; ++p)
                                pm[p] = min(pm[p], f2u(s32(u2f(c.x), u2f(c.y), u2f(c.z), px[p], py[p], pz[p])));
                            c = nx;
                        }
                    }
                }
                if (!wave_real) a = n;  // nothing to fold (not GROUPED: a == n already)
                // GROUPED: up to four centres at a time, their loads in flight
                // together (for the plain fold this measured slower: 100k
                // points 1.074 against 1.038 ms)
                while (a < n) {
                    const int k = min(n - a, 4);
                    uint4 cc[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) cc[i] = cen[a + (i < k ? i : 0)];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (i >= k) break;  // wave-uniform
                        const uint4 c = cc[i];
                        if constexpr (GROUPED) {
                            // the centre's lower bound to the box: per axis
                            // the gap in the distance's own float operations,
                            // whose rounding is monotone, so it never exceeds
                            // the distance of any point in the box. At or
                            // above the wave's largest m, no m of the wave
                            // changes.
                            const float X = u2f(c.x), Y = u2f(c.y), Z = u2f(c.z);
                            const float gx = fmaxf(fmaxf(bx0 - X, X - bx1), 0.f);
                            const float gy = fmaxf(fmaxf(by0 - Y, Y - by1), 0.f);
                            const float gz = fmaxf(fmaxf(bz0 - Z, Z - bz1), 0.f);
                            const float lb = (gx * gx + gy * gy) + gz * gz;
                            if (lb >= u2f(wmax)) continue;  // wave-uniform; false for NaN
                        }
#pragma unroll
                        for (int p = 0; p < PPT; ++p)
                            pm[p] = min(pm[p], f2u(s32(u2f(c.x), u2f(c.y), u2f(c.z), px[p], py[p], pz[p])));
                    }
                    a += k;
                }
                if (d) break;  // done was set after the last count: n is final
                __builtin_amdgcn_s_sleep(1);
            }
        }
        __syncthreads();
        const int t0 = sh_t;
        if (t0 >= M || sh_abort) break;
        ++batch;
        out_t0 = t0;
        if (wave == 0) {
            if (lane == 0) {
                cen_count = 0;
                cen_done = 0;
            }
        } else if (point_wave) {
            // ---- point waves: the two largest keys of this wave (its reports)
            // and a bound, the third largest. Per thread first: its three
            // largest keys in position order (strict > keeps the earlier,
            // smaller-index point first on ties), with the coordinates of the
            // first two.
            // (GROUPED: positions are not in index order, so equal keys
            // compare indices)
            uint32_t m1 = pm[0], m2 = 0, m3 = 0;
            int p1 = 0, p2 = -1, p3 = -1;
            float x1 = px[0], y1 = py[0], z1 = pz[0], x2 = 0.f, y2 = 0.f, z2 = 0.f;
            uint32_t j1 = pj[0], j2 = kNone, j3 = kNone;  // GROUPED
#pragma unroll
            for (int p = 1; p < PPT; ++p) {
                const uint32_t v = pm[p];
                bool a1, a2, a3;
                if constexpr (GROUPED) {
                    const uint32_t jv = pj[p];
                    a1 = v > m1 || (v == m1 && jv < j1);
                    a2 = !a1 && (p2 < 0 || v > m2 || (v == m2 && jv < j2));
                    a3 = !a1 && !a2 && (p3 < 0 || v > m3 || (v == m3 && jv < j3));
                    j3 = a1 || a2 ? j2 : (a3 ? jv : j3);
                    j2 = a1 ? j1 : (a2 ? jv : j2);
                    j1 = a1 ? jv : j1;
                } else {
                    a1 = v > m1;
                    a2 = !a1 && (p2 < 0 || v > m2);
                    a3 = !a1 && !a2 && (p3 < 0 || v > m3);
                }
                // shift down the entries the new key displaces
                m3 = a1 || a2 ? m2 : (a3 ? v : m3);
                p3 = a1 || a2 ? p2 : (a3 ? p : p3);
                m2 = a1 ? m1 : (a2 ? v : m2);
                p2 = a1 ? p1 : (a2 ? p : p2);
                x2 = a1 ? x1 : (a2 ? px[p] : x2);
                y2 = a1 ? y1 : (a2 ? py[p] : y2);
                z2 = a1 ? z1 : (a2 ? pz[p] : z2);
                m1 = a1 ? v : m1;
                p1 = a1 ? p : p1;
                x1 = a1 ? px[p] : x1;
                y1 = a1 ? py[p] : y1;
                z1 = a1 ? pz[p] : z1;
            }
            const int pos = lo + wbase + lane * PPT;  // index of this thread's first point
            // index of this thread's point p (-1: none)
            auto pidx = [&](int p) -> uint32_t {
                if constexpr (GROUPED) {
                    uint32_t j = kNone;
#pragma unroll
                    for (int q = 0; q < PPT; ++q) j = p == q ? pj[q] : j;
                    return j;
                } else {
                    return (uint32_t)(pos + p);
                }
            };
            // the k-th report is a real point only if the wave holds more than
            // k real points (real positions come first and win ties)
            const int reals = cnt - wbase;
            uint32_t am, aj, bm, bj, cm_, cj_;
            int al, bl, cl;
            // (GROUPED: lanes are not in index order either)
            auto wmax_key = [&](uint32_t m, uint32_t j, bool use, uint32_t& om, uint32_t& oj,
                                int& ol) {
                if constexpr (GROUPED)
                    wave_max_key_any(m, j, use, om, oj, ol);
                else
                    wave_max_key(m, j, use, om, oj, ol);
            };
            wmax_key(m1, pidx(p1), true, am, aj, al);
            if constexpr (GROUPED) wmax = am;
            const uint32_t ax = lane_value(f2u(x1), al), ay = lane_value(f2u(y1), al),
                           az = lane_value(f2u(z1), al);
            const bool in1 = lane == al;
            // second: lane al offers its second key, the others their first
            wmax_key(in1 ? m2 : m1, pidx(in1 ? p2 : p1), !in1 || p2 >= 0, bm, bj, bl);
            const uint32_t bx = lane_value(f2u(in1 ? x2 : x1), bl < 0 ? 0 : bl),
                           by = lane_value(f2u(in1 ? y2 : y1), bl < 0 ? 0 : bl),
                           bz = lane_value(f2u(in1 ? z2 : z1), bl < 0 ? 0 : bl);
            // bound: the largest key not reported
            const bool in2 = lane == bl;
            const int taken = (int)in1 + (int)in2;
            const uint32_t nm = taken == 0 ? m1 : (taken == 1 ? m2 : m3);
            const int np = taken == 0 ? p1 : (taken == 1 ? p2 : p3);
            wmax_key(nm, pidx(np), np >= 0, cm_, cj_, cl);
            if (lane == 0) {
                rep[2 * pw + 0] = make_uint4(am, reals > 0 ? aj : kNone, ax, ay);
                rep_z[2 * pw + 0] = az;
                rep[2 * pw + 1] = make_uint4(bm, reals > 1 && bl >= 0 ? bj : kNone, bx, by);
                rep_z[2 * pw + 1] = bz;
                const bool bv = reals > 2 && cl >= 0;
                bnd[pw] = make_uint2(bv ? cm_ : 0u, bv ? cj_ : kNone);
            }
        }
        __syncthreads();
        // A staged set of more than one wave-0 poll (over 16 loads per lane;
        // eight candidate slots per lane, up to 2048 words): the point waves
        // gather it into LDS instead, all of it in one round trip. They start once wave 0 has issued this workgroup's words (a
        // flag in LDS): polling earlier only adds uncached traffic that slows
        // the exchange itself.
        if constexpr (STAGED && CPL >= 8) {
            if (G > 1 && point_wave && G * (3 * RG + 2) > 16 * kWave) {
                constexpr int kNpt = (NW - 1) * kWave;
                constexpr int kHelp = (2048 + kNpt - 1) / kNpt;
                const uint32_t tag = batch;
                const int words_total = G * (3 * RG + 2);
                const uint64_t* set = cw + (size_t)(batch & 1) * fps_set_words(G, RG);
                uint32_t spins = 0;
                while (__hip_atomic_load(&sh_pub, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) !=
                       (int)batch) {
                    if (++spins > spin_limit) break;  // wave 0 has stopped: its own poll times out too
                    __builtin_amdgcn_s_sleep(1);
                }
                if (words_total > kHelp * kNpt) {
                    __hip_atomic_store(&sh_gather_abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                } else {
                    while (true) {
                        uint64_t v[kHelp];
#pragma unroll
                        for (int k = 0; k < kHelp; ++k) {
                            const int w = u + k * kNpt;
                            v[k] = w < words_total ? __hip_atomic_load(&set[w], __ATOMIC_RELAXED,
                                                                       __HIP_MEMORY_SCOPE_AGENT)
                                                   : tag8(0, tag);
                        }
                        bool ready = true;
#pragma unroll
                        for (int k = 0; k < kHelp; ++k)
                            ready &= (uint32_t)(v[k] & 0xFFu) == (tag & 0xFFu);
                        if (ballot(!ready) == 0) {
#pragma unroll
                            for (int k = 0; k < kHelp; ++k) {
                                const int w = u + k * kNpt;
                                if (w < words_total) stage[kSoA ? stage_pos(w, G * RG) : w] = v[k] >> 8;
                            }
                            break;
                        }
                        if (++spins > spin_limit) {
                            __hip_atomic_store(&sh_gather_abort, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_WORKGROUP);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
                __syncthreads();  // the set is in LDS (wave 0 meets this after publishing)
            }
        }
        if (wave != 0) continue;

        // ---- wave 0: exchange, then certify centres ----------------------------
        // Reports r = 2 * wave + k (k = 0, 1): the waves are in index order,
        // but a wave's two reports are in key order, so the larger key comes
        // first even when its index is the larger. The candidates that wave 0
        // certifies must be in index order (the first lane holding the
        // largest key must hold the smallest index: two keys that differ at
        // the exchange can become equal as centres are folded in), so the
        // reports of a wave are put in index order wherever they become
        // candidates.
        uint32_t beta_m = 0, beta_j = kNone;
        uint32_t abort = 0;
        uint32_t total = 0;  // live candidates, compacted into live_a / live_z
        // A candidate stays only if it can still be certified in this batch
        // (key > beta; keys only decrease): in index order into the list. The
        // best candidate is always kept: its key is the largest of the cloud.
        auto keep = [&](bool in, uint32_t m, uint32_t j, uint32_t x, uint32_t y, uint32_t z) {
            const bool live = in && j != kNone && key_gt(m, j, beta_m, beta_j);
            const uint64_t mk = ballot(live);
            if (live) {
                const uint32_t q = total + lanes_below(mk);
                live_a[q] = make_uint4(m, j, x, y);
                live_z[q] = z;
            }
            total += (uint32_t)__popcll(mk);
        };
        {
            const uint4 r = rep[lane];  // lane = report (empty past the last)
            const uint32_t rz = rep_z[lane];
            const uint2 wbd = bnd[lane];  // lane = wave (empty past the last)
            if (G == 1) {
                int l;
                wave_max_key(wbd.x, wbd.y, wbd.y != kNone, beta_m, beta_j, l);
                // the pair's smaller index to its even lane (an empty report,
                // index kNone, sorts last)
                const uint4 rp = rep[lane ^ 1];
                const uint32_t rpz = rep_z[lane ^ 1];
                const bool sw = (lane & 1) == 0 ? rp.y < r.y : rp.y > r.y;
                keep(true, sw ? rp.x : r.x, sw ? rp.y : r.y, sw ? rp.z : r.z, sw ? rp.w : r.w,
                     sw ? rpz : rz);
            } else {
                // publish this workgroup's RG best reports (in index order) and
                // its bound: the best of the wave bounds and unpublished reports
                // the loads the bound and the slots need, issued before the
                // selection so that their latency hides behind it
                const uint4 r0 = rep[(2 * lane) & (kWave - 1)];
                const uint4 r1 = rep[(2 * lane + 1) & (kWave - 1)];
                const uint32_t pj = rep[lane ^ 1].y;  // the pair's other report
                uint64_t alive = ballot(r.y != kNone);  // reports not yet taken
                uint64_t sel = 0;
                for (int k = 0; k < RG && alive != 0; ++k) {
                    const bool a = __builtin_amdgcn_inverse_ballot_w64(alive);
                    const uint32_t mx = wave_max_u32(a ? r.x : 0u);
                    uint64_t tm = alive & ballot(r.x == mx);
                    if (GROUPED && (tm & (tm - 1))) {
                        // the waves are not in index order: the smallest index
                        const bool in = (tm >> lane) & 1ull;
                        const uint32_t jm = ~wave_max_u32(in ? ~r.y : 0u);
                        tm &= ballot(r.y == jm);
                    }
                    const int l = (int)__builtin_ctzll(tm);
                    sel |= 1ull << l;
                    alive &= ~(1ull << l);
                }
                // a wave's keys are ordered: report 0 >= report 1 >= bound, so
                // its best unpublished key is the first of them not published
                const bool p0 = (sel >> ((2 * lane) & 63)) & 1ull,
                           p1 = (sel >> ((2 * lane + 1) & 63)) & 1ull;
                const bool wl = lane < NPW;
                const uint32_t um = !p0 ? r0.x : (!p1 ? r1.x : wbd.x);
                const uint32_t uj = !wl ? kNone : (!p0 ? r0.y : (!p1 ? r1.y : wbd.y));
                uint32_t gm, gj;
                int gl;
                if constexpr (GROUPED)
                    wave_max_key_any(um, uj, uj != kNone, gm, gj, gl);
                else
                    wave_max_key(um, uj, uj != kNone, gm, gj, gl);
                // This batch's word set: the three words of candidate q = g * RG
                // + rank at 3q, then the two of each workgroup's bound (each
                // workgroup's words are contiguous). The set is sized for Q =
                // G * RG rounded up to 64 candidates and G rounded up to 64
                // bounds, so that every lane of a gather loads within it.
                const uint32_t tag = batch;
                const int Q = G * RG;
                uint64_t* set = cw + (size_t)(batch & 1) * fps_set_words(G, RG);
                const int nsel = __popcll(sel);
                // the published slot, in index order: when both reports of a
                // wave are published, the smaller index takes the first slot
                int slot = (int)lanes_below(sel);
                if ((sel >> (lane ^ 1)) & 1ull)
                    slot += (lane & 1) == 0 ? (pj < r.y ? 1 : 0) : (pj > r.y ? -1 : 0);
                if constexpr (GROUPED) {
                    // the waves are not in index order: rank among the
                    // published reports by index
                    slot = 0;
                    for (uint64_t t = sel; t != 0; t &= t - 1)
                        slot += lane_value(r.y, (int)__builtin_ctzll(t)) < r.y ? 1 : 0;
                }
                auto put = [&](uint64_t* w, uint64_t v) {
                    __hip_atomic_store(w, tag8(v, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                };
                auto put_candidate = [&](int q, uint32_t m, uint32_t j, uint32_t x, uint32_t y,
                                         uint32_t z) {
                    uint64_t w0, w1, w2;
                    pack_candidate(m, j, x, y, z, w0, w1, w2);
                    uint64_t* w = set + (size_t)q * 3;
                    put(w, w0);
                    put(w + 1, w1);
                    put(w + 2, w2);
                };
                if ((sel >> lane) & 1ull) put_candidate(g * RG + slot, r.x, r.y, r.z, r.w, rz);
                if (nsel < RG) {
                    // unused candidate ranks are published as empty
                    for (int k = nsel + lane; k < RG; k += kWave)
                        put_candidate(g * RG + k, 0u, kNone, 0u, 0u, 0u);
                }
                if (lane == 0) {
                    put(set + 3 * Q + 2 * g, gm);
                    put(set + 3 * Q + 2 * g + 1, gj);
                    if (STAGED && CPL >= 8)
                        __hip_atomic_store(&sh_pub, (int)batch, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
                }
                auto poll = [&](uint64_t w) {
                    return __hip_atomic_load(&set[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                };
                auto shows_tag = [&](uint64_t v) { return (uint32_t)(v & 0xFFu) == (tag & 0xFFu); };
                // beta: the largest bound over the workgroups (lane order =
                // workgroup order = index order)
                auto merge_bound = [&](bool in, uint32_t m, uint32_t j) {
                    uint32_t om, oj;
                    int ol;
                    wave_max_key(m, j, in && j != kNone, om, oj, ol);
                    if (ol >= 0 && (beta_j == kNone || key_gt(om, oj, beta_m, beta_j))) {
                        beta_m = om;
                        beta_j = oj;
                    }
                };
                if constexpr (!STAGED) {
                    // Gather straight into registers: lane l polls candidates
                    // k * 64 + l and the bound of workgroup l, every load of
                    // the poll in flight at once.
                    constexpr int KC = CPL < 2 ? CPL : 2;
                    uint64_t c0[KC], c1[KC], c2[KC], b0, b1;
                    uint32_t spins = 0;
                    // the host launches this form only for sets it holds
                    if (G > kWave || Q > KC * kWave) abort = 1;
                    while (!abort) {
#pragma unroll
                        for (int k = 0; k < KC; ++k) {
                            if (k * kWave >= Q) break;  // wave-uniform
                            const int q = k * kWave + lane;
                            c0[k] = poll(3 * q);
                            c1[k] = poll(3 * q + 1);
                            c2[k] = poll(3 * q + 2);
                        }
                        b0 = poll(3 * Q + 2 * lane);
                        b1 = poll(3 * Q + 2 * lane + 1);
                        // padding slots are never written
                        bool ready = lane >= G || (shows_tag(b0) && shows_tag(b1));
#pragma unroll
                        for (int k = 0; k < KC; ++k) {
                            if (k * kWave >= Q) break;
                            ready &= k * kWave + lane >= Q ||
                                     (shows_tag(c0[k]) && shows_tag(c1[k]) && shows_tag(c2[k]));
                        }
                        if (ballot(!ready) == 0) break;
                        if (++spins > spin_limit) { abort = 1; break; }
                        __builtin_amdgcn_s_sleep(1);
                    }
                    if (!abort) {
                        merge_bound(lane < G, (uint32_t)(b0 >> 8), (uint32_t)(b1 >> 8));
#pragma unroll
                        for (int k = 0; k < KC; ++k) {
                            if (k * kWave >= Q) break;
                            const int q = k * kWave + lane;
                            uint32_t m, j, x, y, z;
                            unpack_candidate(c0[k] >> 8, c1[k] >> 8, c2[k] >> 8, m, j, x, y, z);
                            keep(q < Q, m, j, x, y, z);
                        }
                    }
                } else {
                    // More words than one poll holds: gather the whole set
                    // into LDS, kPoll loads per lane in flight per poll, then
                    // read it back by candidate.
                    const int words_total = 3 * Q + 2 * G;
                    const bool coop = CPL >= 8 && words_total > 16 * kWave;
                    if (coop) {
                        __syncthreads();  // the point waves' gather (above) is done
                        abort = (uint32_t)__hip_atomic_load(&sh_gather_abort, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_WORKGROUP);
                    }
                    for (int w0 = 0; w0 < words_total && !abort && !coop; w0 += kPoll * kWave) {
                        uint32_t spins = 0;
                        while (true) {
                            uint64_t v[kPoll];
#pragma unroll
                            for (int k = 0; k < kPoll; ++k) {
                                const int w = w0 + k * kWave + lane;
                                v[k] = w < words_total ? poll(w) : tag8(0, tag);
                            }
                            bool ready = true;
#pragma unroll
                            for (int k = 0; k < kPoll; ++k) ready &= shows_tag(v[k]);
                            if (ballot(!ready) == 0) {
#pragma unroll
                                for (int k = 0; k < kPoll; ++k) {
                                    const int w = w0 + k * kWave + lane;
                                    if (w < words_total) stage[kSoA ? stage_pos(w, Q) : w] = v[k] >> 8;
                                }
                                break;
                            }
                            if (++spins > spin_limit) { abort = 1; break; }
                            __builtin_amdgcn_s_sleep(1);
                        }
                    }
                    __builtin_amdgcn_s_waitcnt(0);  // LDS writes of this wave complete
                    __builtin_amdgcn_wave_barrier();
                    if (!abort) {
                        uint64_t cw0[CPL], cw1[CPL], cw2[CPL];
#pragma unroll
                        for (int k = 0; k < CPL; ++k) {
                            const int q = k * kWave + lane;
                            const int qq = q < Q ? q : 0;
                            const uint64_t* c = stage + (kSoA ? qq : 3 * qq);
                            cw0[k] = c[0];
                            cw1[k] = c[kSoA ? Q + kStagePad : 1];
                            cw2[k] = c[kSoA ? 2 * (Q + kStagePad) : 2];
                        }
                        // each lane's best bound over workgroups lane, lane + 64,
                        // ..., then one reduction over the lanes (not in
                        // index order: ties go by index)
                        const uint64_t* bw = stage + 3 * Q + (kSoA ? 2 * kStagePad : 0);
                        if (G <= kWave) {
                            const bool in = lane < G;
                            merge_bound(in, in ? (uint32_t)bw[lane * 2 + 0] : 0u,
                                        in ? (uint32_t)bw[lane * 2 + 1] : kNone);
                        } else {
                            uint32_t lm = 0, lj = kNone;
                            for (int wg = lane; wg < G; wg += kWave) {
                                const uint32_t m = (uint32_t)bw[wg * 2 + 0],
                                               j = (uint32_t)bw[wg * 2 + 1];
                                if (j != kNone && (lj == kNone || key_gt(m, j, lm, lj))) {
                                    lm = m;
                                    lj = j;
                                }
                            }
                            uint32_t om, oj;
                            int ol;
                            wave_max_key_any(lm, lj, lj != kNone, om, oj, ol);
                            if (ol >= 0 && (beta_j == kNone || key_gt(om, oj, beta_m, beta_j))) {
                                beta_m = om;
                                beta_j = oj;
                            }
                        }
#pragma unroll
                        for (int k = 0; k < CPL; ++k) {
                            const int q = k * kWave + lane;
                            uint32_t m, j, x, y, z;
                            unpack_candidate(cw0[k], cw1[k], cw2[k], m, j, x, y, z);
                            keep(q < Q, m, j, x, y, z);
                        }
                    }
                }
            }
        }
        // the live candidates, lane-major: `used` slots per lane
        uint32_t cm[CPL], cj[CPL], cxv[CPL], cyv[CPL], czv[CPL];
        int used = CPL;
        if (!abort) {
            used = (int)((total + kWave - 1) / kWave);  // >= 1: the best is live
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int s = 0; s < CPL; ++s) {
                const int qq = lane * used + s;
                const bool in = s < used && qq < (int)total;
                const uint4 e = live_a[in ? qq : 0];
                const uint32_t ez = live_z[in ? qq : 0];
                cm[s] = in ? e.x : 0u;
                cj[s] = in ? e.y : kNone;
                cxv[s] = in ? e.z : 0u;
                cyv[s] = in ? e.w : 0u;
                czv[s] = in ? ez : 0u;
            }
        }
        int t = t0;
        if (!abort) {
            // The loop for U candidate slots per lane (U = `used`, after the
            // compaction above; usually 1), so no step touches empty slots.
            auto certify = [&](auto u_) {
                constexpr int U = decltype(u_)::value;
                int nc = 0;
                while (true) {
                    // largest key among the valid candidates (lane-major = index order)
                    uint32_t lm = 0, lj = kNone, lx = 0, ly = 0, lz = 0;
#pragma unroll
                    for (int s = 0; s < U; ++s) {
                        const bool b = cj[s] != kNone && (lj == kNone || cm[s] > lm);
                        lm = b ? cm[s] : lm;
                        lj = b ? cj[s] : lj;
                        lx = b ? cxv[s] : lx;
                        ly = b ? cyv[s] : ly;
                        lz = b ? czv[s] : lz;
                    }
                    uint32_t km, kj;
                    int kl;
                    wave_max_key(lm, lj, lj != kNone, km, kj, kl);
                    if (nc > 0 && !key_gt(km, kj, beta_m, beta_j)) break;  // not certified
                    const float X = u2f(lane_value(lx, kl));
                    const float Y = u2f(lane_value(ly, kl));
                    const float Z = u2f(lane_value(lz, kl));
                    if (lane == 0) {
                        cen[nc] = make_uint4(f2u(X), f2u(Y), f2u(Z), kj);
                        __asm__ __volatile__("" ::: "memory");  // entry before count
                        __hip_atomic_store(&cen_count, nc + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    }
                    ++nc;
                    ++t;
#pragma unroll
                    for (int s = 0; s < U; ++s)
                        cm[s] = min(cm[s], f2u(s32(X, Y, Z, u2f(cxv[s]), u2f(cyv[s]), u2f(czv[s]))));
                    if (t >= M || nc == kFpsMaxBatch) break;
                }
            };
            // One or two slots per lane (the usual cases). The live candidates
            // come first in lane-major order; the other slots hold key 0,
            // which the min update keeps at 0, so they can win only when every
            // live key is 0, and then lane 0, slot 0 (live) is the first entry
            // holding the maximum. So no slot needs a validity mask. With
            // several slots each lane offers its best one, the earlier slot on
            // ties (the smaller index).
            //
            // Steps go in blocks of kCertBlock with no exit test inside: a
            // step's test (key above the bound's, or the batch's first centre)
            // is only recorded, and each step writes its entry and folds
            // anyway. A step's entry stays in scalar registers (the lane reads
            // that the fold needs anyway, plus the index); after the block
            // v_writelane puts entry s into lane s and lanes 0-3 store the
            // four entries at once, so no step waits behind an LDS store (a
            // per-step store of the winning lane's entry, with the other lanes
            // writing sink slots, measured 1.09 against 1.02 ms on the 100k
            // cloud). After the block the count takes the leading steps that
            // passed; the entries past it are never read, and the candidates'
            // keys are not used after the batch, so the steps past a failure
            // need no undoing. (A test inside the loop costs a branch per
            // step, which the loop's latency chain pays in full.) A key equal
            // to the bound's can still pass by its index: a block that stops
            // there rewinds to its start, replays the steps that passed and
            // goes on one step at a time with the full test.
            //
            // As certified centres fold into the candidates, keys fall to the
            // bound and below, and those candidates can no longer be
            // certified in this batch. Every eight steps (after a block that
            // passed) a loop of two or more slots counts the candidates whose
            // m is at least the bound's (a superset of the live ones); when
            // they fit in half the slots it compacts them, in the same
            // lane-major order, and goes on with half the slots. A candidate
            // dropped this way has m below the bound's and can never be the
            // certified maximum again; one kept with m equal to it is
            // harmless (it is tested like any other).
            auto certify_fast = [&](auto self, auto c_, int nc0) -> void {
                constexpr int C = decltype(c_)::value;  // slots per lane, <= CPL
                uint32_t m[C], xs[C], ys[C], zs[C], js[C];
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    m[c] = cm[c];
                    xs[c] = cxv[c];
                    ys[c] = cyv[c];
                    zs[c] = czv[c];
                    js[c] = cj[c];
                }
                const int limit = min(M - t0, kFpsMaxBatch);
                int nc = nc0;
                auto fold = [&](float X, float Y, float Z) {
#pragma unroll
                    for (int c = 0; c < C; ++c)
                        m[c] = min(m[c], f2u(s32(X, Y, Z, u2f(xs[c]), u2f(ys[c]), u2f(zs[c]))));
                };
                // the lane's best slot and its entry: a tree of strict
                // compares, so on equal keys the earlier slot (the smaller
                // index) is kept
                auto best = [&](uint32_t& lm, uint32_t& wx, uint32_t& wy, uint32_t& wz,
                                uint32_t& wj) {
                    uint32_t bm[C], bx_[C], by_[C], bz_[C], bj[C];
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        bm[c] = m[c];
                        bx_[c] = xs[c];
                        by_[c] = ys[c];
                        bz_[c] = zs[c];
                        bj[c] = js[c];
                    }
#pragma unroll
                    for (int w = 1; w < C; w *= 2) {
#pragma unroll
                        for (int c = 0; c + w < C; c += 2 * w) {
                            const bool t = bm[c + w] > bm[c];
                            bm[c] = t ? bm[c + w] : bm[c];
                            bx_[c] = t ? bx_[c + w] : bx_[c];
                            by_[c] = t ? by_[c + w] : by_[c];
                            bz_[c] = t ? bz_[c + w] : bz_[c];
                            bj[c] = t ? bj[c + w] : bj[c];
                        }
                    }
                    lm = bm[0];
                    wx = bx_[0];
                    wy = by_[0];
                    wz = bz_[0];
                    wj = bj[0];
                };
                // the candidates' LDS loads are complete here, so the loop's
                // only LDS operations are its own stores, which need no wait
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                bool tied = false;
                while (true) {
                    uint32_t r[C];  // the block's start
#pragma unroll
                    for (int c = 0; c < C; ++c) r[c] = m[c];
                    // the block's entries and each step's largest key,
                    // wave-uniform (scalar registers)
                    uint32_t sx[kCertBlock], sy[kCertBlock], sz[kCertBlock], sj[kCertBlock],
                        sm[kCertBlock];
#pragma unroll
                    for (int s = 0; s < kCertBlock; ++s) {
                        uint32_t lm, wx, wy, wz, wj;
                        best(lm, wx, wy, wz, wj);
                        const uint32_t mx = wave_max_u32(lm);
                        const int kl = (int)__builtin_ctzll(ballot(lm == mx));
                        sm[s] = mx;
                        sx[s] = lane_value(wx, kl);
                        sy[s] = lane_value(wy, kl);
                        sz[s] = lane_value(wz, kl);
                        sj[s] = lane_value(wj, kl);
                        fold(u2f(sx[s]), u2f(sy[s]), u2f(sz[s]));
                    }
                    static_assert(kCertBlock == 4, "entry lanes");
                    // entry s and step s's largest key into lane s. The scalar
                    // registers come from v_readlane, and a VALU read of an
                    // SGPR that a VALU wrote needs two wait states on gfx950
                    // (the compiler keeps them in its own code but cannot see
                    // inside an asm statement), hence the s_nop 1 that leads
                    // each one. The steps' tests against the bound are then
                    // two compares of `mxv` for the whole block.
                    uint32_t ex = 0, ey = 0, ez = 0, ej = 0, mxv = 0;
#define POINTOPS_ENTRY_LANE(S)                                                        \
    __asm__("s_nop 1\n\t"                                                              \
            "v_writelane_b32 %0, %5, " #S "\n\t"                                        \
            "v_writelane_b32 %1, %6, " #S "\n\t"                                        \
            "v_writelane_b32 %2, %7, " #S "\n\t"                                        \
            "v_writelane_b32 %3, %8, " #S "\n\t"                                        \
            "v_writelane_b32 %4, %9, " #S                                              \
            : "+v"(ex), "+v"(ey), "+v"(ez), "+v"(ej), "+v"(mxv)                         \
            : "s"(sx[S]), "s"(sy[S]), "s"(sz[S]), "s"(sj[S]), "s"(sm[S]));
                    POINTOPS_ENTRY_LANE(0)
                    POINTOPS_ENTRY_LANE(1)
                    POINTOPS_ENTRY_LANE(2)
                    POINTOPS_ENTRY_LANE(3)
#undef POINTOPS_ENTRY_LANE
                    // one store for the block's entries, before the count that
                    // takes them (the entries past a failure are never read)
                    if (lane < kCertBlock && nc + lane < limit)
                        cen[nc + lane] = make_uint4(ex, ey, ez, ej);
                    constexpr uint64_t kSteps = (1ull << kCertBlock) - 1;
                    uint32_t fail = (uint32_t)(ballot(mxv <= beta_m) & kSteps);
                    const uint32_t tie = (uint32_t)(ballot(mxv == beta_m) & kSteps);
                    if (nc == 0) fail &= ~1u;  // the batch's first centre: the cloud's largest key
                    const int room = limit - nc;
                    if (room < kCertBlock) fail |= ~0u << room;
                    const int pass = fail ? (int)__builtin_ctz(fail) : kCertBlock;
                    nc += pass;
                    __asm__ __volatile__("" ::: "memory");  // entries before the count
                    __hip_atomic_store(lane == 0 ? &cen_count : &sink_cnt[lane], nc,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    if (pass == kCertBlock) {
                        if constexpr (C >= 2) {
                            if (((nc - nc0) & 7) == 0) {
                                constexpr int H = C / 2;
                                uint64_t keepm[C];
                                uint32_t n = 0;
#pragma unroll
                                for (int c = 0; c < C; ++c) {
                                    keepm[c] = ballot(js[c] != kNone && m[c] >= beta_m);
                                    n += (uint32_t)__popcll(keepm[c]);
                                }
                                if (n >= 1 && n <= (uint32_t)(H * kWave)) {
                                    // position in lane-major order: the kept
                                    // slots of lower lanes, then this lane's
                                    // earlier slots
                                    uint32_t q = 0;
#pragma unroll
                                    for (int c = 0; c < C; ++c) q += lanes_below(keepm[c]);
                                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                                    for (int c = 0; c < C; ++c) {
                                        if ((keepm[c] >> lane) & 1ull) {
                                            live_a[q] = make_uint4(m[c], js[c], xs[c], ys[c]);
                                            live_z[q] = zs[c];
                                            ++q;
                                        }
                                    }
                                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                                    for (int h = 0; h < H; ++h) {
                                        const int qq = lane * H + h;
                                        const bool in = qq < (int)n;
                                        const uint4 e = live_a[in ? qq : 0];
                                        const uint32_t ez = live_z[in ? qq : 0];
                                        cm[h] = in ? e.x : 0u;
                                        cj[h] = in ? e.y : kNone;
                                        cxv[h] = in ? e.z : 0u;
                                        cyv[h] = in ? e.w : 0u;
                                        czv[h] = in ? ez : 0u;
                                    }
                                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                                    self(self, std::integral_constant<int, H>{}, nc);
                                    return;
                                }
                            }
                        }
                        continue;
                    }
                    tied = pass < room && ((tie >> pass) & 1u);
                    if (tied) {
#pragma unroll
                        for (int c = 0; c < C; ++c) m[c] = r[c];
                        for (int i = nc - pass; i < nc; ++i) {
                            const uint4 c = cen[i];
                            fold(u2f(c.x), u2f(c.y), u2f(c.z));
                        }
                    }
                    break;
                }
                // one step at a time with the full test: a key equal to the
                // bound's passes when its index is smaller
                while (tied && nc < limit) {
                    uint32_t lm, wx, wy, wz, wj;
                    best(lm, wx, wy, wz, wj);
                    const uint32_t mx = wave_max_u32(lm);
                    const int kl = (int)__builtin_ctzll(ballot(lm == mx));
                    if (!key_gt(mx, lane_value(wj, kl), beta_m, beta_j)) break;
                    const bool win = lane == kl;
                    *(win ? &cen[nc] : &sink_rec[lane]) = make_uint4(wx, wy, wz, wj);
                    __asm__ __volatile__("" ::: "memory");  // entry before count
                    __hip_atomic_store(win ? &cen_count : &sink_cnt[lane], nc + 1,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    ++nc;
                    fold(u2f(lane_value(wx, kl)), u2f(lane_value(wy, kl)),
                         u2f(lane_value(wz, kl)));
                }
                t = t0 + nc;
            };
            if (used <= 1)
                certify_fast(certify_fast, std::integral_constant<int, 1>{}, 0);
            else if (CPL >= 2 && used <= 2)
                certify_fast(certify_fast, std::integral_constant<int, (CPL >= 2 ? 2 : 1)>{}, 0);
            else if (CPL >= 4 && used <= 3)
                certify_fast(certify_fast, std::integral_constant<int, (CPL >= 4 ? 3 : 1)>{}, 0);
            else if (CPL >= 4 && used <= 4)
                certify_fast(certify_fast, std::integral_constant<int, (CPL >= 4 ? 4 : 1)>{}, 0);
            else
                certify(std::integral_constant<int, CPL>{});
        }
        if (lane == 0) {
            sh_t = t;
            sh_abort = (int)abort;
            __hip_atomic_store(&cen_done, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    if (sh_abort && tid == 0) {
        atomicOr(status, 1u);
        if (g == 0)
            for (int v = sh_t; v < M; ++v) ob[v] = -1;
    }
    // header word 1: the exchanges of the launch's first cloud
    if (blockIdx.x == 0 && tid == 0) status[1] = G > 1 ? batch : 0u;
}

// Workspace: a 256-byte header (word 0: status, word 1: the exchanges of the
// launch's first cloud), then two parity sets of G slots per cloud.
size_t fps_workspace_bytes(int64_t B, int64_t G) {
    return G > 1 ? 256 + (size_t)B * 2 * (size_t)G * sizeof(FpsSlot) : 256;
}

template <int PPT, int BLOCK>
static hipError_t launch_fps_t(dim3 grid, size_t lds, hipStream_t stream, const float* xyz, int N,
                               int M, int start_idx, int G, int slice, int64_t* out_idx,
                               float* out_xyz, FpsSlot* slots, uint32_t* status, uint32_t spin,
                               const int64_t* seg, int nseg) {
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)fps_kernel<PPT, BLOCK>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((fps_kernel<PPT, BLOCK>), grid, dim3(BLOCK), lds, stream, xyz, N, M,
                       start_idx, G, slice, out_idx, out_xyz, slots, status, spin, seg, nseg);
    return hipGetLastError();
}

template <int BLOCK, int... P>
static hipError_t dispatch_ppt(int ppt, std::integer_sequence<int, P...>, dim3 grid, size_t lds,
                               hipStream_t stream, const float* xyz, int N, int M, int start_idx,
                               int G, int slice, int64_t* out_idx, float* out_xyz, FpsSlot* slots,
                               uint32_t* status, uint32_t spin, const int64_t* seg, int nseg) {
    hipError_t e = hipErrorInvalidValue;
    ((ppt == P + 1 ? (void)(e = launch_fps_t<P + 1, BLOCK>(grid, lds, stream, xyz, N, M,
                                                            start_idx, G, slice, out_idx,
                                                            out_xyz, slots, status, spin, seg,
                                                            nseg))
                   : (void)0), ...);
    return e;
}

// Dense: B * G workgroups. Ragged (seg != nullptr): `units` workgroups, one
// per cloud, `N` = the largest cloud (it sizes the LDS copy); B, M, start_idx
// and G are unused.
hipError_t launch_fps(const float* xyz, int64_t B, int64_t N, int64_t M, int64_t start_idx,
                      int64_t* out_idx, float* out_xyz, void* workspace, int G, int ppt,
                      int block, uint32_t spin_limit, hipStream_t stream, const int64_t* seg,
                      int nseg, int64_t units) {
    if (seg) G = 1;
    const int slice = (int)((N + G - 1) / G);
    uint32_t* status = (uint32_t*)workspace;
    FpsSlot* slots = (FpsSlot*)((char*)workspace + 256);
    const size_t lds = (size_t)slice * 3 * sizeof(float);
    dim3 grid((unsigned)(seg ? units : B * G));
    if (block == 256)
        return dispatch_ppt<256>(ppt, std::make_integer_sequence<int, 16>{}, grid, lds, stream,
                                 xyz, (int)N, (int)M, (int)start_idx, G, slice, out_idx, out_xyz,
                                 slots, status, spin_limit, seg, nseg);
    if (block == 1024)
        return dispatch_ppt<1024>(ppt, std::make_integer_sequence<int, 16>{}, grid, lds, stream,
                                  xyz, (int)N, (int)M, (int)start_idx, G, slice, out_idx, out_xyz,
                                  slots, status, spin_limit, seg, nseg);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- batched launch

// Points per thread for which the batched kernel is built.
constexpr int kBatchPpt[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16};

int fps_batch_ppt_round(int ppt) {
    for (int v : kBatchPpt)
        if (v >= ppt) return v;
    return -1;
}

int fps_batch_set_words(int G, int rg) { return fps_set_words(G, rg); }

int fps_batch_point_waves(int block) { return block / kWave - 1; }

size_t fps_batch_workspace_bytes(int64_t B, int64_t G, int rg) {
    return G > 1 ? 256 + (size_t)B * 2 * (size_t)fps_set_words((int)G, rg) * sizeof(uint64_t) : 256;
}

// Dynamic LDS: the staged word set, for clouds of more than 64 workgroups or
// 128 candidates (smaller sets are gathered straight into registers; with up
// to 256 candidates the registers of a four-slot gather measured slower than
// the staging they save: 100k points, 63 workgroups of 4 candidates, 1.077
// against 1.040 ms).
size_t fps_batch_lds_bytes(int G, int rg) {
    return G > 64 || G * rg > 128 ? ((size_t)G * (3 * rg + 2) + 2 * kStagePad) * 8 : 0;
}

// The (points per thread, block, candidates per lane, staged, grouped)
// configurations that are built.
template <int PPT_, int BLOCK_, int CPL_, bool STAGED_, bool GROUPED_ = false>
struct BatchCfg {
    static constexpr int PPT = PPT_, BLOCK = BLOCK_, CPL = CPL_;
    static constexpr bool STAGED = STAGED_, GROUPED = GROUPED_;
};

template <int P>
using BatchCfgsFor =
    std::tuple<BatchCfg<P, 1024, 1, false>, BatchCfg<P, 1024, 2, false>,
               BatchCfg<P, 1024, 1, true>, BatchCfg<P, 1024, 2, true>, BatchCfg<P, 1024, 4, true>,
               BatchCfg<P, 1024, 8, true>, BatchCfg<P, 256, 1, false>, BatchCfg<P, 256, 1, true>>;

// Grouped slices: 1024 threads, 4 to 10 points per thread (slices of at most
// kGroupMaxSlice points); staged sets have more than 128 candidates.
template <int P>
using GroupedCfgsFor =
    std::tuple<BatchCfg<P, 1024, 1, false, true>, BatchCfg<P, 1024, 2, false, true>,
               BatchCfg<P, 1024, 2, true, true>, BatchCfg<P, 1024, 4, true, true>,
               BatchCfg<P, 1024, 8, true, true>>;

using BatchCfgs = decltype(std::tuple_cat(
    BatchCfgsFor<1>{}, BatchCfgsFor<2>{}, BatchCfgsFor<3>{}, BatchCfgsFor<4>{}, BatchCfgsFor<5>{},
    BatchCfgsFor<6>{}, BatchCfgsFor<8>{}, BatchCfgsFor<10>{}, BatchCfgsFor<12>{},
    BatchCfgsFor<16>{}, GroupedCfgsFor<4>{}, GroupedCfgsFor<5>{}, GroupedCfgsFor<6>{},
    GroupedCfgsFor<8>{}, GroupedCfgsFor<10>{}));

bool fps_batch_group_built(int ppt, int block) {
    return block == 1024 && (ppt == 4 || ppt == 5 || ppt == 6 || ppt == 8 || ppt == 10);
}

// Calls fn(Cfg{}) for the built configuration matching the runtime values;
// false when none does. A launch that needs dynamic LDS stages its words.
template <typename Fn>
static bool with_batch_cfg(int ppt, int block, int cpl, size_t lds, bool group, Fn&& fn) {
    const bool staged = lds > 0;
    return std::apply(
        [&](auto... cfg) {
            return ((decltype(cfg)::PPT == ppt && decltype(cfg)::BLOCK == block &&
                     decltype(cfg)::CPL == cpl && decltype(cfg)::STAGED == staged &&
                     decltype(cfg)::GROUPED == group && (fn(cfg), true)) ||
                    ...);
        },
        BatchCfgs{});
}

// Largest number of batched-FPS workgroups that are resident at once.
hipError_t fps_batch_capacity(int ppt, int block, int cpl, size_t lds, bool group, int cus,
                              int* out) {
    hipError_t e = hipErrorInvalidValue;
    int per_cu = 0;
    with_batch_cfg(ppt, block, cpl, lds, group, [&](auto cfg) {
        using C = decltype(cfg);
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu,
            (const void*)fps_batch_kernel<C::PPT, C::BLOCK, C::CPL, C::STAGED, C::GROUPED>,
            C::BLOCK, lds);
    });
    *out = per_cu * cus;
    return e;
}

// Bytes of the grouped points (dense clouds with `group`), after the exchange
// part of the workspace, which is all that the per-call clear touches.
size_t fps_batch_group_bytes(int64_t B, int64_t N) { return (size_t)B * (size_t)N * 16; }

size_t fps_batch_group_offset(int64_t B, int64_t G, int rg) {
    return (fps_batch_workspace_bytes(B, G, rg) + 255) & ~(size_t)255;
}

// Dense: B * G workgroups, exchange words after the 256-byte header, and with
// `group` the grouped points after them (written first by one workgroup per
// slice). Ragged (seg != nullptr): `units` workgroups, `words` = the exchange
// words (each cloud's record locates its own), `lds` = the largest stage of
// any cloud; B, N, M, start_idx, G, rg and group are unused.
hipError_t launch_fps_batch(const float* xyz, int64_t B, int64_t N, int64_t M, int64_t start_idx,
                            int64_t* out_idx, float* out_xyz, void* workspace, int G, int ppt,
                            int block, int rg, int cpl, bool group, uint32_t spin_limit,
                            hipStream_t stream, const int64_t* seg, int nseg, int64_t units,
                            uint64_t* seg_words, size_t seg_lds) {
    if (seg) group = false;
    const int slice = seg ? 0 : (int)((N + G - 1) / G);
    uint32_t* status = (uint32_t*)workspace;
    uint64_t* words = seg ? seg_words : (uint64_t*)((char*)workspace + 256);
    const size_t lds = seg ? seg_lds : fps_batch_lds_bytes(G, rg);
    const unsigned grid = (unsigned)(seg ? units : B * G);
    float4* grouped = nullptr;
    if (group) {
        if (G < 2 || slice > kGroupMaxSlice || !fps_batch_group_built(ppt, block))
            return hipErrorInvalidValue;
        grouped = (float4*)((char*)workspace + fps_batch_group_offset(B, G, rg));
        hipLaunchKernelGGL((fps_group_kernel<1024>), dim3(grid), dim3(1024), 0, stream, xyz,
                           (int)N, G, slice, grouped);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipError_t e = hipErrorInvalidValue;
    with_batch_cfg(ppt, block, cpl, lds, group, [&](auto cfg) {
        using C = decltype(cfg);
        hipLaunchKernelGGL((fps_batch_kernel<C::PPT, C::BLOCK, C::CPL, C::STAGED, C::GROUPED>),
                           dim3(grid), dim3(C::BLOCK), lds, stream, xyz, grouped, (int)N, (int)M,
                           (int)start_idx, G, slice, rg, out_idx, out_xyz, words, status,
                           spin_limit, seg, nseg);
        e = hipGetLastError();
    });
    return e;
}

// Device-side clear of the workspace (a plain fill kernel rather than a memset
// node, so the call can be captured into a graph).
__global__ void fps_clear_kernel(uint32_t* __restrict__ w, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        w[i] = 0;
}

hipError_t launch_fps_clear(void* workspace, size_t bytes, hipStream_t stream) {
    const size_t n = bytes / 4;
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(fps_clear_kernel, dim3(blocks), dim3(256), 0, stream, (uint32_t*)workspace, n);
    return hipGetLastError();
}

}  // namespace pointops
