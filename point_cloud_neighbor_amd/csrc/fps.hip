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
#include <algorithm>
#include <utility>

#include "common.h"

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
    uint32_t* __restrict__ status, uint32_t spin_limit) {
    constexpr int NWAVE = BLOCK / kWave;
    extern __shared__ float lds_xyz[];  // the slice's coordinates, AoS
    __shared__ uint32_t wave_m[2][NWAVE];
    __shared__ uint32_t wave_j[2][NWAVE];
    __shared__ uint32_t result[2][6];    // m, index, x, y, z, abort

    const int b = blockIdx.x / G;
    const int g = blockIdx.x - b * G;
    const int tid = threadIdx.x;
    const int wave = uniform(tid / kWave);
    const int lane = tid % kWave;
    const float* xb = xyz + (size_t)b * N * 3;
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
    int64_t* ob = out_idx + (size_t)b * M;
    float* oxb = out_xyz ? out_xyz + (size_t)b * M * 3 : nullptr;
    if (g == 0 && tid == 0) {
        ob[0] = c;
        if (oxb) { oxb[0] = cx; oxb[1] = cy; oxb[2] = cz; }
    }
    FpsSlot* cs = slots + (size_t)b * 2 * G;
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
            ob[t] = c;
            if (oxb) { oxb[3 * t + 0] = cx; oxb[3 * t + 1] = cy; oxb[3 * t + 2] = cz; }
        }
    }
}

// Workspace: a 256-byte header (status word), then two parity sets of G slots
// per cloud.
size_t fps_workspace_bytes(int64_t B, int64_t G) {
    return G > 1 ? 256 + (size_t)B * 2 * (size_t)G * sizeof(FpsSlot) : 256;
}

template <int PPT, int BLOCK>
static hipError_t launch_fps_t(dim3 grid, size_t lds, hipStream_t stream, const float* xyz, int N,
                               int M, int start_idx, int G, int slice, int64_t* out_idx,
                               float* out_xyz, FpsSlot* slots, uint32_t* status, uint32_t spin) {
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)fps_kernel<PPT, BLOCK>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((fps_kernel<PPT, BLOCK>), grid, dim3(BLOCK), lds, stream, xyz, N, M,
                       start_idx, G, slice, out_idx, out_xyz, slots, status, spin);
    return hipGetLastError();
}

template <int BLOCK, int... P>
static hipError_t dispatch_ppt(int ppt, std::integer_sequence<int, P...>, dim3 grid, size_t lds,
                               hipStream_t stream, const float* xyz, int N, int M, int start_idx,
                               int G, int slice, int64_t* out_idx, float* out_xyz, FpsSlot* slots,
                               uint32_t* status, uint32_t spin) {
    hipError_t e = hipErrorInvalidValue;
    ((ppt == P + 1 ? (void)(e = launch_fps_t<P + 1, BLOCK>(grid, lds, stream, xyz, N, M,
                                                            start_idx, G, slice, out_idx,
                                                            out_xyz, slots, status, spin))
                   : (void)0), ...);
    return e;
}

hipError_t launch_fps(const float* xyz, int64_t B, int64_t N, int64_t M, int64_t start_idx,
                      int64_t* out_idx, float* out_xyz, void* workspace, int G, int ppt,
                      int block, uint32_t spin_limit, hipStream_t stream) {
    const int slice = (int)((N + G - 1) / G);
    uint32_t* status = (uint32_t*)workspace;
    FpsSlot* slots = (FpsSlot*)((char*)workspace + 256);
    const size_t lds = (size_t)slice * 3 * sizeof(float);
    dim3 grid((unsigned)(B * G));
    if (block == 256)
        return dispatch_ppt<256>(ppt, std::make_integer_sequence<int, 16>{}, grid, lds, stream,
                                 xyz, (int)N, (int)M, (int)start_idx, G, slice, out_idx, out_xyz,
                                 slots, status, spin_limit);
    if (block == 1024)
        return dispatch_ppt<1024>(ppt, std::make_integer_sequence<int, 16>{}, grid, lds, stream,
                                  xyz, (int)N, (int)M, (int)start_idx, G, slice, out_idx, out_xyz,
                                  slots, status, spin_limit);
    return hipErrorInvalidValue;
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
