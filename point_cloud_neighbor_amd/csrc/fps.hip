// Farthest point sampling for gfx950: one persistent launch for all steps.
//
// Contract: project page "mps-pointops", section "The operators in equations",
// "Farthest point sampling" (c_0 = start_idx; m_j is the smallest squared
// distance from x_j to a chosen centre; the next centre is the smallest index
// holding the largest m) and section "Contracts" (the start index; the
// remaining slots repeat index 0 once every point is taken).
//
// Mapping. Each cloud is split into G contiguous slices, one workgroup per
// slice, and all G workgroups of a cloud run together for the whole launch
// (the host keeps the grid within what the device holds at once). Every
// thread keeps PPT points of its slice in registers, with their running
// minimum m, so a step reads no global memory: it folds the last centre into
// m, forms the key
//     key_j = (float bits of m_j) << 32 | (0xFFFFFFFF - j)
// (m >= +0, so its bits order like its value; the larger key has the larger m
// and, on equal m, the smaller j) and takes the maximum key over the wave
// (cross-lane shuffles), the workgroup (LDS) and, when G > 1, the cloud (one
// slot per workgroup in device memory, published with a release store of the
// step number and polled with acquire loads; two slot sets alternate by step
// parity). The winner's coordinates travel with its key, read from an LDS copy
// of the slice, so no step waits on a global load of the new centre.
//
// Compared with the project page's design (one threadgroup per cloud running
// every step, and for one large cloud a second dispatch per step to reduce the
// chunk maxima), the reduction here never leaves the launch.
//
// Slices never leave padding slots unowned: a thread slot past the end of its
// slice holds a copy of the slice's first point with that point's index, so its
// key equals that point's key and the maximum is unchanged.
//
// Termination: every poll loop is bounded. A workgroup that waits longer than
// `spin_limit` polls raises the status word and stops; the others then stop on
// their own bound, output slots not reached are -1.
#include "common.h"

namespace pointops {

struct alignas(32) FpsSlot {
    uint64_t key;
    float x, y, z;
    uint32_t tag;  // step number that wrote this slot (0: never)
    uint32_t pad[2];
};

struct FpsBest {
    uint64_t key;
    float x, y, z;
    uint32_t abort;
};

__device__ __forceinline__ uint64_t fps_key(float m, uint32_t nj) {
    return ((uint64_t)f2u(m) << 32) | nj;
}

template <int PPT, int BLOCK>
__global__ __launch_bounds__(BLOCK) void fps_kernel(
    const float* __restrict__ xyz, int N, int M, int start_idx, int G, int slice,
    int64_t* __restrict__ out_idx, float* __restrict__ out_xyz, FpsSlot* __restrict__ slots,
    uint32_t* __restrict__ status, uint32_t spin_limit) {
    constexpr int NWAVE = BLOCK / kWave;
    extern __shared__ float lds_xyz[];  // slice coordinates, AoS
    __shared__ uint64_t wave_key[NWAVE];
    __shared__ FpsBest best_sh[2];  // alternates by step parity

    const int b = blockIdx.x / G;
    const int g = blockIdx.x - b * G;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const float* xb = xyz + (size_t)b * N * 3;
    const int lo = g * slice;
    const int hi = min(N, lo + slice);
    const int cnt = hi - lo;  // >= 1 (host guarantees every slice is non-empty)

    // Stage the slice: registers for the update, LDS for the winner's coordinates.
    for (int i = tid; i < 3 * cnt; i += BLOCK) lds_xyz[i] = xb[(size_t)3 * lo + i];
    float px[PPT], py[PPT], pz[PPT], pm[PPT];
    uint32_t pn[PPT];
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
        int r = tid + p * BLOCK;
        if (r >= cnt) r = 0;  // padding slot: duplicate of the slice's first point
        const size_t j = (size_t)lo + r;
        px[p] = xb[3 * j + 0];
        py[p] = xb[3 * j + 1];
        pz[p] = xb[3 * j + 2];
        pm[p] = __builtin_inff();
        pn[p] = 0xFFFFFFFFu - (uint32_t)j;
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

    for (int t = 1; t < M; ++t) {
        uint64_t best = 0;
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const float d = s32(cx, cy, cz, px[p], py[p], pz[p]);
            pm[p] = fminf(pm[p], d);  // m stays non-NaN: fminf drops a NaN d
            const uint64_t k = fps_key(pm[p], pn[p]);
            best = k > best ? k : best;
        }
        best = wave_max_u64(best);
        if (lane == 0) wave_key[wave] = best;
        __syncthreads();
        if (wave == 0) {
            uint64_t k = lane < NWAVE ? wave_key[lane] : 0;
            k = wave_max_u64(k);
            const int jw = (int)(0xFFFFFFFFu - (uint32_t)k);  // winner of this slice
            const int r = jw - lo;
            float wx = lds_xyz[3 * r + 0], wy = lds_xyz[3 * r + 1], wz = lds_xyz[3 * r + 2];
            uint32_t abort = 0;
            if (G > 1) {
                FpsSlot* set = cs + (size_t)(t & 1) * G;
                if (lane == 0) {
                    set[g].key = k;
                    set[g].x = wx;
                    set[g].y = wy;
                    set[g].z = wz;
                    __hip_atomic_store(&set[g].tag, (uint32_t)t, __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
                // Gather every slice's winner of step t.
                uint64_t gk = 0;
                float gx = 0.f, gy = 0.f, gz = 0.f;
                for (int base = 0; base < G; base += kWave) {
                    const int s = base + lane;
                    uint32_t spins = 0;
                    bool ready = s >= G;
                    while (true) {
                        if (!ready)
                            ready = __hip_atomic_load(&set[s].tag, __ATOMIC_ACQUIRE,
                                                      __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)t;
                        if (__builtin_amdgcn_ballot_w64(!ready) == 0) break;
                        if (++spins > spin_limit) { abort = 1; break; }
                        __builtin_amdgcn_s_sleep(1);
                    }
                    if (abort) break;
                    if (s < G) {
                        const uint64_t sk = set[s].key;
                        if (sk > gk) { gk = sk; gx = set[s].x; gy = set[s].y; gz = set[s].z; }
                    }
                }
                // Cross-lane argmax that carries the coordinates with the key.
                const uint64_t wmax = wave_max_u64(gk);
                const uint64_t own = ballot(gk == wmax);
                const int src = __builtin_ctzll(own);
                k = wmax;
                wx = __shfl(gx, src, kWave);
                wy = __shfl(gy, src, kWave);
                wz = __shfl(gz, src, kWave);
            }
            if (lane == 0) {
                FpsBest& o = best_sh[t & 1];
                o.key = k;
                o.x = wx;
                o.y = wy;
                o.z = wz;
                o.abort = abort;
            }
        }
        __syncthreads();
        // best_sh[t & 1] is next written at step t + 2, after step t + 1's barrier.
        const FpsBest& o = best_sh[t & 1];
        const uint64_t k = o.key;
        cx = o.x;
        cy = o.y;
        cz = o.z;
        const uint32_t abort = o.abort;
        if (abort) {
            if (tid == 0) {
                atomicOr(status, 1u);
                if (g == 0)
                    for (int u = t; u < M; ++u) ob[u] = -1;
            }
            return;
        }
        c = (int)(0xFFFFFFFFu - (uint32_t)k);
        if (g == 0 && tid == 0) {
            ob[t] = c;
            if (oxb) { oxb[3 * t + 0] = cx; oxb[3 * t + 1] = cy; oxb[3 * t + 2] = cz; }
        }
    }
}

// Slot storage the launch needs: 2 parity sets of G slots per cloud, plus a
// 256-byte header holding the status word.
size_t fps_workspace_bytes(int64_t B, int64_t G) {
    return G > 1 ? 256 + (size_t)B * 2 * (size_t)G * sizeof(FpsSlot) : 256;
}

hipError_t launch_fps(const float* xyz, int64_t B, int64_t N, int64_t M, int64_t start_idx,
                      int64_t* out_idx, float* out_xyz, void* workspace, int G, int ppt,
                      int block, uint32_t spin_limit, hipStream_t stream) {
    const int slice = (int)((N + G - 1) / G);
    uint32_t* status = (uint32_t*)workspace;
    FpsSlot* slots = (FpsSlot*)((char*)workspace + 256);
    const size_t lds = (size_t)slice * 3 * sizeof(float);
    dim3 grid((unsigned)(B * G));
#define POINTOPS_FPS_CASE(P, BL)                                                              \
    if (ppt == P && block == BL) {                                                            \
        hipLaunchKernelGGL((fps_kernel<P, BL>), grid, dim3(BL), lds, stream, xyz, (int)N,     \
                           (int)M, (int)start_idx, G, slice, out_idx, out_xyz, slots, status, \
                           spin_limit);                                                       \
        return hipGetLastError();                                                             \
    }
    POINTOPS_FPS_CASE(1, 256)
    POINTOPS_FPS_CASE(2, 256)
    POINTOPS_FPS_CASE(4, 256)
    POINTOPS_FPS_CASE(1, 1024)
    POINTOPS_FPS_CASE(2, 1024)
    POINTOPS_FPS_CASE(4, 1024)
    POINTOPS_FPS_CASE(8, 1024)
    POINTOPS_FPS_CASE(16, 1024)
#undef POINTOPS_FPS_CASE
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
