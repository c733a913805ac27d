// Exact k nearest neighbours for gfx950.
//
// Contract: project page "mps-pointops", section "The operators in equations",
// "k nearest neighbors" (sort the references by (s, j), keep the first k,
// return sqrt(s)) and "Numerical contracts", "Selection and output" (exact ties
// go to the smaller reference index).
//
// Mapping. A workgroup owns 64 queries, one per lane, and NW waves; wave w
// scans the w-th contiguous range of the references, in increasing index, so
// every wave sees the same query in the same lane. References are wave-uniform
// and come through scalar loads; each (query, reference) pair costs the eight
// float32 operations of s32 plus one integer minimum per lane.
//
// Keys. A candidate's key is (float bits of s) + 1: s >= +0, so the bits order
// like the values, and the +1 keeps 0 free for the "front" sentinels below and
// 0xFFFFFFFF free for "empty". Every lane keeps a list of KCAP (key, index)
// pairs in registers, sorted ascending; when k < KCAP the first KCAP - k slots
// hold key 0 and never move, so the k real entries are always the last k
// slots and the pruning threshold is the fixed last slot. Because a wave visits
// references in increasing index, an insertion only needs the strict test
// key < list key: an equal key already in the list has the smaller index and
// stays in front, which is the (s, j) order.
//
// Candidates. A reference whose key beats a lane's threshold is appended to
// that lane's buffer in LDS (a few instructions, executed by the lanes that
// hit); when some lane's buffer is nearly full, all lanes fold their buffers
// into their lists with the register insertion. Checking eight references at
// once (a v_min3 chain) keeps the test at about one instruction per pair.
//
// Merge. At the end each wave leaves its list in LDS and wave 0 inserts the
// lists of waves 1..NW-1 in order (all their indices are larger than wave 0's
// and increase with the wave), then writes sqrtf(s) (correctly rounded) and
// the indices.
//
// Ragged batches (a cloud table, see segments.h): workgroups are numbered
// cloud after cloud, 64 queries each, and a cloud's references are its own
// segment. A cloud with fewer than k references fills the slots it cannot
// fill with (+inf, -1): the project page's flat kNN emits only the available
// neighbours in that case.
#include "common.h"
#include "segments.h"

namespace pointops {

constexpr int kKnnGroup = 8;     // references tested per threshold check
constexpr int kKnnBuf = 16;      // candidate slots per lane (>= kKnnGroup + 1)

// Median of three unsigned values.
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    __asm__("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

template <int KCAP>
struct TopK {
    uint32_t key[KCAP];
    int32_t id[KCAP];

    __device__ __forceinline__ void init(int k) {
#pragma unroll
        for (int p = 0; p < KCAP; ++p) {
            key[p] = p < KCAP - k ? 0u : 0xFFFFFFFFu;
            id[p] = -1;
        }
    }

    // Insert (kk, jj); equal keys already present stay first. A key that is not
    // below the last slot (0xFFFFFFFF in particular) changes nothing, so callers
    // insert unconditionally instead of branching.
    __device__ __forceinline__ void insert(uint32_t kk, int32_t jj) {
#pragma unroll
        for (int p = KCAP - 1; p >= 1; --p) {
            const bool before_prev = kk < key[p - 1];  // new entry lands left of p-1
            const bool before_this = kk < key[p];
            id[p] = before_prev ? id[p - 1] : (before_this ? jj : id[p]);
            // sorted list: the new key[p] is the median of key[p-1], kk, key[p]
            // (one v_med3_u32, which the compiler cannot infer; measured
            // faster up to 16 entries, slower at 32)
            key[p] = KCAP <= 16 ? med3_u32(key[p - 1], kk, key[p]) : min(max(key[p - 1], kk), key[p]);
        }
        const bool first = kk < key[0];
        id[0] = first ? jj : id[0];
        key[0] = min(kk, key[0]);
    }

    __device__ __forceinline__ uint32_t last() const { return key[KCAP - 1]; }
};

template <int KCAP, int NW>
__global__ __launch_bounds__(NW* kWave) void knn_kernel(
    const float* __restrict__ query, const float* __restrict__ ref, int Q, int P, int k,
    float* __restrict__ out_dist, int64_t* __restrict__ out_idx, const int64_t* __restrict__ seg,
    int nseg, int squared) {
    // LDS: per wave, kKnnBuf candidate rows during the scan, then KCAP list
    // rows for the merge; row e of wave w is uint2[64] (one entry per lane).
    extern __shared__ uint2 lds[];
    constexpr int ROWS = kKnnBuf > KCAP ? kKnnBuf : KCAP;

    // this workgroup's cloud: its first query row, reference row, sizes
    int64_t qrow0, rrow0, ibase, tile;
    if (seg) {
        const int b = seg_find(seg, nseg, blockIdx.x);
        const int64_t* rec = seg_record(seg, nseg, b);
        tile = blockIdx.x - seg[b];
        qrow0 = rec[kSrQOff];
        Q = (int)rec[kSrQCnt];
        rrow0 = rec[kSrROff];
        P = (int)rec[kSrRCnt];
        ibase = rec[kSrIdxBase];
    } else {
        tile = blockIdx.x;
        qrow0 = (int64_t)blockIdx.y * Q;
        rrow0 = (int64_t)blockIdx.y * P;
        ibase = 0;
    }
    const int lane = threadIdx.x % kWave;
    const int w = uniform((int)(threadIdx.x / kWave));
    const int qi = (int)tile * kWave + lane;
    const bool qvalid = qi < Q;
    const float* qp = query + (qrow0 + (qvalid ? qi : Q - 1)) * 3;
    const float qx = qp[0], qy = qp[1], qz = qp[2];
    const float* xb = ref + rrow0 * 3;
    uint2* buf = lds + (size_t)w * ROWS * kWave;

    const int chunk = (P + NW - 1) / NW;
    const int j0 = w * chunk;
    const int j1 = min(P, j0 + chunk);

    TopK<KCAP> top;
    top.init(k);
    uint32_t lim = top.last() - 1u;  // accept iff bits(s) < lim
    int cnt = 0;

    auto flush = [&]() {
        const int rounds = wave_max_i32(cnt);  // <= kKnnBuf
#pragma unroll 1
        for (int e = 0; e < rounds; ++e) {
            const uint2 c = buf[e * kWave + lane];  // row e < kKnnBuf: in bounds
            top.insert(e < cnt ? c.x : 0xFFFFFFFFu, (int32_t)c.y);
        }
        cnt = 0;
        lim = top.last() - 1u;
    };

    int j = j0;
    for (; j + kKnnGroup <= j1; j += kKnnGroup) {
        const float* rp = xb + (size_t)3 * j;
        uint32_t u[kKnnGroup];
#pragma unroll
        for (int r = 0; r < kKnnGroup; ++r)
            u[r] = f2u(s32(qx, qy, qz, rp[3 * r + 0], rp[3 * r + 1], rp[3 * r + 2]));
        uint32_t mn = u[0];
#pragma unroll
        for (int r = 1; r < kKnnGroup; ++r) mn = min(mn, u[r]);
        if (ballot(mn < lim)) {
#pragma unroll
            for (int r = 0; r < kKnnGroup; ++r) {
                if (u[r] < lim) {
                    buf[cnt * kWave + lane] = make_uint2(u[r] + 1u, (uint32_t)(j + r));
                    ++cnt;
                }
            }
            if (ballot(cnt > kKnnBuf - kKnnGroup)) flush();
        }
    }
    // Ragged tail of this wave's range.
    for (; j < j1; ++j) {
        const float* rp = xb + (size_t)3 * j;
        const uint32_t u = f2u(s32(qx, qy, qz, rp[0], rp[1], rp[2]));
        if (u < lim) {
            buf[cnt * kWave + lane] = make_uint2(u + 1u, (uint32_t)j);
            ++cnt;
        }
        if (ballot(cnt >= kKnnBuf)) flush();
    }
    flush();

    // Merge the NW lists through LDS (rows reused from the candidate buffers)
    // as a tree: in the round of distance d, wave w (a multiple of 2d) inserts
    // the list of wave w + d, whose indices are all larger, so the insertion
    // keeps the (s, j) order; log2(NW) rounds instead of NW - 1 in a row.
    if (NW > 1) {
#pragma unroll
        for (int p = 0; p < KCAP; ++p) buf[p * kWave + lane] = make_uint2(top.key[p], (uint32_t)top.id[p]);
#pragma unroll
        for (int d = 1; d < NW; d *= 2) {
            __syncthreads();
            if (w % (2 * d) == 0) {
                const uint2* other = lds + (size_t)(w + d) * ROWS * kWave;
#pragma unroll 1
                for (int p = 0; p < KCAP; ++p) {
                    const uint2 c = other[p * kWave + lane];
                    // front sentinels (key 0) are skipped; empty slots
                    // (0xFFFFFFFF) insert nothing
                    top.insert(c.x != 0u ? c.x : 0xFFFFFFFFu, (int32_t)c.y);
                }
                // the merged list for the next round; nobody reads this
                // wave's rows in the current one (only rows w + d are read)
                if (2 * d < NW) {
#pragma unroll
                    for (int p = 0; p < KCAP; ++p)
                        buf[p * kWave + lane] = make_uint2(top.key[p], (uint32_t)top.id[p]);
                }
            }
        }
        if (w != 0) return;
    }

    if (!qvalid) return;
    float* od = out_dist + (qrow0 + qi) * k;
    int64_t* oi = out_idx + (qrow0 + qi) * k;
    const int front = KCAP - k;
#pragma unroll
    for (int p = 0; p < KCAP; ++p) {
        if (p >= front) {
            // empty slots remain only when the cloud has fewer than k references
            const bool empty = top.key[p] == 0xFFFFFFFFu;
            const float s = u2f(top.key[p] - 1u);
            od[p - front] = squared ? (empty ? 0.0f : s) : (empty ? __builtin_inff() : sqrtf(s));
            oi[p - front] = empty ? (int64_t)-1 : ibase + top.id[p];
        }
    }
}

// Dense: grid (ceil(Q / 64), B). Ragged (seg != nullptr): grid (tiles, 1), with
// tiles = the table's tile_ptr[nseg] and Q, P unused. squared != 0: out_dist
// holds s itself (the nearest-point distances of the Chamfer distance) and
// empty slots hold (0, -1).
hipError_t launch_knn(const float* query, const float* ref, int64_t B, int64_t Q, int64_t P,
                      int64_t k, float* out_dist, int64_t* out_idx, int kcap, int nw,
                      const int64_t* seg, int nseg, int64_t tiles, int squared,
                      hipStream_t stream) {
    dim3 grid = seg ? dim3((unsigned)tiles, 1) : dim3((unsigned)((Q + kWave - 1) / kWave), (unsigned)B);
#define POINTOPS_KNN_CASE(KC, W)                                                             \
    if (kcap == KC && nw == W) {                                                             \
        constexpr int rows = kKnnBuf > KC ? kKnnBuf : KC;                                    \
        const size_t lds = (size_t)W * rows * kWave * sizeof(uint2);                         \
        if (lds > 65536) {                                                                   \
            hipError_t e = hipFuncSetAttribute((const void*)knn_kernel<KC, W>,               \
                                               hipFuncAttributeMaxDynamicSharedMemorySize,   \
                                               (int)lds);                                    \
            if (e != hipSuccess) return e;                                                   \
        }                                                                                    \
        hipLaunchKernelGGL((knn_kernel<KC, W>), grid, dim3(W * kWave), lds, stream, query,  \
                           ref, (int)Q, (int)P, (int)k, out_dist, out_idx, seg, nseg,        \
                           squared);                                                         \
        return hipGetLastError();                                                            \
    }
    POINTOPS_KNN_CASE(1, 1) POINTOPS_KNN_CASE(1, 4) POINTOPS_KNN_CASE(1, 8)
    POINTOPS_KNN_CASE(2, 1) POINTOPS_KNN_CASE(2, 4) POINTOPS_KNN_CASE(2, 8)
    POINTOPS_KNN_CASE(4, 1) POINTOPS_KNN_CASE(4, 4) POINTOPS_KNN_CASE(4, 8)
    POINTOPS_KNN_CASE(8, 1) POINTOPS_KNN_CASE(8, 4) POINTOPS_KNN_CASE(8, 8)
    POINTOPS_KNN_CASE(16, 1) POINTOPS_KNN_CASE(16, 2) POINTOPS_KNN_CASE(16, 4)
    POINTOPS_KNN_CASE(16, 8)
    POINTOPS_KNN_CASE(32, 1) POINTOPS_KNN_CASE(32, 2) POINTOPS_KNN_CASE(32, 4)
    POINTOPS_KNN_CASE(32, 8)
    POINTOPS_KNN_CASE(64, 1) POINTOPS_KNN_CASE(64, 2)
#undef POINTOPS_KNN_CASE
    return hipErrorInvalidValue;
}

}  // namespace pointops
