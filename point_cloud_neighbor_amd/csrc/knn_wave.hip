// Exact k nearest neighbours, one query per wave (k <= 32), for launches with
// few queries per cloud.
//
// Contract: project page "mps-pointops", section "The operators in equations",
// "k nearest neighbors" (sort the references by (s, j), keep the first k,
// return sqrt(s)) and "Numerical contracts", "Selection and output" (exact ties
// go to the smaller reference index) -- the same results as knn.hip.
//
// Mapping. A workgroup of NW waves owns NW * QW queries of one cloud, QW per
// wave, so the queries sit in scalar registers. The cloud's references stream
// through LDS in tiles of kKwTile points: every thread loads its share of the
// next tile into registers (coalesced global loads) while the waves scan the
// current one, then stores it into the other of two buffers, one barrier per
// tile. A wave scans a tile 64 references at a time, one per lane, and each
// reference it reads serves its QW queries: each pair costs the eight float32
// operations of s32 and about one operation of candidate test.
//
// List. The wave keeps, per query, its KL best pairs so far (32, or 16 when
// k <= 16) as 64-bit keys (bits(s) << 32) | j, ascending across lanes
// 0..KL-1: s >= +0, so the high word
// orders like s and the low word breaks ties by index. Lane k-1's key bounds
// the k-th neighbour; because the list holds only earlier references (smaller
// indices), a new reference can enter it only with bits(s) strictly below
// that key's high word, the candidate test.
//
// Merge. Candidates go to an LDS buffer of the query and are merged into the
// list 32 at a time (48 when k <= 16: the list then keeps 16 lanes) by a
// bitonic network of lane moves (wave_list.h).
//
// Ragged batches (a cloud table, see segments.h): workgroups are numbered
// cloud after cloud, NW * QW queries each. A cloud with fewer than k references
// fills the slots it cannot fill with (+inf, -1), as knn.hip does.
#include "common.h"
#include "segments.h"
#include "wave_list.h"

namespace pointops {

constexpr int kKwTile = 1024;            // references per LDS tile
// NW waves per workgroup, QW queries per wave (consecutive rows): each
// reference read from LDS serves the QW queries. KL list lanes: 16 when
// k <= 16 (a 48-entry candidate buffer, so a third fewer merges), else 32.
template <int NW, int QW, int KL>
__global__ __launch_bounds__(NW* kWave) void knn_wave_kernel(
    const float* __restrict__ query, const float* __restrict__ ref, int Q, int P, int k,
    float* __restrict__ out_dist, int64_t* __restrict__ out_idx, const int64_t* __restrict__ seg,
    int nseg, int squared) {
    constexpr int NT = NW * kWave;
    constexpr int PER = kKwTile / NT;  // tile points each thread loads
    static_assert(kKwTile % NT == 0, "tile must split evenly over the threads");
    __shared__ float tile[2][3][kKwTile];
    __shared__ uint64_t cbuf[NW][QW][kWave - KL];

    int64_t qrow0, rrow0, ibase, qtile;
    if (seg) {
        const int b = seg_find(seg, nseg, blockIdx.x);
        const int64_t* rec = seg_record(seg, nseg, b);
        qtile = blockIdx.x - seg[b];
        qrow0 = rec[kSrQOff];
        Q = (int)rec[kSrQCnt];
        rrow0 = rec[kSrROff];
        P = (int)rec[kSrRCnt];
        ibase = rec[kSrIdxBase];
    } else {
        qtile = blockIdx.x;
        qrow0 = (int64_t)blockIdx.y * Q;
        rrow0 = (int64_t)blockIdx.y * P;
        ibase = 0;
    }
    const int lane = lane_id();
    const int tid = threadIdx.x;
    const int w = uniform(tid / kWave);
    const int q0 = ((int)qtile * NW + w) * QW;  // this wave's first query
    const bool active = q0 < Q;  // wave-uniform; idle waves still stage tiles
    const float* xb = ref + rrow0 * 3;

    float qx[QW], qy[QW], qz[QW];
    KwQuery st[QW];
#pragma unroll
    for (int h = 0; h < QW; ++h) {
        const float* qp = query + (qrow0 + (q0 + h < Q ? q0 + h : 0)) * 3;
        qx[h] = qp[0];
        qy[h] = qp[1];
        qz[h] = qp[2];
        // a query past the cloud's last gets bound 0: nothing passes the test
        st[h] = KwQuery{kKwEmpty, q0 + h < Q ? ~0u : 0u, 0, cbuf[w][h]};
    }

    const int ntiles = (P + kKwTile - 1) / kKwTile;
    float rx[PER], ry[PER], rz[PER];
    auto load = [&](int t) {
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int j = t * kKwTile + r * NT + tid;
            rx[r] = ry[r] = rz[r] = 0.0f;
            if (j < P) {
                const float* p = xb + (size_t)3 * j;
                rx[r] = p[0];
                ry[r] = p[1];
                rz[r] = p[2];
            }
        }
    };
    auto store = [&](int slot) {
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            tile[slot][0][r * NT + tid] = rx[r];
            tile[slot][1][r * NT + tid] = ry[r];
            tile[slot][2][r * NT + tid] = rz[r];
        }
    };

    if (ntiles > 0) {
        load(0);
        store(0);
    }
    __syncthreads();
    // The first 64 references all pass the test of an empty list: one pass of
    // the network sorts them into it directly (instead of two buffer merges).
    // A key whose distance bits are all ones stays out, as it never passes
    // the test.
    if (active && ntiles > 0) {
        const float x = tile[0][0][lane], y = tile[0][1][lane], z = tile[0][2][lane];
#pragma unroll
        for (int h = 0; h < QW; ++h) {
            if (q0 + h >= Q) break;
            const uint32_t u = f2u(s32(qx[h], qy[h], qz[h], x, y, z));
            const uint64_t key =
                lane < P && u != ~0u ? ((uint64_t)u << 32) | (uint32_t)lane : kKwEmpty;
            st[h].list = kw_sort_merge(key, lane);
            st[h].bound = lane_value((uint32_t)(st[h].list >> 32), k - 1);
        }
    }
    for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) load(t + 1);
        if (active) {
            const float* tx = tile[t & 1][0];
            const float* ty = tile[t & 1][1];
            const float* tz = tile[t & 1][2];
            const int j0 = t * kKwTile;
            const int n = min(kKwTile, P - j0);  // references in this tile
            // Four chunks at a time (the LDS reads take immediate offsets and
            // overlap), one test of their minimum per query; only when some
            // lane has a candidate are the four offered, in order. Lanes past
            // the cloud (jl >= n, last tile only) take the empty key, which
            // never passes.
            for (int c = t == 0 ? 1 : 0; c * kWave < n; c += 4) {
                uint32_t u[QW][4];
                const bool tail = (c + 4) * kWave > n;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int jl = (c + r) * kWave + lane;  // < kKwTile: in the buffer
                    const float x = tx[jl], y = ty[jl], z = tz[jl];
#pragma unroll
                    for (int h = 0; h < QW; ++h) u[h][r] = f2u(s32(qx[h], qy[h], qz[h], x, y, z));
                }
                if (tail) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int h = 0; h < QW; ++h)
                            if ((c + r) * kWave + lane >= n) u[h][r] = ~0u;
                }
#pragma unroll
                for (int h = 0; h < QW; ++h) {
                    const uint32_t mn = min(min(u[h][0], u[h][1]), min(u[h][2], u[h][3]));
                    if (ballot(mn < st[h].bound)) {
                        // unrolled, so each offer tests its chunk's value in
                        // place (no run-time choice among the four)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            kw_offer<false, KL>(st[h], u[h][r] < st[h].bound, u[h][r],
                                                j0 + (c + r) * kWave + lane, lane, k);
                    }
                }
            }
        }
        if (t + 1 < ntiles) store((t + 1) & 1);
        __syncthreads();
    }
    if (!active) return;

#pragma unroll
    for (int h = 0; h < QW; ++h) {
        if (q0 + h >= Q) break;
        if (st[h].cnt > 0) kw_merge<KL>(st[h], lane, k);
        if (lane < k) {
            const uint64_t e = st[h].list;
            const bool empty = e == kKwEmpty;  // only when the cloud has < k references
            const float s = u2f((uint32_t)(e >> 32));
            const int64_t o = (qrow0 + q0 + h) * k + lane;
            out_dist[o] = squared ? (empty ? 0.0f : s) : (empty ? __builtin_inff() : sqrtf(s));
            out_idx[o] = empty ? (int64_t)-1 : ibase + (int64_t)(uint32_t)e;
        }
    }
}

// Dense: grid (ceil(Q / (nw * qw)), B). Ragged (seg != nullptr): grid (tiles,
// 1), with tiles = the table's tile_ptr[nseg] (nw * qw queries per unit) and
// Q, P unused. Requires 1 <= k <= 32.
hipError_t launch_knn_wave(const float* query, const float* ref, int64_t B, int64_t Q, int64_t P,
                           int64_t k, float* out_dist, int64_t* out_idx, int nw, int qw,
                           const int64_t* seg, int nseg, int64_t tiles, int squared,
                           hipStream_t stream) {
    if (k < 1 || k > kKwBuf) return hipErrorInvalidValue;
    const int per = nw * qw;
    const dim3 grid = seg ? dim3((unsigned)tiles, 1) : dim3((unsigned)((Q + per - 1) / per), (unsigned)B);
#define POINTOPS_KNN_WAVE_CASE(W, H)                                                         \
    if (nw == W && qw == H) {                                                                \
        if (k <= 16)                                                                         \
            hipLaunchKernelGGL((knn_wave_kernel<W, H, 16>), grid, dim3(W * kWave), 0, stream, \
                               query, ref, (int)Q, (int)P, (int)k, out_dist, out_idx, seg,   \
                               nseg, squared);                                               \
        else                                                                                 \
            hipLaunchKernelGGL((knn_wave_kernel<W, H, 32>), grid, dim3(W * kWave), 0, stream, \
                               query, ref, (int)Q, (int)P, (int)k, out_dist, out_idx, seg,   \
                               nseg, squared);                                               \
        return hipGetLastError();                                                            \
    }
    POINTOPS_KNN_WAVE_CASE(4, 1) POINTOPS_KNN_WAVE_CASE(8, 1) POINTOPS_KNN_WAVE_CASE(16, 1)
    POINTOPS_KNN_WAVE_CASE(4, 2) POINTOPS_KNN_WAVE_CASE(8, 2) POINTOPS_KNN_WAVE_CASE(16, 2)
#undef POINTOPS_KNN_WAVE_CASE
    return hipErrorInvalidValue;
}

}  // namespace pointops
