// Dense first-K Ball Query for gfx950.
//
// Contract: project page "mps-pointops", section "The operators in equations",
// "Ball Query: first K within a radius", and the "Numerical contracts" page,
// "Selection and output": for each query, the references j with
// s32(q, x_j) < R2 in increasing j; the first K are kept as (j, s32), the
// remaining slots are (-1, +0.0f). R2 = fl32(r32 * r32) is formed on the host.
//
// Mapping: one wave per group of QW queries of one cloud. The queries are
// wave-uniform (scalar registers); the 64 lanes take 64 consecutive
// references per block, so one v_cmp gives a 64-bit mask that is already in
// input order. The rank of a hit inside its block is mbcnt(mask), its output
// slot is count + rank, and count += popcount(mask): the first-K order of the
// project page's SIMD kernel (one SIMD group per query, prefix rank per block),
// here with wave64 ballots and several queries sharing every block of
// references. A query stops contributing once it has K hits; the wave stops
// when all of its queries have.
//
// Ragged batches (a cloud table, see segments.h): waves are numbered cloud
// after cloud, QW queries each, and scan their own cloud's references.
#include "common.h"
#include "segments.h"

namespace pointops {

template <int QW>
__global__ __launch_bounds__(kWave) void ball_query_kernel(
    const float* __restrict__ query, const float* __restrict__ ref, int Q, int P, float r2,
    int K, float* __restrict__ out_d2, int64_t* __restrict__ out_idx,
    const int64_t* __restrict__ seg, int nseg) {
    // this wave's cloud: its first query row, reference row, sizes
    int64_t qrow0, rrow0, ibase, unit;
    if (seg) {
        const int b = seg_find(seg, nseg, blockIdx.x);
        const int64_t* rec = seg_record(seg, nseg, b);
        unit = blockIdx.x - seg[b];
        qrow0 = rec[kSrQOff];
        Q = (int)rec[kSrQCnt];
        rrow0 = rec[kSrROff];
        P = (int)rec[kSrRCnt];
        ibase = rec[kSrIdxBase];
    } else {
        unit = blockIdx.x;
        qrow0 = (int64_t)blockIdx.y * Q;
        rrow0 = (int64_t)blockIdx.y * P;
        ibase = 0;
    }
    const int row0 = (int)unit * QW;
    const int lane = threadIdx.x;
    const float* qb = query + qrow0 * 3;
    const float* xb = ref + rrow0 * 3;
    const size_t out0 = (size_t)(qrow0 + row0) * (size_t)K;

    float qx[QW], qy[QW], qz[QW];
    int cnt[QW];
#pragma unroll
    for (int i = 0; i < QW; ++i) {
        const int row = row0 + i < Q ? row0 + i : Q - 1;
        qx[i] = qb[(size_t)3 * row + 0];
        qy[i] = qb[(size_t)3 * row + 1];
        qz[i] = qb[(size_t)3 * row + 2];
        cnt[i] = row0 + i < Q ? 0 : K;  // rows past the end take no hits
    }

    // Software-pipelined reference loads: block n+1 is in flight while block n
    // is compared. Lanes past the last reference hold NaN coordinates, whose
    // distance compares false against R2, so no separate range test is needed.
    const float nan = __builtin_nanf("");
    float nx = nan, ny = nan, nz = nan;
    if (lane < P) {
        nx = xb[(size_t)3 * lane + 0];
        ny = xb[(size_t)3 * lane + 1];
        nz = xb[(size_t)3 * lane + 2];
    }
    for (int base = 0; base < P; base += kWave) {
        const int j = base + lane;
        const float x = nx, y = ny, z = nz;
        const int jn = j + kWave;
        nx = ny = nz = nan;
        if (jn < P) {
            nx = xb[(size_t)3 * jn + 0];
            ny = xb[(size_t)3 * jn + 1];
            nz = xb[(size_t)3 * jn + 2];
        }
        bool live = false;
#pragma unroll
        for (int i = 0; i < QW; ++i) {
            if (cnt[i] < K) {
                const float s = s32(qx[i], qy[i], qz[i], x, y, z);
                const uint64_t m = ballot(s < r2);
                if (m) {
                    const int slot = cnt[i] + (int)lanes_below(m);
                    if (((m >> lane) & 1ull) && slot < K) {
                        out_idx[out0 + (size_t)i * K + slot] = ibase + j;
                        out_d2[out0 + (size_t)i * K + slot] = s;
                    }
                    cnt[i] += __popcll(m);
                }
                live |= cnt[i] < K;
            }
        }
        if (!live) break;
    }

    // Padding: slots count..K-1 of each row hold (-1, +0.0f).
#pragma unroll
    for (int i = 0; i < QW; ++i) {
        if (row0 + i < Q) {
            for (int slot = cnt[i] + lane; slot < K; slot += kWave) {
                out_idx[out0 + (size_t)i * K + slot] = -1;
                out_d2[out0 + (size_t)i * K + slot] = 0.0f;
            }
        }
    }
}

// Launch helper used by the C ABI: grid (ceil(Q / QW), B), one wave per group;
// ragged (seg != nullptr): grid (waves, 1) with waves = the table's
// tile_ptr[nseg], Q and P unused.
hipError_t launch_ball_query(const float* query, const float* ref, int64_t B, int64_t Q,
                             int64_t P, float r2, int64_t K, float* out_d2, int64_t* out_idx,
                             int qw, const int64_t* seg, int nseg, int64_t waves,
                             hipStream_t stream) {
    dim3 block(kWave);
    switch (qw) {
#define POINTOPS_BQ_CASE(W)                                                                  \
    case W: {                                                                                \
        dim3 grid = seg ? dim3((unsigned)waves, 1)                                           \
                        : dim3((unsigned)((Q + W - 1) / W), (unsigned)B);                    \
        hipLaunchKernelGGL(ball_query_kernel<W>, grid, block, 0, stream, query, ref, (int)Q, \
                           (int)P, r2, (int)K, out_d2, out_idx, seg, nseg);                  \
        break;                                                                               \
    }
        POINTOPS_BQ_CASE(1)
        POINTOPS_BQ_CASE(2)
        POINTOPS_BQ_CASE(4)
        POINTOPS_BQ_CASE(8)
        POINTOPS_BQ_CASE(16)
#undef POINTOPS_BQ_CASE
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pointops
