// Dense first-K Ball Query for clouds in any order: an index-order scan with a
// budget, then a grid pass for the queries it leaves short of K.
//
// Contract: as ball_query.hip (project page "mps-pointops", section "The
// operators in equations", "Ball Query: first K within a radius"; "Numerical
// contracts", "Selection and output"): the references j with s32(q, x_j) < R2
// in increasing j, the first K kept as (j, s32), padding (-1, +0.0f). The
// project page's roadmap points to spatial structures (a uniform grid) for
// large clouds; this is that structure, with the result unchanged.
//
// 1. The culled scan (ball_query.hip) runs in index order as usual but stops a
//    wave after `budget` scanned blocks of 64 references. A query that has K
//    hits by then, or whose wave finished, is complete. Any other query
//    records its hit count c and the first reference index t its wave did not
//    examine: its first c hits are final, and the rest of its first K are the
//    hits with index >= t, in index order.
// 2. Only when some query was left (a device flag: no host round trip) the
//    grid of the references is built (launch_grid_build: Morton-sorted copies
//    and boxes of 16 and 1024 sorted references) and this pass runs: one wave
//    per left query, in the grid's order of the queries (neighbouring waves
//    read neighbouring references). The lanes test 64 boxes at a time, first
//    of the superblocks, then of the blocks of a surviving superblock, and then
//    test the references of up to four surviving blocks at a time, one per
//    lane. A box whose lower bound of s32 (in the float32 order of s32, so
//    never above the s32 of a point in it) is >= R2 holds no hit, nor does one
//    whose original indices all lie outside [t, the current (K - c)-th
//    smallest index): the list's bound then prunes by index too, so even a
//    radius that covers the whole cloud visits few blocks once the list is
//    full. The wave
//    keeps the K - c smallest indices of the hits with index >= t in its list
//    (wave_list.h) as keys (index << 32) | bits(s); a hit is a candidate when
//    its index is below that of the (K - c)-th smallest so far (indices are
//    unique, so the strict test is exact). Lane n < K - c then writes the n-th
//    key into slot c + n of the query's row; slots left hold the scan's
//    padding.
//
// Dense clouds in index order finish in step 1 (few blocks survive the
// culling, or K hits come early); queries in sparse regions of clouds in
// random order are the ones left, and they find their few hits through the
// grid instead of scanning every reference.
//
// Ragged batches (the clouds' records, grid.h GridCloud) take the plain
// index-order scan in its budgeted mode as step 1 (ball_query.hip: no boxes;
// it stops a query at K hits, at a budget of references, or early when the
// query's hit rate says K would take longer), then step 2 as above.
#include "common.h"
#include "grid.h"
#include "wave_list.h"

namespace pointops {

constexpr uint32_t kBqgDone = 0xFFFFFFFFu;  // state: the query is complete
constexpr int kBqgWaves = 4;                // waves (queries) per workgroup

// A box may hold a hit the pass still needs: its lower bound of s32 is
// below R2 and its index range meets [from, bound).
__device__ __forceinline__ bool bqg_box_open(const float* __restrict__ o, float qx, float qy,
                                             float qz, float r2, uint32_t from, uint32_t bound) {
    return box_bound(o, qx, qy, qz) < r2 && (uint32_t)__float_as_int(o[6]) < bound &&
           __float_as_int(o[7]) >= (int)from;
}

__global__ __launch_bounds__(kBqgWaves* kWave) void ball_query_grid_kernel(
    const float4* __restrict__ sq, const float4* __restrict__ sr, int Q, int P, float r2, int K,
    const float* __restrict__ box, const float* __restrict__ sbox, int nblk, int nsb,
    const uint2* __restrict__ state, const uint32_t* __restrict__ flag,
    float* __restrict__ out_d2, int64_t* __restrict__ out_idx, const int64_t* __restrict__ clouds) {
    if (flag && *flag == 0) return;  // no query was left: nothing to do
    __shared__ uint64_t cbuf[kBqgWaves][kKwBuf];
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
    const int lane = lane_id();
    const int w = uniform((int)(threadIdx.x / kWave));
    const int qi = (int)blockIdx.x * kBqgWaves + w;
    if (qi >= Qb) return;  // whole waves (no barrier in this kernel)
    const float4 q = sq[(size_t)b * Q + qi];
    const int row = __float_as_int(q.w);  // the query's index in its cloud
    const uint2 st = state[(size_t)b * Q + row];
    if (st.y == kBqgDone) return;
    const int have = (int)st.x;     // hits the scan found, < K
    const int need = K - have;      // 1 .. K <= 32
    const uint32_t from = st.y;     // first index the scan did not examine
    const float4* rb = sr + (size_t)b * P;
    const float* bx = box + (size_t)b * nblk * 8;
    const float* sbx = sbox + (size_t)b * nsb * 8;

    KwQuery L{kKwEmpty, ~0u, 0, cbuf[w]};
    for (int sb0 = 0; sb0 < nsbb; sb0 += kWave) {
        const int my_sb = sb0 + lane;
        uint64_t ms = ballot(my_sb < nsbb && bqg_box_open(sbx + (size_t)min(my_sb, nsbb - 1) * 8,
                                                          q.x, q.y, q.z, r2, from, L.bound));
        while (ms) {
            const int s = sb0 + __builtin_ctzll(ms);
            ms &= ms - 1;
            const int my_blk = s * kWave + lane;
            uint64_t mb = ballot(my_blk < nbb && bqg_box_open(bx + (size_t)min(my_blk, nbb - 1) * 8,
                                                              q.x, q.y, q.z, r2, from, L.bound));
            while (mb) {
                // the next four surviving blocks (or fewer), 16 lanes each
                int blk[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    blk[r] = mb ? s * kWave + __builtin_ctzll(mb) : -1;
                    mb &= mb - 1;  // no-op once empty
                }
                const int g = lane >> 4;
                const int mine = g == 0 ? blk[0] : g == 1 ? blk[1] : g == 2 ? blk[2] : blk[3];
                const int j = mine * kGridBlk + (lane & (kGridBlk - 1));
                bool hit = false;
                uint32_t idx = 0u, us = 0u;
                if (mine >= 0 && j < Pb) {
                    const float4 p = rb[j];
                    const float sv = s32(q.x, q.y, q.z, p.x, p.y, p.z);
                    idx = (uint32_t)__float_as_int(p.w);
                    us = f2u(sv);
                    hit = sv < r2 && idx >= from && idx < L.bound;
                }
                kw_offer(L, hit, idx, (int)us, lane, need);
            }
        }
    }
    if (L.cnt > 0) kw_merge(L, lane, need);

    // lane n < need: the n-th smallest index found, or the padding (-1, +0)
    // where there is none (the scans wrote it there already)
    if (lane < need) {
        const size_t o = (size_t)(orow0 + row) * (size_t)K + have + lane;
        const bool empty = L.list == kKwEmpty;
        out_idx[o] = empty ? (int64_t)-1 : ibase + (int64_t)(uint32_t)(L.list >> 32);
        out_d2[o] = empty ? 0.0f : u2f((uint32_t)L.list);
    }
}

// Workspace: the culled scan's boxes, the per-query state, the flag, the grid.
struct BqGridLayout {
    size_t box, state, flag, grid, total;
};

size_t ball_query_box_bytes(int64_t B, int64_t P);

static size_t bqg_al(size_t n) { return (n + 255) / 256 * 256; }

static BqGridLayout bq_grid_layout(int64_t B, int64_t Q, int64_t P) {
    BqGridLayout l;
    size_t o = 0;
    l.box = o; o += bqg_al(ball_query_box_bytes(B, P));
    l.state = o; o += bqg_al((size_t)B * Q * sizeof(uint2));
    l.flag = o; o += 256;
    l.grid = o; o += bqg_al(grid_workspace_bytes(B, Q, P, 7));  // room for any level
    l.total = o;
    return l;
}

size_t ball_query_grid_bytes(int64_t B, int64_t Q, int64_t P) {
    return bq_grid_layout(B, Q, P).total;
}

hipError_t launch_ball_query_culled(const float* query, const float* ref, int64_t B, int64_t Q,
                                    int64_t P, float r2, int64_t K, float* out_d2,
                                    int64_t* out_idx, int qw, float* box, int budget,
                                    uint2* state, uint32_t* flag, hipStream_t stream);

// The culled scan with `budget` blocks per wave, then (gated on the device by
// the flag) the build of a grid of 2^level cells per axis and the grid pass.
// Requires 1 <= K <= 32 and 2 <= level <= 7.
hipError_t launch_ball_query_grid(const float* query, const float* ref, int64_t B, int64_t Q,
                                  int64_t P, float r2, int64_t K, float* out_d2,
                                  int64_t* out_idx, int qw, int budget, int level,
                                  void* workspace, hipStream_t stream) {
    if (K < 1 || K > kKwBuf || B < 1 || Q < 1 || P < 1 || level < 2 || level > 7)
        return hipErrorInvalidValue;
    const BqGridLayout l = bq_grid_layout(B, Q, P);
    char* ws = (char*)workspace;
    uint2* state = (uint2*)(ws + l.state);
    uint32_t* flag = (uint32_t*)(ws + l.flag);
    hipError_t e = launch_ball_query_culled(query, ref, B, Q, P, r2, K, out_d2, out_idx, qw,
                                            (float*)(ws + l.box), budget, state, flag, stream);
    if (e != hipSuccess) return e;
    GridView v;
    e = launch_grid_build(query, ref, B, Q, P, level, ws + l.grid, flag, nullptr, stream,
                          &v);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((Q + kBqgWaves - 1) / kBqgWaves), (unsigned)B);
    hipLaunchKernelGGL(ball_query_grid_kernel, grid, dim3(kBqgWaves * kWave), 0, stream,
                       v.squery, v.sref, (int)Q, (int)P, r2, (int)K, v.box, v.sbox, v.nblk,
                       v.nsb, state, flag, out_d2, out_idx, nullptr);
    return hipGetLastError();
}

size_t ball_query_ragged_grid_bytes(int64_t B, int64_t Q, int64_t P, int level) {
    return grid_workspace_bytes(B, Q, P, level);
}

// The second step for a ragged batch described by `clouds` (device memory, B
// records; see GridCloud), P and Q being the largest counts, after the
// budgeted scan (ball_query.hip) wrote `state` (B x Q) and `flag`: gated on
// the flag, the grid build and the grid pass. The workspace holds
// ball_query_ragged_grid_bytes(B, Q, P, level). Requires 1 <= K <= 32.
hipError_t launch_ball_query_ragged_grid(const float* query, const float* ref, int64_t B,
                                         int64_t Q, int64_t P, float r2, int64_t K,
                                         float* out_d2, int64_t* out_idx, int level,
                                         const int64_t* clouds, uint32_t* flag, uint2* state,
                                         void* workspace, hipStream_t stream) {
    if (K < 1 || K > kKwBuf || B < 1 || Q < 1 || P < 1 || level < 2 || level > 7)
        return hipErrorInvalidValue;
    GridView v;
    hipError_t e = launch_grid_build(query, ref, B, Q, P, level, workspace, flag, clouds, stream,
                                     &v);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((Q + kBqgWaves - 1) / kBqgWaves), (unsigned)B);
    hipLaunchKernelGGL(ball_query_grid_kernel, grid, dim3(kBqgWaves * kWave), 0, stream,
                       v.squery, v.sref, (int)Q, (int)P, r2, (int)K, v.box, v.sbox, v.nblk,
                       v.nsb, state, flag, out_d2, out_idx, clouds);
    return hipGetLastError();
}

}  // namespace pointops
