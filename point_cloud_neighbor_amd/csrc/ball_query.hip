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
//
// Budgeted scan (the ragged batches' first step, see BqBudget): a query also
// stops after `budget` references, or after the first `probe` when its hit
// count is too low to reach K within the budget at that rate. Its first hits
// are then in place (they are the first ones: every later index is larger),
// the rest of its row is padding, and it records (hits, references examined),
// or done. A query left adds its estimate of the references it still needs
// (from its hit rate so far); the sum decides (ball_query_decide_kernel)
// whether the grid pass of ball_query_grid.hip takes the queries left, or
// the resume mode of this kernel, which continues each from its first
// unexamined index with its count so far: the same first K either way.
#include <type_traits>

#include "common.h"
#include "segments.h"

namespace pointops {

constexpr uint32_t kBqDone = 0xFFFFFFFFu;  // state: the query is complete
constexpr int kXcds = 8;  // accelerator complex dies of the device, one L2 each

// MODE: kBqPlain, kBqBudgeted or kBqResume (see BqBudget); a template
// parameter, so the plain scan's loop carries none of the others' tests.
constexpr int kBqPlain = 0, kBqBudgeted = 1, kBqResume = 2;

template <int QW, int MODE>
__global__ __launch_bounds__(kWave) void ball_query_kernel(
    const float* __restrict__ query, const float* __restrict__ ref, int Q, int P, float r2,
    int K, float* __restrict__ out_d2, int64_t* __restrict__ out_idx,
    const int64_t* __restrict__ seg, int nseg, BqBudget bud) {
    // this wave's cloud: its first query row, reference row, sizes
    int64_t qrow0, rrow0, ibase, unit, cloud;
    if (seg) {
        const int b = seg_find(seg, nseg, blockIdx.x);
        const int64_t* rec = seg_record(seg, nseg, b);
        unit = blockIdx.x - seg[b];
        qrow0 = rec[kSrQOff];
        Q = (int)rec[kSrQCnt];
        rrow0 = rec[kSrROff];
        P = (int)rec[kSrRCnt];
        ibase = rec[kSrIdxBase];
        cloud = rec[kSrCloud];
    } else {
        unit = blockIdx.x;
        qrow0 = (int64_t)blockIdx.y * Q;
        rrow0 = (int64_t)blockIdx.y * P;
        ibase = 0;
        cloud = blockIdx.y;
    }
    constexpr bool BUD = MODE == kBqBudgeted;
    if (MODE == kBqResume && *bud.gate == 0) return;  // the grid pass takes the queries left
    const int n = BUD ? min(P, bud.budget) : P;  // references this wave may scan
    const int row0 = (int)unit * QW;
    const int lane = threadIdx.x;
    const float* qb = query + qrow0 * 3;
    const float* xb = ref + rrow0 * 3;
    const size_t out0 = (size_t)(qrow0 + row0) * (size_t)K;

    float qx[QW], qy[QW], qz[QW];
    int cnt[QW];
    bool stopped[QW];  // left at the probe (budgeted scan)
    int from[QW];      // first index a resumed query takes
    int start = 0;     // first block of the scan
#pragma unroll
    for (int i = 0; i < QW; ++i) {
        const int row = row0 + i < Q ? row0 + i : Q - 1;
        qx[i] = qb[(size_t)3 * row + 0];
        qy[i] = qb[(size_t)3 * row + 1];
        qz[i] = qb[(size_t)3 * row + 2];
        cnt[i] = row0 + i < Q ? 0 : K;  // rows past the end take no hits
        stopped[i] = false;
        from[i] = 0;
    }
    if constexpr (MODE == kBqResume) {
        // done queries take no hits; the others keep their count and go on
        // from the first index they did not examine
        start = n;
#pragma unroll
        for (int i = 0; i < QW; ++i) {
            if (row0 + i < Q) {
                const uint2 st = bud.state[(size_t)cloud * bud.stride + row0 + i];
                cnt[i] = st.y == kBqDone ? K : (int)st.x;
                from[i] = st.y == kBqDone ? n : (int)st.y;
                start = min(start, from[i]);
            }
        }
        start &= ~(kWave - 1);
    }
    // the queries still taking hits, bit i for query i (wave-uniform): short
    // of K and not stopped at the probe
    uint32_t open = 0;
#pragma unroll
    for (int i = 0; i < QW; ++i) open |= (cnt[i] < K ? 1u : 0u) << i;

    // Software-pipelined reference loads: block n+1 is in flight while block n
    // is compared. Lanes past the last reference hold NaN coordinates, whose
    // distance compares false against R2, so no separate range test is needed.
    const float nan = __builtin_nanf("");
    float nx = nan, ny = nan, nz = nan;
    if (start + lane < n) {
        nx = xb[(size_t)3 * (start + lane) + 0];
        ny = xb[(size_t)3 * (start + lane) + 1];
        nz = xb[(size_t)3 * (start + lane) + 2];
    }
    // One block of 64 references for every live query. FULL: the next block
    // is complete (base + 2 * kWave <= n), so its load needs no range test.
    auto block = [&](int base, auto full_) -> bool {
        constexpr bool FULL = decltype(full_)::value;
        const int j = base + lane;
        const float x = nx, y = ny, z = nz;
        const int jn = j + kWave;
        if constexpr (FULL) {
            nx = xb[(size_t)3 * jn + 0];
            ny = xb[(size_t)3 * jn + 1];
            nz = xb[(size_t)3 * jn + 2];
        } else {
            nx = ny = nz = nan;
            if (jn < n) {
                nx = xb[(size_t)3 * jn + 0];
                ny = xb[(size_t)3 * jn + 1];
                nz = xb[(size_t)3 * jn + 2];
            }
        }
        const bool at_probe = BUD && base + kWave == bud.probe;
#pragma unroll
        for (int i = 0; i < QW; ++i) {
            if ((open >> i) & 1u) {
                const float s = s32(qx[i], qy[i], qz[i], x, y, z);
                const bool h = s < r2 && (MODE != kBqResume || j >= from[i]);
                const uint64_t m = ballot(h);
                if (m) {
                    const int slot = cnt[i] + (int)lanes_below(m);
                    if (h && slot < K) {
                        out_idx[out0 + (size_t)i * K + slot] = ibase + j;
                        out_d2[out0 + (size_t)i * K + slot] = s;
                    }
                    cnt[i] += __popcll(m);
                    if (cnt[i] >= K) open &= ~(1u << i);
                }
                if constexpr (BUD) {
                    // at this rate K hits would take more than the budget
                    if (at_probe && cnt[i] < K &&
                        (int64_t)cnt[i] * bud.budget < (int64_t)K * bud.probe) {
                        stopped[i] = true;
                        open &= ~(1u << i);
                    }
                }
            }
        }
        return open != 0;
    };
    int base = start;
    bool live = true;
    for (; live && base + 2 * kWave <= n; base += kWave) live = block(base, std::true_type{});
    for (; live && base < n; base += kWave) live = block(base, std::false_type{});

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
    if (BUD && lane == 0) {
        // A query that neither has K hits nor stopped scanned all n
        // references. A query left estimates the references it still needs
        // from its hit rate so far (the rest of its cloud without a hit).
        unsigned long long est = 0;
#pragma unroll
        for (int i = 0; i < QW; ++i) {
            if (row0 + i < Q) {
                const int seen = stopped[i] ? bud.probe : n;
                const bool done = cnt[i] >= K || seen >= P;
                bud.state[(size_t)cloud * bud.stride + row0 + i] =
                    done ? make_uint2(0u, kBqDone) : make_uint2((uint32_t)cnt[i], (uint32_t)seen);
                if (!done) {
                    const float rest = (float)(P - seen);
                    const float need = cnt[i] > 0
                                           ? (float)(K - cnt[i]) * (float)seen / (float)cnt[i] + 1.0f
                                           : rest;
                    est += (unsigned long long)fminf(rest, need);
                }
            }
        }
        // spread over kBqEstimates counters: one word would serialise the
        // waves' atomics at its L2 channel
        if (est) atomicAdd(&bud.estimate[blockIdx.x % kBqEstimates], est);
    }
}

// One wave: the sum of the estimates decides between the grid pass (gate[0])
// and resuming the scan (gate[1]) for the queries left; neither when none is.
__global__ __launch_bounds__(kWave) void ball_query_decide_kernel(
    const unsigned long long* __restrict__ estimate, unsigned long long grid_pairs,
    uint32_t* __restrict__ gate) {
    static_assert(kBqEstimates % kWave == 0, "counters split evenly over the lanes");
    unsigned long long v = 0;
#pragma unroll
    for (int i = 0; i < kBqEstimates / kWave; ++i) v += estimate[i * kWave + threadIdx.x];
#pragma unroll
    for (int o = kWave / 2; o >= 1; o /= 2) v += __shfl_xor(v, o);
    if (threadIdx.x == 0) {
        gate[0] = v >= grid_pairs ? 1u : 0u;
        gate[1] = v > 0 && v < grid_pairs ? 1u : 0u;
    }
}

hipError_t launch_ball_query_decide(const unsigned long long* estimate,
                                    unsigned long long grid_pairs, uint32_t* gate,
                                    hipStream_t stream) {
    hipLaunchKernelGGL(ball_query_decide_kernel, dim3(1), dim3(kWave), 0, stream, estimate,
                       grid_pairs, gate);
    return hipGetLastError();
}

// Launch helper used by the C ABI: grid (ceil(Q / QW), B), one wave per group;
// ragged (seg != nullptr): grid (waves, 1) with waves = the table's
// tile_ptr[nseg], Q and P unused.
// mode: kBqPlain, kBqBudgeted or kBqResume (the last two with `bud`).
hipError_t launch_ball_query(const float* query, const float* ref, int64_t B, int64_t Q,
                             int64_t P, float r2, int64_t K, float* out_d2, int64_t* out_idx,
                             int qw, const int64_t* seg, int nseg, int64_t waves,
                             hipStream_t stream, int mode, BqBudget bud) {
    dim3 block(kWave);
    switch (qw) {
#define POINTOPS_BQ_CASE(W)                                                                  \
    case W: {                                                                                \
        dim3 grid = seg ? dim3((unsigned)waves, 1)                                           \
                        : dim3((unsigned)((Q + W - 1) / W), (unsigned)B);                    \
        if (mode == kBqBudgeted)                                                             \
            hipLaunchKernelGGL((ball_query_kernel<W, kBqBudgeted>), grid, block, 0, stream,   \
                               query, ref, (int)Q, (int)P, r2, (int)K, out_d2, out_idx, seg, \
                               nseg, bud);                                                   \
        else if (mode == kBqResume)                                                          \
            hipLaunchKernelGGL((ball_query_kernel<W, kBqResume>), grid, block, 0, stream,     \
                               query, ref, (int)Q, (int)P, r2, (int)K, out_d2, out_idx, seg, \
                               nseg, bud);                                                   \
        else                                                                                 \
            hipLaunchKernelGGL((ball_query_kernel<W, kBqPlain>), grid, block, 0, stream,      \
                               query, ref, (int)Q, (int)P, r2, (int)K, out_d2, out_idx, seg, \
                               nseg, bud);                                                   \
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

// ---------------------------------------------------------------- culled scan
//
// For spatially ordered references (consecutive indices close in space) most
// 64-reference blocks lie far from a query. A block's bounding box gives a
// lower bound of s32 over its points that never exceeds the true value:
// per axis the gap g = max(lo - q, q - hi, 0) is computed with the same
// float32 subtraction as the distance, and rounding is monotone, so
// |fl(q - x)| >= fl(gap) for every x of the block; squaring and the two
// additions, in the order of s32, are monotone too. A block whose bound is
// >= R2 therefore holds no reference with s32 < R2 and is skipped; the
// remaining blocks are scanned in increasing order exactly as before, so the
// first K hits, their order and their bits do not change.
//
// The test is made first once per block for the wave's whole group of
// queries: the gap between the block's box and the box of the group's queries
// bounds the gap of every (query, point) pair the same way (lo_b - hi_q <=
// x - q), so a block is skipped for the group when even that bound reaches
// R2. Only in the runs of 64 blocks where some block survives does each query
// test the blocks on its own, and a block is then scanned for the queries
// whose own test it passed. One level up, the union box of every 64 blocks
// lets a wave find the runs worth loading with one load per lane, instead of
// loading every run's 64 boxes in turn.

constexpr int kBoxFloats = 8;  // min x, y, z, max x, y, z, 2 unused

__device__ __forceinline__ float wave_min_f32(float v) {
#pragma unroll
    for (int o = kWave / 2; o >= 1; o /= 2) v = fminf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int o = kWave / 2; o >= 1; o /= 2) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// One wave per block of 64 references: box[(b * nblk + k) * 8 + 0..5].
// `flag` (nullable): cleared here, set by the culled scan when a query is left
// for the grid pass.
__global__ __launch_bounds__(256) void ball_query_boxes_kernel(const float* __restrict__ ref,
                                                               int64_t B, int P, int nblk,
                                                               float* __restrict__ box,
                                                               uint32_t* __restrict__ flag) {
    if (flag && blockIdx.x == 0 && threadIdx.x == 0) *flag = 0u;
    const int64_t w = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (w >= B * nblk) return;  // whole waves leave together
    const int64_t b = w / nblk;
    const int k = (int)(w - b * nblk);
    const int j = k * kWave + lane;
    const float inf = __builtin_inff();
    float x = inf, y = inf, z = inf, X = -inf, Y = -inf, Z = -inf;
    if (j < P) {
        const float* p = ref + ((size_t)b * P + j) * 3;
        x = X = p[0];
        y = Y = p[1];
        z = Z = p[2];
    }
    x = wave_min_f32(x); y = wave_min_f32(y); z = wave_min_f32(z);
    X = wave_max_f32(X); Y = wave_max_f32(Y); Z = wave_max_f32(Z);
    if (lane == 0) {
        float* o = box + (size_t)w * kBoxFloats;
        o[0] = x; o[1] = y; o[2] = z; o[3] = X; o[4] = Y; o[5] = Z;
    }
}

// Budget (state != nullptr): a wave scans at most `budget` blocks. Where it
// stops early, each of its queries still short of K records (hits so far,
// first reference index not examined) in state[b * Q + row], and the wave
// sets *flag; every other query records (count, kBqDone). The grid pass then
// looks only at references from that index on, so the hits it adds come
// after these in index order.

// One wave per 64 blocks: their union box, sbox[(b * nsb + s) * 8 + 0..5].
__global__ __launch_bounds__(256) void ball_query_superboxes_kernel(const float* __restrict__ box,
                                                                    int64_t B, int nblk, int nsb,
                                                                    float* __restrict__ sbox) {
    const int64_t w = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (w >= B * nsb) return;  // whole waves leave together
    const int64_t b = w / nsb;
    const int k = (int)(w - b * nsb) * kWave + lane;
    const float inf = __builtin_inff();
    float x = inf, y = inf, z = inf, X = -inf, Y = -inf, Z = -inf;
    if (k < nblk) {
        const float* o = box + ((size_t)b * nblk + k) * kBoxFloats;
        x = o[0]; y = o[1]; z = o[2]; X = o[3]; Y = o[4]; Z = o[5];
    }
    x = wave_min_f32(x); y = wave_min_f32(y); z = wave_min_f32(z);
    X = wave_max_f32(X); Y = wave_max_f32(Y); Z = wave_max_f32(Z);
    if (lane == 0) {
        float* o = sbox + (size_t)w * kBoxFloats;
        o[0] = x; o[1] = y; o[2] = z; o[3] = X; o[4] = Y; o[5] = Z;
    }
}

template <int QW, bool STAGE>
__global__ __launch_bounds__(kWave) void ball_query_cull_kernel(
    const float* __restrict__ query, const float* __restrict__ ref, int Q, int P, float r2,
    int K, float* __restrict__ out_d2, int64_t* __restrict__ out_idx,
    const float* __restrict__ box, int nblk, const float* __restrict__ sbox, int nsb, int budget,
    uint2* __restrict__ state, uint32_t* __restrict__ flag) {
    const int b = blockIdx.y;
    // Workgroups go round-robin to the 8 XCDs, each with its own L2: XCD x
    // takes the x-th contiguous run of query groups, so on a spatially
    // sorted cloud its L2 holds only its region's references.
    const int groups = (Q + QW - 1) / QW;
    const int per_xcd = (groups + kXcds - 1) / kXcds;
    const int group = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    if (group >= groups) return;
    const int row0 = group * QW;
    const int lane = threadIdx.x;
    const float* qb = query + (size_t)b * Q * 3;
    const float* xb = ref + (size_t)b * P * 3;
    const float* bb = box + (size_t)b * nblk * kBoxFloats;
    const float* sbb = sbox + (size_t)b * nsb * kBoxFloats;
    const size_t out0 = ((size_t)b * Q + row0) * (size_t)K;
    // STAGE (K <= 64): hits go to the wave's rows in LDS, and each row is
    // written to HBM once at the end, in whole lines with its padding,
    // instead of a few slots per block (a partial line is read before it is
    // written).
    __shared__ int32_t stage_j[STAGE ? QW : 1][kWave];
    __shared__ float stage_s[STAGE ? QW : 1][kWave];

    float qx[QW], qy[QW], qz[QW];
    int cnt[QW];
#pragma unroll
    for (int i = 0; i < QW; ++i) {
        const int row = row0 + i < Q ? row0 + i : Q - 1;
        qx[i] = qb[(size_t)3 * row + 0];
        qy[i] = qb[(size_t)3 * row + 1];
        qz[i] = qb[(size_t)3 * row + 2];
        cnt[i] = row0 + i < Q ? 0 : K;
    }
    // the queries still short of K hits, bit i for query i (wave-uniform)
    uint32_t open = 0;
#pragma unroll
    for (int i = 0; i < QW; ++i) open |= (cnt[i] < K ? 1u : 0u) << i;
    const float nan = __builtin_nanf("");
    const float inf = __builtin_inff();
    // the box of the group's queries (rows past Q repeat row Q - 1)
    float gqx = qx[0], gqy = qy[0], gqz = qz[0], gQx = qx[0], gQy = qy[0], gQz = qz[0];
#pragma unroll
    for (int i = 1; i < QW; ++i) {
        gqx = fminf(gqx, qx[i]); gqy = fminf(gqy, qy[i]); gqz = fminf(gqz, qz[i]);
        gQx = fmaxf(gQx, qx[i]); gQy = fmaxf(gQy, qy[i]); gQz = fmaxf(gQz, qz[i]);
    }

    int scanned = 0;    // blocks this wave has scanned
    int stop_blk = -1;  // first block not examined when the budget ran out
    bool finished = false;
    // Runs of 64 blocks in increasing order, only those whose union box the
    // group's box can reach (the same bound, one level up)
    for (int s0 = 0; s0 < nsb && !finished; s0 += kWave) {
      uint64_t ms;
      {
        const int sl = s0 + lane;
        float lx = inf, ly = inf, lz = inf, hx = -inf, hy = -inf, hz = -inf;
        if (sl < nsb) {
            const float* o = sbb + (size_t)sl * kBoxFloats;
            lx = o[0]; ly = o[1]; lz = o[2]; hx = o[3]; hy = o[4]; hz = o[5];
        }
        const float gx = fmaxf(fmaxf(lx - gQx, gqx - hx), 0.0f);
        const float gy = fmaxf(fmaxf(ly - gQy, gqy - hy), 0.0f);
        const float gz = fmaxf(fmaxf(lz - gQz, gqz - hz), 0.0f);
        ms = ballot((gx * gx + gy * gy) + gz * gz < r2);
      }
      while (ms) {
        const int c0 = (s0 + __builtin_ctzll(ms)) * kWave;
        ms &= ms - 1;
        // lane l: block c0 + l; blocks past the end have an empty box (bound +inf)
        const int k = c0 + lane;
        float lx = inf, ly = inf, lz = inf, hx = -inf, hy = -inf, hz = -inf;
        if (k < nblk) {
            const float* o = bb + (size_t)k * kBoxFloats;
            lx = o[0]; ly = o[1]; lz = o[2]; hx = o[3]; hy = o[4]; hz = o[5];
        }
        const float gx = fmaxf(fmaxf(lx - gQx, gqx - hx), 0.0f);
        const float gy = fmaxf(fmaxf(ly - gQy, gqy - hy), 0.0f);
        const float gz = fmaxf(fmaxf(lz - gQz, gqz - hz), 0.0f);
        const float lb = (gx * gx + gy * gy) + gz * gz;
        if (ballot(lb < r2) == 0) continue;
        // lane l: bit i set when query i can reach block c0 + l (the same
        // bound per query); a block is scanned for the queries of its mask
        // that are still open
        uint32_t qm = 0;
#pragma unroll
        for (int i = 0; i < QW; ++i) {
            const float ex = fmaxf(fmaxf(lx - qx[i], qx[i] - hx), 0.0f);
            const float ey = fmaxf(fmaxf(ly - qy[i], qy[i] - hy), 0.0f);
            const float ez = fmaxf(fmaxf(lz - qz[i], qz[i] - hz), 0.0f);
            qm |= ((ex * ex + ey * ey) + ez * ez < r2 ? 1u : 0u) << i;
        }
        const uint64_t any = ballot((qm & open) != 0);
        if (any == 0) continue;
        // Candidate blocks in increasing order. The next block's load is
        // issued before the current one is tested, but the compiler waits
        // for it with the current one (it is skippable, and copied into the
        // current registers); a form with two register sets in turn and
        // unconditional loads, whose waits cover only the current block,
        // measured no faster (0.087 against 0.084 ms on the sorted 100k
        // workload): the scan is bound by issue, not by these loads.
        int cur = __builtin_ctzll(any);
        float nx = nan, ny = nan, nz = nan;
        {
            const int j = (c0 + cur) * kWave + lane;
            if (j < P) { nx = xb[(size_t)3 * j + 0]; ny = xb[(size_t)3 * j + 1]; nz = xb[(size_t)3 * j + 2]; }
        }
        uint64_t rest = any & (any - 1);
        bool live = true;
        while (true) {
            const float x = nx, y = ny, z = nz;
            const int blk = cur;
            if (scanned == budget) {  // budget spent: block c0 + blk is left to the grid pass
                stop_blk = c0 + blk;
                break;
            }
            ++scanned;
            if (rest) {
                cur = __builtin_ctzll(rest);
                rest &= rest - 1;
                const int j = (c0 + cur) * kWave + lane;
                nx = ny = nz = nan;
                if (j < P) { nx = xb[(size_t)3 * j + 0]; ny = xb[(size_t)3 * j + 1]; nz = xb[(size_t)3 * j + 2]; }
            } else {
                cur = -1;
            }
            const int j = (c0 + blk) * kWave + lane;
            const uint32_t act = (uint32_t)__builtin_amdgcn_readlane((int)qm, blk) & open;
#pragma unroll
            for (int i = 0; i < QW; ++i) {
                if ((act >> i) & 1u) {
                    const float s = s32(qx[i], qy[i], qz[i], x, y, z);
                    const bool h = s < r2;
                    const uint64_t m = ballot(h);
                    if (m) {
                        const int slot = cnt[i] + (int)lanes_below(m);
                        if (h && slot < K) {
                            if constexpr (STAGE) {
                                stage_j[i][slot] = j;
                                stage_s[i][slot] = s;
                            } else {
                                out_idx[out0 + (size_t)i * K + slot] = j;
                                out_d2[out0 + (size_t)i * K + slot] = s;
                            }
                        }
                        cnt[i] += __popcll(m);
                        if (cnt[i] >= K) open &= ~(1u << i);
                    }
                }
            }
            live = open != 0;
            if (!live || cur < 0) break;
        }
        if (!live || stop_blk >= 0) {
            finished = true;
            break;
        }
      }
    }

    bool left = false;
    if constexpr (STAGE) {
        // the rows' LDS stores (any lane) before the reads of every lane: one
        // wave, whose LDS operations complete in order
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int i = 0; i < QW; ++i) {
        if (row0 + i < Q) {
            if constexpr (STAGE) {
                if (lane < K) {  // lane = slot: hits, then (-1, +0.0) padding
                    const bool hit = lane < cnt[i];
                    out_idx[out0 + (size_t)i * K + lane] = hit ? (int64_t)stage_j[i][lane] : -1;
                    out_d2[out0 + (size_t)i * K + lane] = hit ? stage_s[i][lane] : 0.0f;
                }
            } else {
                for (int slot = cnt[i] + lane; slot < K; slot += kWave) {
                    out_idx[out0 + (size_t)i * K + slot] = -1;
                    out_d2[out0 + (size_t)i * K + slot] = 0.0f;
                }
            }
            if (state && lane == 0) {
                const bool open = stop_blk >= 0 && cnt[i] < K;
                state[(size_t)b * Q + row0 + i] =
                    make_uint2((uint32_t)min(cnt[i], K), open ? (uint32_t)stop_blk * kWave : kBqDone);
                left |= open;
            }
        }
    }
    // lane 0 only; only the waves that still see the flag clear raise it (one
    // atomic per wave on one word would serialise at its L2 channel)
    if (left && __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u)
        atomicOr(flag, 1u);
}

// Boxes of the 64-reference blocks, then of every 64 blocks.
size_t ball_query_box_bytes(int64_t B, int64_t P) {
    const int64_t nblk = (P + kWave - 1) / kWave, nsb = (nblk + kWave - 1) / kWave;
    return (size_t)B * (size_t)(nblk + nsb) * kBoxFloats * sizeof(float);
}

// Boxes of every 64-reference block into `box`, then the culled scan: grid
// (ceil(Q / QW), B), one wave per group of QW queries.
// With `state` non-null, the scan keeps to `budget` blocks per wave and leaves
// the rest to the grid pass (see ball_query_cull_kernel).
hipError_t launch_ball_query_culled(const float* query, const float* ref, int64_t B, int64_t Q,
                                    int64_t P, float r2, int64_t K, float* out_d2,
                                    int64_t* out_idx, int qw, float* box, int budget,
                                    uint2* state, uint32_t* flag, hipStream_t stream) {
    const int nblk = (int)((P + kWave - 1) / kWave), nsb = (nblk + kWave - 1) / kWave;
    float* sbox = box + (size_t)B * nblk * kBoxFloats;
    if (!state) budget = -1;  // never reached
    if (B * nblk > 0) {
        const int64_t waves = B * nblk;
        hipLaunchKernelGGL(ball_query_boxes_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256),
                           0, stream, ref, B, (int)P, nblk, box, flag);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(ball_query_superboxes_kernel,
                           dim3((unsigned)((B * nsb + 3) / 4)), dim3(256), 0, stream, box, B,
                           nblk, nsb, sbox);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 block(kWave);
    switch (qw) {
#define POINTOPS_BQC_CASE(W)                                                                  \
    case W: {                                                                                 \
        dim3 grid((unsigned)(((Q + W - 1) / W + kXcds - 1) / kXcds * kXcds), (unsigned)B);  \
        if (K <= kWave)                                                                       \
            hipLaunchKernelGGL((ball_query_cull_kernel<W, true>), grid, block, 0, stream,     \
                               query, ref, (int)Q, (int)P, r2, (int)K, out_d2, out_idx, box,  \
                               nblk, sbox, nsb, budget, state, flag);                         \
        else                                                                                  \
            hipLaunchKernelGGL((ball_query_cull_kernel<W, false>), grid, block, 0, stream,    \
                               query, ref, (int)Q, (int)P, r2, (int)K, out_d2, out_idx, box,  \
                               nblk, sbox, nsb, budget, state, flag);                         \
        break;                                                                                \
    }
        POINTOPS_BQC_CASE(1)
        POINTOPS_BQC_CASE(2)
        POINTOPS_BQC_CASE(4)
        POINTOPS_BQC_CASE(8)
        POINTOPS_BQC_CASE(16)
#undef POINTOPS_BQC_CASE
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pointops
