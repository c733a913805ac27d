// Ragged batches: each cloud is a segment of a flat (rows, 3) float32 buffer.
//
// The project page's flat API (section "Flat torch_cluster subset") keeps the
// clouds of a batch back to back in one point array, delimited by sorted batch
// vectors or ptr offsets, with separate offsets for queries and references;
// its PyTorch3D-style adapter (section "PyTorch3D-style Ball Query") takes
// padded clouds with per-cloud lengths. Both are segments: cloud b is rows
// [off_b, off_b + cnt_b) of its buffer.
//
// The host describes the clouds of a launch in a table that it writes into
// the caller's workspace before the launch: tile_ptr, B + 1 words (padded to a
// multiple of 8), then one 8-word record per cloud. The launch's workgroups
// (or, for Ball Query, waves) are numbered cloud after cloud; unit w belongs
// to the cloud b with tile_ptr[b] <= w < tile_ptr[b + 1].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pointops {

constexpr int kSegRecWords = 8;

// Record of a kNN / Ball Query cloud (kSrCloud: its index in the caller's
// arrays, since the table orders the clouds by size).
enum SearchRec { kSrQOff = 0, kSrQCnt, kSrROff, kSrRCnt, kSrIdxBase, kSrCloud };
// Record of an FPS cloud: points, outputs, local start index, first exchange
// word, candidates published per workgroup.
enum FpsRec { kFrXOff = 0, kFrXCnt, kFrOOff, kFrOCnt, kFrIdxBase, kFrStart, kFrWOff, kFrRG };

// The budgeted and resume modes of the Ball Query scan (ball_query.hip).
// Budgeted: a query also stops after `budget` references, or after `probe`
// when its hits come too slowly, records its state at
// state[cloud * stride + row], and adds its estimate of the references it
// still needs to one of kBqEstimates 64-bit counters at `estimate`. Resume
// (only while *gate != 0): the queries left continue from their state.
constexpr int kBqEstimates = 256;
struct BqBudget {
    uint2* state;
    unsigned long long* estimate;
    const uint32_t* gate;
    int probe, budget, stride;
};

__host__ __device__ inline int64_t seg_ptr_words(int64_t B) { return (B + 1 + 7) / 8 * 8; }
__host__ __device__ inline int64_t seg_table_words(int64_t B) { return seg_ptr_words(B) + B * kSegRecWords; }

// The cloud of unit `u`, for 0 <= u < tp[B]: the largest b with tp[b] <= u
// (clouds without units have tp[b] == tp[b + 1] and are never returned).
__device__ __forceinline__ int seg_find(const int64_t* __restrict__ tp, int B, int64_t u) {
    int lo = 0, hi = B;  // tp[lo] <= u < tp[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tp[mid] <= u) lo = mid;
        else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ const int64_t* seg_record(const int64_t* __restrict__ table, int B,
                                                     int b) {
    return table + seg_ptr_words(B) + (int64_t)b * kSegRecWords;
}

// Writes n host words to device memory on `stream` through kernel arguments
// (no host-to-device copy, so the host array may be reused at once and the
// call can be captured into a graph).
hipError_t upload_words(const int64_t* host, int64_t n, int64_t* dev, hipStream_t stream);

}  // namespace pointops
