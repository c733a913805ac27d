// Internal declarations shared by the C ABI sources: error reporting, the
// device check, environment knobs and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <array>
#include <vector>

#include "segments.h"

namespace pointops {

// mode: 0 plain, 1 budgeted, 2 resume (ball_query.hip)
hipError_t launch_ball_query(const float*, const float*, int64_t, int64_t, int64_t, float,
                             int64_t, float*, int64_t*, int, const int64_t*, int, int64_t,
                             hipStream_t, int = 0,
                             BqBudget = BqBudget{nullptr, nullptr, nullptr, 0, 0, 0});
hipError_t launch_ball_query_decide(const unsigned long long*, unsigned long long, uint32_t*,
                                    hipStream_t);
hipError_t launch_zero_f32(float*, size_t, hipStream_t);  // a fill kernel (ball_query_backward.hip)
hipError_t launch_ball_query_culled(const float*, const float*, int64_t, int64_t, int64_t,
                                    float, int64_t, float*, int64_t*, int, float*, int, uint2*,
                                    uint32_t*, hipStream_t);
size_t ball_query_box_bytes(int64_t B, int64_t P);
hipError_t launch_ball_query_grid(const float*, const float*, int64_t, int64_t, int64_t, float,
                                  int64_t, float*, int64_t*, int, int, int, void*, hipStream_t);
int knn_grid_level(int64_t P);
size_t ball_query_grid_bytes(int64_t B, int64_t Q, int64_t P);
size_t ball_query_ragged_grid_bytes(int64_t B, int64_t Q, int64_t P, int level);
hipError_t launch_ball_query_ragged_grid(const float*, const float*, int64_t, int64_t, int64_t,
                                         float, int64_t, float*, int64_t*, int, const int64_t*,
                                         uint32_t*, uint2*, void*, hipStream_t);
hipError_t launch_knn_grid(const float*, const float*, int64_t, int64_t, int64_t, int64_t, float*,
                           int64_t*, int, int, void*, int, const int64_t*, hipStream_t);
size_t knn_grid_workspace_bytes(int64_t B, int64_t Q, int64_t P);
hipError_t launch_fps(const float*, int64_t, int64_t, int64_t, int64_t, int64_t*, float*, void*,
                      int, int, int, uint32_t, hipStream_t, const int64_t*, int, int64_t);
hipError_t launch_fps_clear(void*, size_t, hipStream_t);
size_t fps_workspace_bytes(int64_t B, int64_t G);
hipError_t launch_fps_batch(const float*, int64_t, int64_t, int64_t, int64_t, int64_t*, float*,
                            void*, int, int, int, int, int, bool, uint32_t, hipStream_t,
                            const int64_t*, int, int64_t, uint64_t*, size_t);
hipError_t fps_batch_capacity(int ppt, int block, int cpl, size_t lds, bool group, int cus,
                              int* out);
bool fps_batch_group_built(int ppt, int block);
constexpr int kFpsGroupMaxSlice = 8192;  // points per slice that the grouping sorts in LDS
size_t fps_batch_group_bytes(int64_t B, int64_t N);
size_t fps_batch_group_offset(int64_t B, int64_t G, int rg);
size_t fps_batch_workspace_bytes(int64_t B, int64_t G, int rg);
size_t fps_batch_lds_bytes(int G, int rg);
int fps_batch_ppt_round(int ppt);
int fps_batch_set_words(int G, int rg);
int fps_batch_point_waves(int block);  // waves of a workgroup that hold points
hipError_t launch_knn(const float*, const float*, int64_t, int64_t, int64_t, int64_t, float*,
                      int64_t*, int, int, const int64_t*, int, int64_t, int, hipStream_t);
hipError_t launch_knn_wave(const float*, const float*, int64_t, int64_t, int64_t, int64_t, float*,
                           int64_t*, int, int, const int64_t*, int, int64_t, int, hipStream_t);
hipError_t launch_ball_query_backward(const float*, const float*, const int64_t*, const float*,
                                      int64_t, int64_t, int64_t, int64_t, float*, float*, void*,
                                      hipStream_t);
size_t bq_backward_workspace_bytes(int64_t B, int64_t Q, int64_t K);

namespace api {

constexpr int64_t kMaxPoints = (int64_t)1 << 31;  // indices are int32 internally
constexpr int64_t kMaxGridY = 65535;

struct DeviceInfo {
    int checked = 0;  // 0: unknown, 1: supported, -1: unsupported
    int cus = 0;
    size_t lds_per_block = 0;
    char arch[64] = {0};
};

// Sets the calling thread's error message; returns `status`.
int fail(int status, const char* fmt, ...);
int hip_fail(hipError_t e, const char* what);
void clear_error();
const char* last_error();
// POINTOPS_OK if the device is supported (cached per device); *out gets its
// properties.
int check_device(int device, DeviceInfo** out);
int current_device(DeviceInfo** out);
long env_long(const char* name, long dflt);
// The largest G' <= G for which slices of ceil(N / G') points are all non-empty.
int64_t split_even(int64_t N, int64_t G);
// The cloud table of a ragged launch (see segments.h): tile_ptr over the
// clouds in `order` (units per cloud), then their records.
struct Table {
    std::vector<int64_t> words;
    int64_t units = 0;
    int nseg = 0;
};
Table make_table(const std::vector<int64_t>& order, const std::vector<int64_t>& units,
                 const std::vector<std::array<int64_t, 8>>& recs);
// kNN / Ball Query table: clouds with queries, `per_unit` queries per
// workgroup or wave, largest reference sets first.
Table search_table(const int64_t* q_off, const int64_t* q_cnt, const int64_t* r_off,
                   const int64_t* r_cnt, int64_t B, int per_unit, bool global_index);
// Writes the table to the start of the workspace on `stream`.
int upload(const Table& t, void* workspace, size_t workspace_bytes, hipStream_t s,
           int64_t** dev_table);
// Knobs shared by the dense and ragged launches.
int knn_waves(int kcap, int64_t tiles, int cus);
// kNN takes the grid search for this shape (when given a workspace).
bool knn_use_grid(int64_t B, int64_t Q, int64_t P);
// ... and the grid search beats the full scans for this k and shape.
bool knn_grid_pays(int64_t k, int64_t B, int64_t Q, int64_t P);
// The same two rules for `pairs` query-reference pairs in all and at most P
// references per cloud (ragged batches).
bool knn_use_grid_pairs(int64_t pairs, int64_t P);
bool knn_grid_pays_pairs(int64_t k, int64_t pairs, int64_t P);
// kNN of a ragged batch through the grid search: the workspace holds the
// per-cloud records (grid.h, GridCloud) at `clouds`, then the grid at `grid`;
// P and Q are the largest reference and query counts (every cloud keeps that
// many slots). `use` is false when the grid does not pay for these counts or
// the padding to the largest cloud would take more than eight times the
// points' own room; `total` then is the full scan's need alone.
struct RaggedKnnGrid {
    bool use = false;
    int64_t P = 0, Q = 0;
    size_t clouds = 0, grid = 0, total = 0;
    size_t grid_bytes = 0;  // the grid's own room (at `grid`)
};
RaggedKnnGrid ragged_knn_grid(const int64_t* q_cnt, const int64_t* r_cnt, int64_t B, int64_t k);
// Ball Query of a ragged batch through the index-order scan with a budget,
// then the grid pass or the resumed scan: the scan's cloud table at 0, the
// grid's records at `clouds` followed by kBqGateWords words (two gate words,
// the estimate counters), the per-query state (B x Q) at `state` and the grid
// of 2^level cells per axis at `grid`; `use` for K <= 32 and clouds of 8192
// references or more (POINTOPS_BQ_GRID=0 / 1 forbids or allows it at any
// size), with the same padding limit as the kNN grid. `grid_pairs`: the
// estimated reference tests left from which the grid pass pays.
constexpr int kBqGateWords = 1 + kBqEstimates;
struct RaggedBqGrid {
    bool use = false;
    int64_t P = 0, Q = 0;
    int level = 2;
    size_t clouds = 0, state = 0, grid = 0, total = 0;
    unsigned long long grid_pairs = 0;
};
RaggedBqGrid ragged_bq_grid(const int64_t* q_cnt, const int64_t* r_cnt, int64_t B, int64_t K);
// The ragged scan's probe (references after which a query whose hit rate
// would need more than the budget leaves for the grid) and budget, both
// multiples of 64 (POINTOPS_BQ_PROBE, POINTOPS_BQ_RAGGED_BUDGET override).
int bq_ragged_probe();
int bq_ragged_budget();
// Writes the records of the clouds (q_off[b], q_cnt[b], r_off[b], r_cnt[b],
// index base) to `dev` on `stream`, then `extra` zero words (gates and
// counters of the kernels that follow).
int upload_grid_clouds(const int64_t* q_off, const int64_t* q_cnt, const int64_t* r_off,
                       const int64_t* r_cnt, int64_t B, bool global_index, int64_t* dev,
                       int extra, hipStream_t s);
// Waves per workgroup of the grid search (one query per lane).
int knn_grid_waves(int kcap);
// The grid search's launch: 0 / -2 for one / two queries per wave, else
// knn_grid_waves (one query per lane).
int knn_grid_nw(int64_t k, int kcap, int64_t queries, int64_t refs);
int bq_queries_per_wave(int64_t rows, int cus, int max_qw);
bool bq_grid_possible(int64_t P);
int bq_scan_budget();
int bq_grid_level(int64_t P);
// Candidates a workgroup publishes per exchange of the batched FPS when its
// cloud spans G > 1 workgroups of `npw` point waves (each wave reports two):
// at most 256 in all, 512 when G > 128.
int fps_batch_rg(int64_t G, int npw);
// One-query-per-wave kNN: waves per workgroup and queries per wave; nw == 0
// selects the lane-per-query kernel.
struct KnnWavePlan {
    int nw = 0, qw = 1;
};
KnnWavePlan knn_wave_plan(int64_t k, int64_t queries, int64_t max_refs, int cus);
// Largest cloud for which FPS takes the one-exchange-per-step kernel (one
// workgroup per cloud); larger clouds take certified batches.
constexpr int64_t kFpsStepMaxPoints = 4096;

}  // namespace api
}  // namespace pointops
