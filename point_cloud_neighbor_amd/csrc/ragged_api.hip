// C ABI of the ragged-batch entry points: validation of the host-side cloud
// descriptions, launch planning, and the cloud table each launch reads.
// Declarations and contracts are in include/pointops.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <vector>

#include "../../include/pointops.h"
#include "api_internal.h"
#include "grid.h"
#include "segments.h"

using namespace pointops::api;
using pointops::kSegRecWords;
using pointops::seg_ptr_words;
using pointops::seg_table_words;
static_assert(pointops::kSegRecWords == 8, "api_internal.h declares 8-word records");

namespace pointops {
namespace api {

// The cloud table: tile_ptr over `order` (units per cloud), then the records.
Table make_table(const std::vector<int64_t>& order, const std::vector<int64_t>& units,
                 const std::vector<std::array<int64_t, kSegRecWords>>& recs) {
    Table t;
    const int64_t n = (int64_t)order.size();
    t.nseg = (int)n;
    t.words.assign((size_t)seg_table_words(n), 0);
    int64_t acc = 0;
    for (int64_t i = 0; i < n; ++i) {
        t.words[(size_t)i] = acc;
        acc += units[(size_t)order[(size_t)i]];
        const auto& r = recs[(size_t)order[(size_t)i]];
        std::copy(r.begin(), r.end(),
                  t.words.begin() + seg_ptr_words(n) + i * kSegRecWords);
    }
    t.words[(size_t)n] = acc;
    t.units = acc;
    return t;
}

// kNN and Ball Query: clouds with queries, largest reference sets first (the
// longest-running workgroups start first).
Table search_table(const int64_t* q_off, const int64_t* q_cnt, const int64_t* r_off,
                   const int64_t* r_cnt, int64_t B, int per_unit, bool global_index) {
    std::vector<int64_t> order, units((size_t)B);
    std::vector<std::array<int64_t, kSegRecWords>> recs((size_t)B);
    for (int64_t b = 0; b < B; ++b) {
        units[(size_t)b] = (q_cnt[b] + per_unit - 1) / per_unit;
        recs[(size_t)b] = {q_off[b], q_cnt[b], r_off[b], r_cnt[b], global_index ? r_off[b] : 0,
                           b, 0, 0};
        if (units[(size_t)b] > 0) order.push_back(b);
    }
    std::stable_sort(order.begin(), order.end(),
                     [&](int64_t a, int64_t c) { return r_cnt[a] > r_cnt[c]; });
    return make_table(order, units, recs);
}

static size_t al256(size_t n) { return (n + 255) / 256 * 256; }

// The grid's room grows with B times the largest counts; clouds of similar
// sizes waste little of it, one large cloud among many small ones would waste
// most (such batches keep the full scan).
constexpr int64_t kGridPadRatio = 8;

RaggedKnnGrid ragged_knn_grid(const int64_t* q_cnt, const int64_t* r_cnt, int64_t B, int64_t k) {
    RaggedKnnGrid g;
    int64_t pairs = 0, points = 0;
    for (int64_t b = 0; b < B; ++b) {
        g.P = std::max(g.P, r_cnt[b]);
        g.Q = std::max(g.Q, q_cnt[b]);
        pairs += q_cnt[b] * r_cnt[b];
        points += q_cnt[b] + r_cnt[b];
    }
    g.clouds = 0;
    g.total = B > 0 ? (size_t)seg_table_words(B) * sizeof(int64_t) : 0;  // the full scan's table
    if (B < 1 || B > kMaxGridY || g.P < 1 || g.Q < 1) return g;
    if (!knn_use_grid_pairs(pairs, g.P) || !knn_grid_pays_pairs(k, pairs, g.P)) return g;
    if (B * (g.P + g.Q) > kGridPadRatio * points) return g;
    g.use = true;
    g.grid = al256((size_t)B * kGcWords * sizeof(int64_t));  // the records
    g.grid_bytes = al256(pointops::grid_workspace_bytes(B, g.Q, g.P, pointops::knn_grid_level(g.P)));
    g.total = std::max(g.total, g.grid + g.grid_bytes);
    return g;
}

static int round64(long v) { return (int)((v + 63) / 64 * 64); }

int bq_ragged_probe() {
    const long env = env_long("POINTOPS_BQ_PROBE", 0);
    return env > 0 && env < (1L << 24) ? round64(env) : 256;
}

int bq_ragged_budget() {
    const long env = env_long("POINTOPS_BQ_RAGGED_BUDGET", 0);
    return env > 0 && env < (1L << 24) ? round64(env) : 2048;
}

RaggedBqGrid ragged_bq_grid(const int64_t* q_cnt, const int64_t* r_cnt, int64_t B, int64_t K) {
    RaggedBqGrid g;
    int64_t points = 0;
    for (int64_t b = 0; b < B; ++b) {
        g.P = std::max(g.P, r_cnt[b]);
        g.Q = std::max(g.Q, q_cnt[b]);
        points += q_cnt[b] + r_cnt[b];
    }
    g.total = B > 0 ? (size_t)seg_table_words(B) * sizeof(int64_t) : 0;  // the scan's table
    if (K < 1 || K > 32 || B < 1 || B > kMaxGridY || g.P < 1 || g.Q < 1) return g;
    const long env = env_long("POINTOPS_BQ_GRID", -1);
    if (env == 0 || (env != 1 && g.P < 8192)) return g;
    if (B * (g.P + g.Q) > kGridPadRatio * points) return g;
    g.use = true;
    g.level = bq_grid_level(g.P);
    g.clouds = al256((size_t)seg_table_words(B) * sizeof(int64_t));  // the scan's table
    g.state = g.clouds + al256(((size_t)B * kGcWords + kBqGateWords) * sizeof(int64_t));
    g.grid = g.state + al256((size_t)B * g.Q * sizeof(uint2));
    g.total = g.grid + al256(pointops::ball_query_ragged_grid_bytes(B, g.Q, g.P, g.level));
    // The grid pays once the reference tests left would take longer than its
    // build and pass: measured on the ragged 16-cloud batch (317k points),
    // about 40 us plus 0.25 ns per point, against scans of about 1.1 * 10^12
    // tests per second. POINTOPS_BQ_GRID_PAIRS overrides.
    const long env_pairs = env_long("POINTOPS_BQ_GRID_PAIRS", -1);
    g.grid_pairs = env_pairs >= 0 ? (unsigned long long)env_pairs
                                  : (unsigned long long)(1.1e6 * (40.0 + 2.5e-4 * (double)points));
    return g;
}

int upload_grid_clouds(const int64_t* q_off, const int64_t* q_cnt, const int64_t* r_off,
                       const int64_t* r_cnt, int64_t B, bool global_index, int64_t* dev,
                       int extra, hipStream_t s) {
    std::vector<int64_t> w((size_t)B * kGcWords + (size_t)extra, 0);
    for (int64_t b = 0; b < B; ++b) {
        int64_t* r = w.data() + b * kGcWords;
        r[kGcROff] = r_off[b];
        r[kGcRCnt] = r_cnt[b];
        r[kGcQOff] = q_off[b];
        r[kGcQCnt] = q_cnt[b];
        r[kGcIdxBase] = global_index ? r_off[b] : 0;
    }
    hipError_t e = pointops::upload_words(w.data(), (int64_t)w.size(), dev, s);
    return e == hipSuccess ? POINTOPS_OK : hip_fail(e, "cloud record upload");
}

int upload(const Table& t, void* workspace, size_t workspace_bytes, hipStream_t s,
           int64_t** dev_table) {
    const size_t need = t.words.size() * sizeof(int64_t);
    if (!workspace || workspace_bytes < need)
        return fail(POINTOPS_INVALID_ARGUMENT, "workspace of %zu bytes given, %zu needed",
                    workspace_bytes, need);
    *dev_table = (int64_t*)workspace;
    hipError_t e = pointops::upload_words(t.words.data(), (int64_t)t.words.size(), *dev_table, s);
    if (e != hipSuccess) return hip_fail(e, "cloud table upload");
    return POINTOPS_OK;
}

}  // namespace api
}  // namespace pointops

namespace {

constexpr size_t kHeader = 256;  // status word of FPS, then the table

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Every segment inside [0, rows) with fewer than 2^31 points; with `disjoint`,
// no two non-empty segments share a row (they are output rows).
int check_segments(const char* what, const int64_t* off, const int64_t* cnt, int64_t B,
                   int64_t rows, bool disjoint) {
    if (B > 0 && (!off || !cnt)) return fail(POINTOPS_INVALID_ARGUMENT, "%s: null segment array", what);
    for (int64_t b = 0; b < B; ++b) {
        if (off[b] < 0 || cnt[b] < 0 || off[b] > rows || cnt[b] > rows - off[b])
            return fail(POINTOPS_INVALID_ARGUMENT,
                        "%s: segment %lld = [%lld, +%lld) is not inside the %lld rows", what,
                        (long long)b, (long long)off[b], (long long)cnt[b], (long long)rows);
        if (cnt[b] >= kMaxPoints)
            return fail(POINTOPS_UNSUPPORTED, "%s: segment %lld has 2^31 or more points", what,
                        (long long)b);
    }
    if (disjoint) {
        std::vector<int64_t> order;
        for (int64_t b = 0; b < B; ++b)
            if (cnt[b] > 0) order.push_back(b);
        std::sort(order.begin(), order.end(),
                  [&](int64_t a, int64_t c) { return off[a] < off[c]; });
        for (size_t i = 1; i < order.size(); ++i)
            if (off[order[i - 1]] + cnt[order[i - 1]] > off[order[i]])
                return fail(POINTOPS_INVALID_ARGUMENT, "%s: segments %lld and %lld overlap", what,
                            (long long)order[i - 1], (long long)order[i]);
    }
    return POINTOPS_OK;
}

int check_search(const float* query, int64_t q_rows, const int64_t* q_off, const int64_t* q_cnt,
                 const float* ref, int64_t r_rows, const int64_t* r_off, const int64_t* r_cnt,
                 int64_t B, const void* out_a, const void* out_b) {
    if (B < 0 || q_rows < 0 || r_rows < 0) return fail(POINTOPS_INVALID_ARGUMENT, "negative size");
    if (B >= kMaxPoints) return fail(POINTOPS_UNSUPPORTED, "B >= 2^31");
    int st = check_segments("query", q_off, q_cnt, B, q_rows, true);
    if (st != POINTOPS_OK) return st;
    st = check_segments("ref", r_off, r_cnt, B, r_rows, false);
    if (st != POINTOPS_OK) return st;
    if (q_rows > 0 && (!query || !out_a || !out_b))
        return fail(POINTOPS_INVALID_ARGUMENT, "null pointer");
    if (r_rows > 0 && !ref) return fail(POINTOPS_INVALID_ARGUMENT, "null pointer");
    return POINTOPS_OK;
}

// ------------------------------------------------------------------ FPS plan

struct RaggedFps {
    bool batch = false;
    int ppt = 0, block = 0, cpl = 1;
    int64_t max_n = 0;   // largest cloud (step launch: LDS copy size)
    size_t lds = 0;      // batch launch: largest candidate stage
    int64_t words = 0;   // exchange words (batch)
    Table table;
    int err = POINTOPS_OK;
};

size_t fps_ragged_bytes(const RaggedFps& p) {
    return kHeader + align256(p.table.words.size() * sizeof(int64_t)) +
           (size_t)p.words * sizeof(uint64_t);
}

// One workgroup per cloud when every cloud fits one (the step kernel: no
// exchange at all); otherwise the certified-batch kernel with each cloud's
// own number of workgroups (about 1600 points each, at most 128), clouds
// spanning several workgroups numbered first so that they are all resident
// together, then the one-workgroup clouds, longest first.
RaggedFps plan_fps_ragged(const int64_t* x_off, const int64_t* x_cnt, const int64_t* o_off,
                          const int64_t* o_cnt, const int64_t* start, int64_t B,
                          bool global_index, const DeviceInfo& dev) {
    RaggedFps p;
    std::vector<int64_t> active;
    for (int64_t b = 0; b < B; ++b)
        if (o_cnt[b] > 0) {
            active.push_back(b);
            p.max_n = std::max(p.max_n, x_cnt[b]);
        }
    std::vector<std::array<int64_t, kSegRecWords>> recs((size_t)B);
    std::vector<int64_t> units((size_t)B, 0);
    auto rec = [&](int64_t b) -> std::array<int64_t, kSegRecWords> {
        return {x_off[b], x_cnt[b], o_off[b], o_cnt[b], global_index ? x_off[b] : 0,
                start ? start[b] : 0, 0, 0};
    };
    const char* mode = getenv("POINTOPS_FPS_MODE");
    const int64_t max_slice =
        std::min<int64_t>(16 * 1024, ((int64_t)dev.lds_per_block - 1024) / 12);
    const bool step = mode && strcmp(mode, "step") == 0 ? p.max_n <= max_slice
                                                         : p.max_n <= kFpsStepMaxPoints;
    if (!(mode && strcmp(mode, "batch") == 0) && step) {
        p.batch = false;
        p.block = p.max_n > 1024 ? 1024 : 256;
        p.ppt = (int)((p.max_n + p.block - 1) / p.block);
        for (int64_t b : active) {
            units[(size_t)b] = 1;
            recs[(size_t)b] = rec(b);
        }
        std::stable_sort(active.begin(), active.end(),
                         [&](int64_t a, int64_t c) { return o_cnt[a] > o_cnt[c]; });
        p.table = make_table(active, units, recs);
        return p;
    }
    p.batch = true;
    std::vector<int64_t> want((size_t)B, 1), G((size_t)B, 1), rg((size_t)B, 1);
    for (int64_t b : active)
        want[(size_t)b] = x_cnt[b] <= 2048 ? 1 : std::min<int64_t>((x_cnt[b] + 1599) / 1600, 128);
    int block = 0;
    for (int attempt = 0; attempt < 12; ++attempt) {
        int64_t slice_max = 1;
        for (int64_t b : active) {
            G[(size_t)b] = split_even(x_cnt[b], want[(size_t)b]);
            slice_max = std::max(slice_max, (x_cnt[b] + G[(size_t)b] - 1) / G[(size_t)b]);
        }
        p.block = block ? block : (slice_max <= 768 ? 256 : 1024);
        const int npw = pointops::fps_batch_point_waves(p.block);
        p.ppt = pointops::fps_batch_ppt_round((int)((slice_max + npw * 64 - 1) / (npw * 64)));
        if (p.ppt < 0) {  // more than 16 points per thread somewhere
            if (p.block == 256) { block = 1024; continue; }
            for (int64_t b : active)
                want[(size_t)b] = std::max(want[(size_t)b], (x_cnt[b] + 16 * 768 - 1) / (16 * 768));
            continue;
        }
        int64_t cand = 0, multi = 0;
        p.lds = 0;
        for (int64_t b : active) {
            const int64_t g = G[(size_t)b];
            if (g == 1) { rg[(size_t)b] = npw; continue; }
            const int64_t r = fps_batch_rg(g, npw);
            rg[(size_t)b] = r;
            cand = std::max(cand, g * r);
            multi += g;
            p.lds = std::max(p.lds, pointops::fps_batch_lds_bytes((int)g, (int)r));
        }
        if (cand > 512) break;
        p.cpl = cand <= 64 ? 1 : cand <= 128 ? 2 : cand <= 256 ? 4 : 8;
        if (p.block == 256 && p.cpl > 1) { block = 1024; continue; }
        int cap = 0;
        hipError_t e =
            pointops::fps_batch_capacity(p.ppt, p.block, p.cpl, p.lds, false, dev.cus, &cap);
        if (e != hipSuccess) { p.err = hip_fail(e, "fps occupancy query"); return p; }
        if (multi > cap) {  // fewer, larger slices
            for (int64_t b : active)
                want[(size_t)b] = std::max<int64_t>(1, G[(size_t)b] * cap / (multi + 1));
            continue;
        }
        // exchange words: the clouds spanning several workgroups, in unit order
        std::vector<int64_t> order = active;
        std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t c) {
            const bool ma = G[(size_t)a] > 1, mc = G[(size_t)c] > 1;
            if (ma != mc) return ma;
            return ma ? x_cnt[a] > x_cnt[c] : o_cnt[a] > o_cnt[c];
        });
        p.words = 0;
        for (int64_t b : order) {
            units[(size_t)b] = G[(size_t)b];
            recs[(size_t)b] = rec(b);
            recs[(size_t)b][pointops::kFrRG] = rg[(size_t)b];
            if (G[(size_t)b] > 1) {
                recs[(size_t)b][pointops::kFrWOff] = p.words;
                p.words += 2 * pointops::fps_batch_set_words((int)G[(size_t)b], (int)rg[(size_t)b]);
            }
        }
        p.table = make_table(order, units, recs);
        return p;
    }
    p.err = fail(POINTOPS_UNSUPPORTED, "no FPS launch shape fits this ragged batch");
    return p;
}

int check_fps_ragged(const float* xyz, int64_t rows, const int64_t* x_off, const int64_t* x_cnt,
                     const int64_t* start, int64_t B, const int64_t* out_idx, int64_t out_rows,
                     const int64_t* o_off, const int64_t* o_cnt) {
    if (B < 0 || rows < 0 || out_rows < 0) return fail(POINTOPS_INVALID_ARGUMENT, "negative size");
    if (B >= kMaxPoints) return fail(POINTOPS_UNSUPPORTED, "B >= 2^31");
    int st = check_segments("xyz", x_off, x_cnt, B, rows, false);
    if (st != POINTOPS_OK) return st;
    st = check_segments("out", o_off, o_cnt, B, out_rows, true);
    if (st != POINTOPS_OK) return st;
    for (int64_t b = 0; b < B; ++b) {
        if (o_cnt[b] == 0) continue;
        if (x_cnt[b] == 0)
            return fail(POINTOPS_INVALID_ARGUMENT, "cloud %lld: no points but %lld samples",
                        (long long)b, (long long)o_cnt[b]);
        const int64_t s = start ? start[b] : 0;
        if (s < 0 || s >= x_cnt[b])
            return fail(POINTOPS_INVALID_ARGUMENT, "cloud %lld: start %lld not in [0, %lld)",
                        (long long)b, (long long)s, (long long)x_cnt[b]);
    }
    if (out_rows > 0 && !out_idx) return fail(POINTOPS_INVALID_ARGUMENT, "null pointer");
    if (rows > 0 && !xyz) return fail(POINTOPS_INVALID_ARGUMENT, "null pointer");
    return POINTOPS_OK;
}

}  // namespace

extern "C" {

size_t pointops_ragged_workspace_bytes(int64_t B) {
    return B < 0 ? 0 : (size_t)seg_table_words(B) * sizeof(int64_t);
}

size_t pointops_ball_query_ragged_workspace_bytes(const int64_t* q_cnt, const int64_t* r_cnt,
                                                  int64_t B, int64_t K) {
    if (B < 0 || (B > 0 && (!q_cnt || !r_cnt))) return 0;
    for (int64_t b = 0; b < B; ++b)
        if (q_cnt[b] < 0 || r_cnt[b] < 0 || q_cnt[b] >= kMaxPoints || r_cnt[b] >= kMaxPoints)
            return 0;
    return std::max(pointops_ragged_workspace_bytes(B), ragged_bq_grid(q_cnt, r_cnt, B, K).total);
}

size_t pointops_knn_ragged_workspace_bytes(const int64_t* q_cnt, const int64_t* r_cnt, int64_t B,
                                           int64_t k) {
    if (B < 0 || (B > 0 && (!q_cnt || !r_cnt))) return 0;
    for (int64_t b = 0; b < B; ++b)
        if (q_cnt[b] < 0 || r_cnt[b] < 0 || q_cnt[b] >= kMaxPoints || r_cnt[b] >= kMaxPoints)
            return 0;
    return std::max(pointops_ragged_workspace_bytes(B), ragged_knn_grid(q_cnt, r_cnt, B, k).total);
}

int pointops_knn_ragged(const float* query, int64_t q_rows, const int64_t* q_off,
                        const int64_t* q_cnt, const float* ref, int64_t r_rows,
                        const int64_t* r_off, const int64_t* r_cnt, int64_t B, int64_t k,
                        int global_index, float* out_dist, int64_t* out_idx, void* workspace,
                        size_t workspace_bytes, void* stream) {
    clear_error();
    if (k < 1) return fail(POINTOPS_INVALID_ARGUMENT, "k = %lld must be >= 1", (long long)k);
    if (k > POINTOPS_KNN_KMAX)
        return fail(POINTOPS_UNSUPPORTED, "k = %lld exceeds POINTOPS_KNN_KMAX = %d",
                    (long long)k, POINTOPS_KNN_KMAX);
    int st = check_search(query, q_rows, q_off, q_cnt, ref, r_rows, r_off, r_cnt, B, out_dist,
                          out_idx);
    if (st != POINTOPS_OK) return st;
    DeviceInfo* dev = nullptr;
    st = current_device(&dev);
    if (st != POINTOPS_OK) return st;
    int64_t queries = 0, max_refs = 0;
    for (int64_t b = 0; b < B; ++b) {
        queries += q_cnt[b];
        if (q_cnt[b] > 0) max_refs = std::max(max_refs, r_cnt[b]);
    }
    if (queries == 0) return POINTOPS_OK;
    hipStream_t s = (hipStream_t)stream;
    int kcap = 1;
    while (kcap < k) kcap *= 2;
    // Grid search when it pays and the workspace has its room; otherwise the
    // full scans below.
    const RaggedKnnGrid g = ragged_knn_grid(q_cnt, r_cnt, B, k);
    if (g.use && workspace && workspace_bytes >= g.total) {
        char* ws = (char*)workspace;
        int64_t* clouds = (int64_t*)(ws + g.clouds);
        st = upload_grid_clouds(q_off, q_cnt, r_off, r_cnt, B, global_index != 0, clouds, 0, s);
        if (st != POINTOPS_OK) return st;
        int64_t refs = 0;
        for (int64_t b = 0; b < B; ++b) refs += q_cnt[b] > 0 ? r_cnt[b] : 0;
        hipError_t e = pointops::launch_knn_grid(query, ref, B, g.Q, g.P, k, out_dist, out_idx,
                                                 kcap, knn_grid_nw(k, kcap, queries, refs),
                                                 ws + g.grid, 0, clouds, s);
        if (e != hipSuccess) return hip_fail(e, "knn launch");
        return POINTOPS_OK;
    }
    const KnnWavePlan wp = knn_wave_plan(k, queries, max_refs, dev->cus);
    const Table t = search_table(q_off, q_cnt, r_off, r_cnt, B, wp.nw ? wp.nw * wp.qw : 64,
                                 global_index != 0);
    if (t.units == 0) return POINTOPS_OK;
    if (t.units >= kMaxPoints) return fail(POINTOPS_UNSUPPORTED, "too many workgroups");
    int64_t* table = nullptr;
    st = upload(t, workspace, workspace_bytes, s, &table);
    if (st != POINTOPS_OK) return st;
    if (wp.nw) {
        hipError_t e = pointops::launch_knn_wave(query, ref, 0, 0, 0, k, out_dist, out_idx, wp.nw,
                                                 wp.qw, table, t.nseg, t.units, 0, s);
        if (e != hipSuccess) return hip_fail(e, "knn launch");
        return POINTOPS_OK;
    }
    hipError_t e = pointops::launch_knn(query, ref, 0, 0, 0, k, out_dist, out_idx, kcap,
                                        knn_waves(kcap, t.units, dev->cus), table, t.nseg,
                                        t.units, 0, s);
    if (e != hipSuccess) return hip_fail(e, "knn launch");
    return POINTOPS_OK;
}

int pointops_ball_query_ragged(const float* query, int64_t q_rows, const int64_t* q_off,
                               const int64_t* q_cnt, const float* ref, int64_t r_rows,
                               const int64_t* r_off, const int64_t* r_cnt, int64_t B,
                               float radius, int64_t K, int global_index, float* out_dist2,
                               int64_t* out_idx, void* workspace, size_t workspace_bytes,
                               void* stream) {
    clear_error();
    if (!(radius > 0.0f) || std::isinf(radius))
        return fail(POINTOPS_INVALID_ARGUMENT, "radius must be finite and > 0");
    if (K < 1) return fail(POINTOPS_INVALID_ARGUMENT, "K must be >= 1");
    if (K >= kMaxPoints) return fail(POINTOPS_UNSUPPORTED, "K >= 2^31");
    int st = check_search(query, q_rows, q_off, q_cnt, ref, r_rows, r_off, r_cnt, B, out_dist2,
                          out_idx);
    if (st != POINTOPS_OK) return st;
    DeviceInfo* dev = nullptr;
    st = current_device(&dev);
    if (st != POINTOPS_OK) return st;
    int64_t rows = 0;
    for (int64_t b = 0; b < B; ++b) rows += q_cnt[b];
    if (rows == 0) return POINTOPS_OK;
    hipStream_t s = (hipStream_t)stream;
    // R2 = fl32(r32 * r32), as for dense batches.
    volatile float r32 = radius;
    const float r2 = r32 * r32;
    // At most 2 queries per wave: clouds differ in size and queries stop at K
    // at different points, so short waves balance better (measured on ragged
    // batches of 35k queries: 0.26 ms with 1 or 2, 0.37 ms with 8).
    const int qw = bq_queries_per_wave(rows, dev->cus, 2);
    const Table t = search_table(q_off, q_cnt, r_off, r_cnt, B, qw, global_index != 0);
    if (t.units == 0) return POINTOPS_OK;
    if (t.units >= kMaxPoints) return fail(POINTOPS_UNSUPPORTED, "too many waves");
    int64_t* table = nullptr;
    st = upload(t, workspace, workspace_bytes, s, &table);
    if (st != POINTOPS_OK) return st;
    // With the grid's room: the scan in its budgeted mode; then, as the
    // estimate of the tests left decides on the device (no host round trip),
    // the grid build and the grid pass, or the scan resumed where each query
    // left off. Every step after the first reads its gate and may do nothing.
    const RaggedBqGrid g = ragged_bq_grid(q_cnt, r_cnt, B, K);
    if (g.use && workspace_bytes >= g.total) {
        char* ws = (char*)workspace;
        int64_t* clouds = (int64_t*)(ws + g.clouds);
        uint32_t* gate = (uint32_t*)(clouds + B * pointops::kGcWords);  // grid, resume
        unsigned long long* estimate = (unsigned long long*)(clouds + B * pointops::kGcWords + 1);
        uint2* state = (uint2*)(ws + g.state);
        st = upload_grid_clouds(q_off, q_cnt, r_off, r_cnt, B, global_index != 0, clouds, 1, s);
        if (st != POINTOPS_OK) return st;
        hipError_t ez = pointops::launch_zero_f32((float*)estimate, 2 * pointops::kBqEstimates, s);
        if (ez != hipSuccess) return hip_fail(ez, "ball_query estimate clear");
        pointops::BqBudget bud{state, estimate, gate + 1, bq_ragged_probe(), bq_ragged_budget(),
                               (int)g.Q};
        hipError_t e = pointops::launch_ball_query(query, ref, 0, 0, 0, r2, K, out_dist2,
                                                   out_idx, qw, table, t.nseg, t.units, s, 1, bud);
        if (e == hipSuccess) e = pointops::launch_ball_query_decide(estimate, g.grid_pairs, gate, s);
        if (e == hipSuccess)
            e = pointops::launch_ball_query_ragged_grid(query, ref, B, g.Q, g.P, r2, K, out_dist2,
                                                        out_idx, g.level, clouds, gate, state,
                                                        ws + g.grid, s);
        if (e == hipSuccess)
            e = pointops::launch_ball_query(query, ref, 0, 0, 0, r2, K, out_dist2, out_idx, qw,
                                            table, t.nseg, t.units, s, 2, bud);
        if (e != hipSuccess) return hip_fail(e, "ball_query launch");
        return POINTOPS_OK;
    }
    hipError_t e = pointops::launch_ball_query(query, ref, 0, 0, 0, r2, K, out_dist2, out_idx,
                                               qw, table, t.nseg, t.units, s);
    if (e != hipSuccess) return hip_fail(e, "ball_query launch");
    return POINTOPS_OK;
}

size_t pointops_fps_ragged_workspace_bytes(const int64_t* x_cnt, const int64_t* out_cnt,
                                           int64_t B) {
    if (B <= 0 || !x_cnt || !out_cnt) return kHeader;
    DeviceInfo* dev = nullptr;
    DeviceInfo fallback;
    fallback.cus = 256;
    fallback.lds_per_block = 160 * 1024;
    if (current_device(&dev) != POINTOPS_OK) dev = &fallback;
    std::vector<int64_t> zeros((size_t)B, 0);
    for (int64_t b = 0; b < B; ++b)
        if (x_cnt[b] < 0 || out_cnt[b] < 0 || (out_cnt[b] > 0 && x_cnt[b] == 0) ||
            x_cnt[b] >= kMaxPoints)
            return 0;
    const RaggedFps p = plan_fps_ragged(zeros.data(), x_cnt, zeros.data(), out_cnt, nullptr, B,
                                        false, *dev);
    clear_error();
    return p.err == POINTOPS_OK ? fps_ragged_bytes(p) : 0;
}

int pointops_fps_ragged(const float* xyz, int64_t rows, const int64_t* x_off,
                        const int64_t* x_cnt, const int64_t* start, int64_t B, int64_t* out_idx,
                        float* out_xyz, int64_t out_rows, const int64_t* out_off,
                        const int64_t* out_cnt, int global_index, void* workspace,
                        size_t workspace_bytes, void* stream) {
    clear_error();
    int st = check_fps_ragged(xyz, rows, x_off, x_cnt, start, B, out_idx, out_rows, out_off,
                              out_cnt);
    if (st != POINTOPS_OK) return st;
    DeviceInfo* dev = nullptr;
    st = current_device(&dev);
    if (st != POINTOPS_OK) return st;
    const RaggedFps p = plan_fps_ragged(x_off, x_cnt, out_off, out_cnt, start, B,
                                        global_index != 0, *dev);
    if (p.err != POINTOPS_OK) return p.err;
    if (p.table.units == 0) return POINTOPS_OK;
    const size_t need = fps_ragged_bytes(p);
    if (!workspace || workspace_bytes < need)
        return fail(POINTOPS_INVALID_ARGUMENT, "workspace of %zu bytes given, %zu needed",
                    workspace_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    // clear the status word and the exchange words, then write the table
    hipError_t e = pointops::launch_fps_clear(workspace, need, s);
    if (e != hipSuccess) return hip_fail(e, "fps workspace clear");
    int64_t* table = (int64_t*)((char*)workspace + kHeader);
    e = pointops::upload_words(p.table.words.data(), (int64_t)p.table.words.size(), table, s);
    if (e != hipSuccess) return hip_fail(e, "cloud table upload");
    uint64_t* words = (uint64_t*)((char*)table + align256(p.table.words.size() * sizeof(int64_t)));
    const uint32_t spin = (uint32_t)env_long("POINTOPS_FPS_SPIN_LIMIT", 1L << 22);
    if (p.batch)
        e = pointops::launch_fps_batch(xyz, 0, 0, 0, 0, out_idx, out_xyz, workspace, 0, p.ppt,
                                       p.block, 0, p.cpl, false, spin, s, table, p.table.nseg,
                                       p.table.units, words, p.lds);
    else
        e = pointops::launch_fps(xyz, 0, p.max_n, 0, 0, out_idx, out_xyz, workspace, 1, p.ppt,
                                 p.block, spin, s, table, p.table.nseg, p.table.units);
    if (e != hipSuccess) return hip_fail(e, "fps launch");
    return POINTOPS_OK;
}

}  // extern "C"
