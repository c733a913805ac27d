// C ABI of the pointops library: argument validation, device check, launch
// geometry. Declarations and the contract of every entry point are in
// include/pointops.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <utility>

#include "../../include/pointops.h"
#include "api_internal.h"


namespace pointops {
namespace api {

thread_local char g_err[512];

void clear_error() { g_err[0] = 0; }
const char* last_error() { return g_err; }

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(POINTOPS_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

int check_device(int device, DeviceInfo** out) {
    if (device < 0 || device >= kMaxDevices)
        return fail(POINTOPS_UNSUPPORTED_DEVICE, "device %d out of range", device);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DeviceInfo& d = g_dev[device];
    if (d.checked == 0) {
        hipDeviceProp_t prop;
        hipError_t e = hipGetDeviceProperties(&prop, device);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
        snprintf(d.arch, sizeof d.arch, "%s", prop.gcnArchName);
        d.cus = prop.multiProcessorCount;
        d.lds_per_block = prop.sharedMemPerBlock;
        const bool gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        const char* force = getenv("POINTOPS_FORCE_UNSUPPORTED_DEVICE");  // test hook
        d.checked = (gfx950 && prop.warpSize == 64 && !(force && force[0] == '1')) ? 1 : -1;
    }
    if (out) *out = &d;
    if (d.checked != 1)
        return fail(POINTOPS_UNSUPPORTED_DEVICE,
                    "device %d (%s) is not a gfx950 GPU with 64-wide wavefronts", device, d.arch);
    return POINTOPS_OK;
}

int current_device(DeviceInfo** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    return check_device(dev, out);
}

long env_long(const char* name, long dflt) {
    const char* v = getenv(name);
    if (!v || !*v) return dflt;
    char* end = nullptr;
    long x = strtol(v, &end, 10);
    return (end && *end == 0) ? x : dflt;
}

int64_t split_even(int64_t N, int64_t G) {
    // every slice non-empty: with slice = ceil(N/G) the last slice starts at
    // (G-1)*slice, which must be < N
    G = std::max<int64_t>(1, std::min<int64_t>(G, N));
    while (G > 1 && (G - 1) * ((N + G - 1) / G) >= N) --G;
    return G;
}

// kNN: waves per workgroup, each scanning its share of the references. Four
// (two for k > 32, whose lists need more registers and LDS); eight when the
// launch has too few 64-query workgroups to give every SIMD four waves
// (measured on ragged batches of 35k queries: 0.60 ms with eight, 0.83 ms with
// four).
int knn_waves(int kcap, int64_t tiles, int cus) {
    int nw = kcap >= 64 ? 2 : 4;
    // few workgroups: more waves each (k = 32 is best at 4: the merge of the
    // waves' lists grows with k)
    if (kcap <= 16 && tiles * 4 < (int64_t)std::max(1, cus) * 16) nw = 8;
    const long nw_env = env_long("POINTOPS_KNN_WAVES", 0);
    if (nw_env == 1 || (nw_env == 2 && kcap >= 16) || (nw_env == 4 && kcap < 64) ||
        (nw_env == 8 && kcap < 64))
        nw = (int)nw_env;
    return nw;
}

// kNN takes the grid path (sort, boxes, culled search) when the references
// are many enough for the sort to pay: at least 8192 per cloud and 2^22
// query-reference pairs in all. POINTOPS_KNN_GRID=0 / 1 forces either path.
bool knn_use_grid_pairs(int64_t pairs, int64_t P) {
    const long env = env_long("POINTOPS_KNN_GRID", -1);
    if (env == 0 || env == 1) return env == 1 && P >= 1;
    return P >= 8192 && pairs >= ((int64_t)1 << 22);
}

bool knn_use_grid(int64_t B, int64_t Q, int64_t P) { return knn_use_grid_pairs(B * Q * P, P); }

// With one query per wave (k <= 32) the grid search, its sort and box build
// included, is at least as fast as the best full scan wherever it is taken
// (uniform clouds, grid / full scan: 256 queries on 100k references, k = 16:
// 0.064 / 0.18 ms; 16384 on 100k, k = 32: 0.091 / 0.47 ms; 256 on 16384,
// k = 1: 0.044 / 0.047 ms; 4096 on 16384, k = 16: 0.056 / 0.065 ms; 1024 on
// 2^20, k = 16: 0.18 / 1.18 ms; 32 clouds of 512 queries on 8192 points near
// a sphere, k = 32: 0.094 / 0.108 ms). Above k = 32 only the lane-per-query
// grid kernel remains, and it pays from 32768 references. POINTOPS_KNN_GRID=1
// forces the grid.
bool knn_grid_pays_pairs(int64_t k, int64_t pairs, int64_t P) {
    (void)pairs;
    if (env_long("POINTOPS_KNN_GRID", -1) == 1) return true;
    return k <= 32 || P >= 32768;
}

bool knn_grid_pays(int64_t k, int64_t B, int64_t Q, int64_t P) {
    return knn_grid_pays_pairs(k, B * Q * P, P);
}

// Full scans with k <= 32 take one query per wave (knn_wave.hip): its lists
// merge candidates 32 at a time, where the lane-per-query kernel pays a
// k-long insertion per candidate and needs many queries to fill the chip.
// Measured on uniform clouds (lane-per-query / one / two queries per wave):
// 1024 queries, 100k references, k = 16: 0.75 / 0.19 / 0.26 ms; 32 clouds of
// 512 queries and 8192 references, k = 32: 0.31 / 0.11 / 0.11 ms; 100k x
// 100k, k = 16: 2.81 / 2.94 / 2.27 ms. Two queries per wave share each
// reference read and pay from 64 queries per CU on. The lane-per-query kernel
// stays for k <= 8 with many queries on small clouds (16 clouds of 8192
// queries and 2048 references, k = 3: 0.12 / 0.20 / 0.18 ms; 16 clouds of 4096
// queries and 8192 references, k = 8: 0.21 / - / 0.26 ms), where the wave's
// fixed cost per query (the first sort, the merges) outweighs its short
// scan. POINTOPS_KNN_WAVE=0 / 1 forces either kernel; POINTOPS_KNN_WAVE_NW
// picks 4, 8 or 16 waves per workgroup and POINTOPS_KNN_WAVE_QW 1 or 2
// queries per wave.
KnnWavePlan knn_wave_plan(int64_t k, int64_t queries, int64_t max_refs, int cus) {
    KnnWavePlan p;
    if (k > 32) return p;
    const long env = env_long("POINTOPS_KNN_WAVE", -1);
    if (env == 0) return p;
    const int64_t c = std::max(1, cus);
    if (env != 1 && k <= 8 && queries >= 256 * c && max_refs <= 16384) return p;
    const long nw = env_long("POINTOPS_KNN_WAVE_NW", 8);
    p.nw = nw == 4 || nw == 16 ? (int)nw : 8;
    const long qw = env_long("POINTOPS_KNN_WAVE_QW", 0);
    p.qw = qw == 1 || qw == 2 ? (int)qw : (queries >= 64 * c ? 2 : 1);
    return p;
}

// Two waves per 64 queries: each wave keeps its own list, so more waves mean
// more insertions; fewer leave too few waves to hide latency (100k uniform,
// k=16: 0.44 / 0.33 / 0.37 / 0.49 ms for 1 / 2 / 4 / 8).
int knn_grid_waves(int kcap) {
    const long env = env_long("POINTOPS_KNN_GRID_WAVES", 0);
    if (kcap == 16 && (env == 1 || env == 2 || env == 4 || env == 8)) return (int)env;
    return 2;
}

// The grid search's kernel: for k <= 32 one query per wave (0), or two (-2)
// where the queries are at least half as many as the references (neighbours
// in grid order then open nearly the same boxes and share their loads); else
// one query per lane (knn_grid_waves). Measured (uniform clouds, build
// included, per lane / one per wave / two per wave): 100k queries on 100k
// references, k = 16: 0.31 / 0.20 / 0.184 ms; k = 3: 0.18 / 0.156 / 0.144 ms;
// 12500 on 100k, k = 16: 0.38 / 0.079 / 0.083 ms; 16384 on 2^20, k = 32:
// 1.54 / 0.218 / 0.224 ms; the ragged 16-cloud batch (35k queries, k = 16):
// 0.47 / 0.177 / 0.175 ms. POINTOPS_KNN_GRID_WAVE=0 / 1 / 2 forces one
// (1 and 2 only for k <= 32).
int knn_grid_nw(int64_t k, int kcap, int64_t queries, int64_t refs) {
    const long env = env_long("POINTOPS_KNN_GRID_WAVE", -1);
    if (k > 32 || env == 0) return knn_grid_waves(kcap);
    if (env == 1) return 0;
    return env == 2 || queries * 2 >= refs ? -2 : 0;
}

// Ball Query: queries per wave. Fewer queries per wave until the grid is about
// one device-full of waves; at most 8 (measured faster than 16 on 100k x 100k:
// the shorter waves balance better).
// Up to 256 candidates per cloud (four slots per lane of the certifying wave)
// and at most 8 per workgroup (beyond that the exchanges hardly fall while each
// grows: 32 clouds of 8192 points on 6 workgroups each, 4 / 6 / 8 / 12 / 30
// candidates per workgroup: 0.354 / 0.305 / 0.295 / 0.308 / 0.366 ms);
// POINTOPS_FPS_RG overrides it up to 512 candidates (eight slots per lane,
// the most the kernel holds) or the workgroup's 2 * npw reports.
int fps_batch_rg(int64_t G, int npw) {
    const long env = env_long("POINTOPS_FPS_RG", 0);
    const int64_t g = std::max<int64_t>(G, 1);
    const int64_t total = G > 128 ? 512 : 256;  // candidates per exchange in all
    const int64_t cap =
        std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(2 * npw, 8), total / g));
    const int64_t most = std::max<int64_t>(1, std::min<int64_t>(2 * npw, 512 / g));
    return (int)(env > 0 ? std::min<int64_t>(env, most) : cap);
}

// Ball Query with a workspace: the culled index-order scan, and for clouds of
// more than 32768 references a budget of 128 scanned blocks (8192 references)
// per wave, after which the queries still short of K go to the grid pass
// (clouds in random order; sorted clouds finish within the budget, and the
// grid kernels then return at once). POINTOPS_BQ_GRID=0 / 1 forbids or allows
// it at any size; POINTOPS_BQ_BUDGET sets the budget in blocks.
bool bq_grid_possible(int64_t P) {
    const long env = env_long("POINTOPS_BQ_GRID", -1);
    if (env == 0 || env == 1) return env == 1;
    return P > 32768;
}

int bq_scan_budget() {
    const long env = env_long("POINTOPS_BQ_BUDGET", 0);
    return env > 0 && env < (1L << 30) ? (int)env : 128;
}

// Cells per axis of the Ball Query's grid: one level finer than the kNN
// search's, so the counting sort's atomics spread over more cells where points
// cluster (the cells decide only the order of the sorted copies, so no result
// depends on them). POINTOPS_BQ_GRID_LEVEL overrides (2..7).
int bq_grid_level(int64_t P) {
    const long env = env_long("POINTOPS_BQ_GRID_LEVEL", 0);
    if (env >= 2 && env <= 7) return (int)env;
    return std::min(7, pointops::knn_grid_level(P) + 1);
}

int bq_queries_per_wave(int64_t rows, int cus, int max_qw) {
    const int64_t slots = (int64_t)std::max(1, cus) * 4 * 8;
    int qw = max_qw;
    for (int c : {1, 2, 4, 8})
        if (c < max_qw && rows / c <= slots) { qw = c; break; }
    const long qw_env = env_long("POINTOPS_BQ_QUERIES_PER_WAVE", 0);
    if (qw_env == 1 || qw_env == 2 || qw_env == 4 || qw_env == 8 || qw_env == 16) qw = (int)qw_env;
    return qw;
}

}  // namespace api
}  // namespace pointops

namespace {

using namespace pointops::api;

// ------------------------------------------------------------------ FPS geometry

struct FpsPlan {
    bool batch;  // certified-batch kernel (default) or one exchange per step
    int G;       // workgroups per cloud
    int ppt;     // points per thread
    int block;   // threads per workgroup
    int rg;      // candidates each workgroup publishes per exchange (batch, G > 1)
    int cpl;     // candidates per lane of the certifying wave (batch)
    bool group;  // slices grouped by position, folds culled per wave (batch)
    int err;     // POINTOPS_OK or why no plan fits
};


// One exchange per step. One workgroup per cloud avoids the cross-workgroup
// exchange and is fastest whenever the cloud fits in one workgroup (16 points
// per thread, its coordinates in LDS); larger clouds take about 4096 points
// per workgroup, at most 128 workgroups, more only if a slice would not fit.
FpsPlan fps_plan_step(int64_t B, int64_t N, const DeviceInfo& dev) {
    const int64_t cus = std::max(1, dev.cus);
    const int64_t max_slice = std::min<int64_t>(16 * 1024, ((int64_t)dev.lds_per_block - 1024) / 12);
    const long g_env = env_long("POINTOPS_FPS_WG_PER_CLOUD", 0);
    int64_t G;
    if (g_env > 0) {
        G = g_env;
    } else if (N <= max_slice) {
        G = 1;
    } else {
        G = std::min<int64_t>((N + 4095) / 4096, 128);
        G = std::max<int64_t>(G, (N + max_slice - 1) / max_slice);
        G = std::min<int64_t>(G, std::max<int64_t>(1, 4 * cus / std::max<int64_t>(B, 1)));
    }
    G = split_even(N, G);
    const int64_t slice = (N + G - 1) / G;
    FpsPlan p{};
    p.batch = false;
    p.G = (int)G;
    p.block = slice > 1024 ? 1024 : 256;
    p.ppt = (int)((slice + p.block - 1) / p.block);
    p.err = POINTOPS_OK;
    if (p.ppt > 16 || slice * 12 > (int64_t)dev.lds_per_block - 1024)
        p.err = fail(POINTOPS_UNSUPPORTED, "cloud of %lld points needs %d workgroups of %lld points",
                     (long long)N, p.G, (long long)slice);
    else if (B * p.G > cus * 8 && p.G > 1)
        p.err = fail(POINTOPS_UNSUPPORTED, "B*G = %lld workgroups exceed what runs at once",
                     (long long)(B * p.G));
    return p;
}

// Certified batches. About 1600 points per workgroup keeps the per-centre
// update short; at most 128 workgroups per cloud (more make the exchange of
// candidates slower than the update they save, measured on 100k points) up to
// kFpsWideMin points, and 256 from there on, each publishing two reports (512
// candidates, eight per lane of the certifying wave): at that size the update
// of a centre outweighs the longer certification (uniform clouds, 4096
// samples, 128 workgroups / 256: 400k points 1.62 / 1.56 ms, 786k 2.36 /
// 1.74 ms; 2^20 clustered points, 16384 samples, 9.07 / 6.10 ms; 200k points
// 1.42 / 1.60 ms). A cloud spanning several workgroups gets no more of them
// than the device holds at once (they wait on each other).
constexpr int64_t kFpsWideMin = 393216;

FpsPlan fps_plan_batch(int64_t B, int64_t N, const DeviceInfo& dev) {
    const int cus = std::max(1, dev.cus);
    const long g_env = env_long("POINTOPS_FPS_WG_PER_CLOUD", 0);
    const long block_env = env_long("POINTOPS_FPS_BLOCK", 0);
    int64_t want = g_env > 0          ? g_env
                   : N <= 2048        ? 1
                   : N >= kFpsWideMin ? 256
                                      : std::min<int64_t>((N + 1599) / 1600, 128);
    int block = block_env == 256 || block_env == 1024 ? (int)block_env : 0;
    FpsPlan p{};
    p.batch = true;
    for (int attempt = 0; attempt < 8; ++attempt) {
        const int64_t G = split_even(N, want);
        const int64_t slice = (N + G - 1) / G;
        p.G = (int)G;
        p.block = block ? block : (slice <= 768 ? 256 : 1024);
        const int npw = pointops::fps_batch_point_waves(p.block);
        p.ppt = pointops::fps_batch_ppt_round((int)((slice + npw * 64 - 1) / (npw * 64)));
        if (p.ppt < 0) {  // more than 16 points per thread
            if (p.block == 256) { block = 1024; continue; }
            if (g_env > 0) break;
            want = (N + 16 * 768 - 1) / (16 * 768);
            continue;
        }
        if (G == 1) {
            p.rg = npw;
            p.cpl = 1;
        } else {
            if (G > 256) break;
            p.rg = fps_batch_rg(G, npw);
            const int64_t cand = G * p.rg;
            p.cpl = cand <= 64 ? 1 : cand <= 128 ? 2 : cand <= 256 ? 4 : 8;
            if (p.block == 256 && p.cpl > 1) { block = 1024; continue; }
        }
        // Grouped slices where a centre's fold outweighs its certification
        // (four or more points per thread); POINTOPS_FPS_GROUP = 0 / 1 turns
        // the grouping off, or on wherever it is built.
        const long group_env = env_long("POINTOPS_FPS_GROUP", -1);
        p.group = G > 1 && slice <= pointops::kFpsGroupMaxSlice &&
                  pointops::fps_batch_group_built(p.ppt, p.block) &&
                  (group_env == 1 || (group_env != 0 && p.ppt >= 4));
        int cap = 0;
        hipError_t e = pointops::fps_batch_capacity(p.ppt, p.block, p.cpl,
                                                    pointops::fps_batch_lds_bytes(p.G, p.rg),
                                                    p.group, cus, &cap);
        if (e != hipSuccess) { p.err = hip_fail(e, "fps occupancy query"); return p; }
        if (G == 1 || B * G <= cap) {
            p.err = POINTOPS_OK;
            return p;
        }
        if (g_env > 0) break;
        want = std::max<int64_t>(1, cap / std::max<int64_t>(B, 1));
    }
    p.err = fail(POINTOPS_UNSUPPORTED, "no FPS launch shape fits B=%lld N=%lld", (long long)B,
                 (long long)N);
    return p;
}

// The step kernel wins on clouds of up to kFpsStepMaxPoints (one workgroup, no
// exchange at all, and certified batches there are only a few steps long);
// the batched kernel beyond (measured: 32 clouds of 4096 points, 512 samples:
// 0.32 ms stepping, 0.36 ms batched; of 8192 points: 0.42 / 0.34 ms; of 16384,
// 1024 samples: 1.83 / 0.55 ms).
FpsPlan fps_plan(int64_t B, int64_t N, const DeviceInfo& dev) {
    const char* mode = getenv("POINTOPS_FPS_MODE");
    if (mode && strcmp(mode, "step") == 0) return fps_plan_step(B, N, dev);
    if (mode && strcmp(mode, "batch") == 0) return fps_plan_batch(B, N, dev);
    const FpsPlan step = fps_plan_step(B, N, dev);
    if (step.err == POINTOPS_OK && step.G == 1 && N <= kFpsStepMaxPoints) return step;
    g_err[0] = 0;
    return fps_plan_batch(B, N, dev);
}

// The part of the workspace that every call clears (status and exchange words).
size_t plan_clear_bytes(int64_t B, const FpsPlan& p) {
    return p.batch ? pointops::fps_batch_workspace_bytes(B, p.G, p.rg)
                   : pointops::fps_workspace_bytes(B, p.G);
}

size_t plan_workspace_bytes(int64_t B, int64_t N, const FpsPlan& p) {
    if (p.batch && p.group)
        return pointops::fps_batch_group_offset(B, p.G, p.rg) +
               pointops::fps_batch_group_bytes(B, N);
    return plan_clear_bytes(B, p);
}

// The static scratch of pointops_fps_noalloc: FPS's workspace (status word,
// exchange words) for callers that cannot allocate device memory. Each GPU
// holds its own copy for the life of the process; its device address comes
// from hipGetSymbolAddress once per device (the array's name is only a host
// stand-in), and only that address is ever passed to a kernel or a fill.
constexpr size_t kFpsScratchBytes = (size_t)1 << 20;
static __device__ __align__(256) uint8_t scratch[kFpsScratchBytes];
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `device`'s scratch (the device is current), after
// checking that `need` bytes fit. POINTOPS_FPS_SCRATCH_LIMIT lowers the limit
// (so a test can reach the refusal); it never raises it.
int static_scratch(int device, size_t need, void** out) {
    size_t limit = kFpsScratchBytes;
    const long env = env_long("POINTOPS_FPS_SCRATCH_LIMIT", 0);
    if (env > 0 && (size_t)env < limit) limit = (size_t)env;
    if (need > limit)
        return fail(POINTOPS_UNSUPPORTED,
                    "this FPS needs %zu bytes of scratch; the static scratch holds %zu "
                    "(use pointops_fps with a workspace)",
                    need, limit);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[device]) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(POINTOPS_HIP_ERROR, "hipGetSymbolAddress(scratch) gave NULL");
        g_scratch[device] = p;
    }
    *out = g_scratch[device];
    return POINTOPS_OK;
}

}  // namespace

using namespace pointops::api;

extern "C" {

int pointops_abi_version(void) { return 5; }

const char* pointops_status_string(int status) {
    switch (status) {
        case POINTOPS_OK: return "ok";
        case POINTOPS_INVALID_ARGUMENT: return "invalid argument";
        case POINTOPS_UNSUPPORTED: return "unsupported (beyond a compiled limit)";
        case POINTOPS_UNSUPPORTED_DEVICE: return "unsupported device (needs gfx950, wave64)";
        case POINTOPS_HIP_ERROR: return "HIP runtime error";
        case POINTOPS_EXEC_TIMEOUT: return "FPS gave up a bounded wait (workgroups not co-resident)";
        default: return "unknown status";
    }
}

const char* pointops_last_error(void) { return g_err; }

int pointops_device_check(int device) {
    g_err[0] = 0;
    return check_device(device, nullptr);
}

size_t pointops_fps_workspace_bytes(int64_t B, int64_t N, int64_t M) {
    if (B <= 0 || N <= 0 || M <= 0) return 0;
    DeviceInfo* dev = nullptr;
    DeviceInfo fallback;
    fallback.cus = 256;
    if (current_device(&dev) != POINTOPS_OK) dev = &fallback;
    const FpsPlan p = fps_plan(B, N, *dev);
    g_err[0] = 0;
    return p.err == POINTOPS_OK ? plan_workspace_bytes(B, N, p) : 0;
}

}  // extern "C"

namespace {

// Shared by pointops_fps and pointops_fps_noalloc: validation, plan and launch
// on `ws` (a workspace of ws_bytes bytes, or the static scratch when
// ws_limit is set: then the plan's need is checked against that limit).
int fps_run(const float* xyz, int64_t B, int64_t N, int64_t M, int64_t start_idx,
            int64_t* out_idx, float* out_xyz, void* ws, size_t ws_bytes, bool scratch,
            void* stream) {
    g_err[0] = 0;
    if (B < 0 || N < 0 || M < 0) return fail(POINTOPS_INVALID_ARGUMENT, "negative size");
    if (B == 0 || M == 0) return POINTOPS_OK;
    if (N == 0) return fail(POINTOPS_INVALID_ARGUMENT, "N == 0 with M >= 1");
    if (start_idx < 0 || start_idx >= N)
        return fail(POINTOPS_INVALID_ARGUMENT, "start_idx %lld not in [0, %lld)",
                    (long long)start_idx, (long long)N);
    if (N >= kMaxPoints || M >= kMaxPoints)
        return fail(POINTOPS_UNSUPPORTED, "N and M must be below 2^31");
    if (!xyz || !out_idx) return fail(POINTOPS_INVALID_ARGUMENT, "null pointer");
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    DeviceInfo* dev = nullptr;
    int st = check_device(device, &dev);
    if (st != POINTOPS_OK) return st;
    FpsPlan p = fps_plan(B, N, *dev);
    if (p.err != POINTOPS_OK) return p.err;
    if (scratch) p.group = false;  // the static scratch holds the exchange words only
    const size_t need = plan_workspace_bytes(B, N, p);
    if (scratch) {
        st = static_scratch(device, need, &ws);
        if (st != POINTOPS_OK) return st;
    } else if (!ws || ws_bytes < need) {
        return fail(POINTOPS_INVALID_ARGUMENT, "workspace of %zu bytes given, %zu needed",
                    ws_bytes, need);
    }
    hipStream_t s = (hipStream_t)stream;
    e = pointops::launch_fps_clear(ws, plan_clear_bytes(B, p), s);
    if (e != hipSuccess) return hip_fail(e, "fps workspace clear");
    const uint32_t spin = (uint32_t)env_long("POINTOPS_FPS_SPIN_LIMIT", 1L << 22);
    if (p.batch)
        e = pointops::launch_fps_batch(xyz, B, N, M, start_idx, out_idx, out_xyz, ws, p.G,
                                       p.ppt, p.block, p.rg, p.cpl, p.group, spin, s, nullptr, 0, 0,
                                       nullptr, 0);
    else
        e = pointops::launch_fps(xyz, B, N, M, start_idx, out_idx, out_xyz, ws, p.G, p.ppt,
                                 p.block, spin, s, nullptr, 0, 0);
    if (e != hipSuccess) return hip_fail(e, "fps launch");
    return POINTOPS_OK;
}

}  // namespace

extern "C" {

int pointops_fps(const float* xyz, int64_t B, int64_t N, int64_t M, int64_t start_idx,
                 int64_t* out_idx, float* out_xyz, void* workspace, size_t workspace_bytes,
                 void* stream) {
    return fps_run(xyz, B, N, M, start_idx, out_idx, out_xyz, workspace, workspace_bytes, false,
                   stream);
}

int pointops_fps_noalloc(const float* xyz, int64_t B, int64_t N, int64_t M, int64_t start_idx,
                         int64_t* out_idx, float* out_xyz, void* stream) {
    return fps_run(xyz, B, N, M, start_idx, out_idx, out_xyz, nullptr, 0, true, stream);
}

int pointops_fps_status(const void* workspace, size_t workspace_bytes, int64_t* exchanges,
                        void* stream) {
    g_err[0] = 0;
    if (!workspace || workspace_bytes < 2 * sizeof(uint32_t))
        return fail(POINTOPS_INVALID_ARGUMENT, "FPS status needs the call's workspace");
    // the copy is ordered after the FPS launch on `stream`; the synchronize
    // waits for both (pageable host memory: no registration involved)
    hipStream_t s = (hipStream_t)stream;
    uint32_t words[2] = {0, 0};  // status, exchanges of the first cloud
    hipError_t e = hipMemcpyAsync(words, workspace, sizeof words, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "fps status: read status word");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "fps status: stream synchronize");
    if (exchanges) *exchanges = (int64_t)words[1];
    if (words[0] != 0)
        return fail(POINTOPS_EXEC_TIMEOUT,
                    "FPS gave up waiting for a workgroup of its cloud (status word %u); output "
                    "slots from that step on hold -1",
                    words[0]);
    return POINTOPS_OK;
}

size_t pointops_knn_workspace_bytes(int64_t B, int64_t Q, int64_t P) {
    if (B <= 0 || Q <= 0 || P <= 0 || !knn_use_grid(B, Q, P)) return 0;
    return pointops::knn_grid_workspace_bytes(B, Q, P);
}

int pointops_knn_search(int64_t B, int64_t Q, int64_t P, int64_t k, int with_workspace) {
    g_err[0] = 0;
    if (B < 0 || Q < 0 || P < 0 || k < 1 || k > P || k > POINTOPS_KNN_KMAX)
        return -fail(POINTOPS_INVALID_ARGUMENT, "no kNN search for this shape");
    DeviceInfo* dev = nullptr;
    const int st = current_device(&dev);
    if (st != POINTOPS_OK) return -st;
    if (with_workspace && knn_use_grid(B, Q, P) && knn_grid_pays(k, B, Q, P))
        return POINTOPS_KNN_SEARCH_GRID;
    return knn_wave_plan(k, B * Q, P, dev->cus).nw ? POINTOPS_KNN_SEARCH_WAVES
                                                   : POINTOPS_KNN_SEARCH_LANES;
}

int pointops_knn(const float* query, const float* ref, int64_t B, int64_t Q, int64_t P,
                 int64_t k, float* out_dist, int64_t* out_idx, void* workspace,
                 size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    if (B < 0 || Q < 0 || P < 0) return fail(POINTOPS_INVALID_ARGUMENT, "negative size");
    if (k < 1 || k > P)
        return fail(POINTOPS_INVALID_ARGUMENT, "k = %lld must satisfy 1 <= k <= P = %lld",
                    (long long)k, (long long)P);
    if (k > POINTOPS_KNN_KMAX)
        return fail(POINTOPS_UNSUPPORTED, "k = %lld exceeds POINTOPS_KNN_KMAX = %d",
                    (long long)k, POINTOPS_KNN_KMAX);
    if (B == 0 || Q == 0) return POINTOPS_OK;
    if (Q >= kMaxPoints || P >= kMaxPoints) return fail(POINTOPS_UNSUPPORTED, "sizes >= 2^31");
    if (B > kMaxGridY) return fail(POINTOPS_UNSUPPORTED, "B > %lld", (long long)kMaxGridY);
    if (!query || !ref || !out_dist || !out_idx)
        return fail(POINTOPS_INVALID_ARGUMENT, "null pointer");
    DeviceInfo* dev = nullptr;
    int st = current_device(&dev);
    if (st != POINTOPS_OK) return st;
    int kcap = 1;
    while (kcap < k) kcap *= 2;
    if (workspace && knn_use_grid(B, Q, P)) {
        const size_t need = pointops::knn_grid_workspace_bytes(B, Q, P);
        if (workspace_bytes < need)
            return fail(POINTOPS_INVALID_ARGUMENT, "workspace of %zu bytes given, %zu needed",
                        workspace_bytes, need);
    }
    if (workspace && knn_use_grid(B, Q, P) && knn_grid_pays(k, B, Q, P)) {
        hipError_t e = pointops::launch_knn_grid(query, ref, B, Q, P, k, out_dist, out_idx, kcap,
                                                 knn_grid_nw(k, kcap, B * Q, B * P), workspace,
                                                 0, nullptr, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "knn launch");
        return POINTOPS_OK;
    }
    const KnnWavePlan wp = knn_wave_plan(k, B * Q, P, dev->cus);
    if (wp.nw) {
        hipError_t e = pointops::launch_knn_wave(query, ref, B, Q, P, k, out_dist, out_idx, wp.nw,
                                                 wp.qw, nullptr, 0, 0, 0, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "knn launch");
        return POINTOPS_OK;
    }
    const int64_t tiles = B * ((Q + 63) / 64);
    hipError_t e = pointops::launch_knn(query, ref, B, Q, P, k, out_dist, out_idx, kcap,
                                        knn_waves(kcap, tiles, dev->cus), nullptr, 0, 0, 0,
                                        (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "knn launch");
    return POINTOPS_OK;
}

size_t pointops_ball_query_workspace_bytes(int64_t B, int64_t Q, int64_t P) {
    if (B <= 0 || Q <= 0 || P <= 0) return 0;
    return bq_grid_possible(P) ? pointops::ball_query_grid_bytes(B, Q, P)
                               : pointops::ball_query_box_bytes(B, P);
}

int pointops_ball_query_search(int64_t B, int64_t Q, int64_t P, int64_t K, int with_workspace) {
    g_err[0] = 0;
    if (B < 0 || Q < 0 || P < 0 || K < 1)
        return -fail(POINTOPS_INVALID_ARGUMENT, "no Ball Query for this shape");
    if (!with_workspace || P == 0) return POINTOPS_BQ_SEARCH_SCAN;
    return bq_grid_possible(P) && K <= 32 ? POINTOPS_BQ_SEARCH_GRID : POINTOPS_BQ_SEARCH_CULLED;
}

int pointops_ball_query(const float* query, const float* ref, int64_t B, int64_t Q, int64_t P,
                        float radius, int64_t K, float* out_dist2, int64_t* out_idx,
                        void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    if (B < 0 || Q < 0 || P < 0) return fail(POINTOPS_INVALID_ARGUMENT, "negative size");
    if (!(radius > 0.0f) || std::isinf(radius))
        return fail(POINTOPS_INVALID_ARGUMENT, "radius must be finite and > 0");
    if (K < 1) return fail(POINTOPS_INVALID_ARGUMENT, "K must be >= 1");
    if (B == 0 || Q == 0) return POINTOPS_OK;
    if (Q >= kMaxPoints || P >= kMaxPoints || K >= kMaxPoints)
        return fail(POINTOPS_UNSUPPORTED, "sizes >= 2^31");
    if (B > kMaxGridY) return fail(POINTOPS_UNSUPPORTED, "B > %lld", (long long)kMaxGridY);
    if (!query || (!ref && P > 0) || !out_dist2 || !out_idx)
        return fail(POINTOPS_INVALID_ARGUMENT, "null pointer");
    DeviceInfo* dev = nullptr;
    int st = current_device(&dev);
    if (st != POINTOPS_OK) return st;
    // R2 = fl32(r32 * r32), the project page's dense threshold.
    volatile float r32 = radius;
    const float r2 = r32 * r32;
    const int qw = bq_queries_per_wave(B * Q, dev->cus, 8);
    const size_t need = pointops_ball_query_workspace_bytes(B, Q, P);
    if (workspace && workspace_bytes < need)
        return fail(POINTOPS_INVALID_ARGUMENT, "workspace of %zu bytes given, %zu needed",
                    workspace_bytes, need);
    hipError_t e;
    if (workspace && P > 0 && bq_grid_possible(P) && K <= 32)
        e = pointops::launch_ball_query_grid(query, ref, B, Q, P, r2, K, out_dist2, out_idx, qw,
                                             bq_scan_budget(), bq_grid_level(P), workspace,
                                             (hipStream_t)stream);
    else if (workspace && P > 0)  // the boxes come first in either layout
        e = pointops::launch_ball_query_culled(query, ref, B, Q, P, r2, K, out_dist2, out_idx,
                                               qw, (float*)workspace, -1, nullptr, nullptr,
                                               (hipStream_t)stream);
    else
        e = pointops::launch_ball_query(query, ref, B, Q, P, r2, K, out_dist2, out_idx, qw,
                                        nullptr, 0, 0, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ball_query launch");
    return POINTOPS_OK;
}

}  // extern "C"

extern "C" size_t pointops_ball_query_backward_workspace_bytes(int64_t B, int64_t Q, int64_t P,
                                                              int64_t K) {
    if (B <= 0 || Q <= 0 || K < 1 || Q != P) return 0;
    return pointops::bq_backward_workspace_bytes(B, Q, K);
}

extern "C" int pointops_ball_query_backward(const float* query, const float* ref,
                                            const int64_t* idx, const float* grad_dist2,
                                            int64_t B, int64_t Q, int64_t P, int64_t K,
                                            float* grad_query, float* grad_ref, void* workspace,
                                            size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    if (B < 0 || Q < 0 || P < 0) return fail(POINTOPS_INVALID_ARGUMENT, "negative size");
    if (K < 1) return fail(POINTOPS_INVALID_ARGUMENT, "K must be >= 1");
    if (Q >= kMaxPoints || P >= kMaxPoints || K >= kMaxPoints)
        return fail(POINTOPS_UNSUPPORTED, "sizes >= 2^31");
    if (B > 0 && Q > (int64_t)INT32_MAX * 4 / B)
        return fail(POINTOPS_UNSUPPORTED, "B * Q above 2^33 rows");
    if (!grad_query && !grad_ref) return POINTOPS_OK;
    const bool rows = B > 0 && Q > 0;
    if ((rows && (!query || !idx || !grad_dist2 || (!ref && P > 0))) ||
        (grad_ref && B * P > 0 && !ref))
        return fail(POINTOPS_INVALID_ARGUMENT, "null pointer");
    // the workspace serves only a cloud queried by its own points
    const bool self = rows && query == ref && Q == P;
    if (workspace && self) {
        const size_t need = pointops::bq_backward_workspace_bytes(B, Q, K);
        if (workspace_bytes < need)
            return fail(POINTOPS_INVALID_ARGUMENT, "workspace of %zu bytes given, %zu needed",
                        workspace_bytes, need);
    }
    int st = current_device(nullptr);
    if (st != POINTOPS_OK) return st;
    hipError_t e = pointops::launch_ball_query_backward(
        query, ref, idx, grad_dist2, rows ? B : 0, rows ? Q : 0, P, K, grad_query, grad_ref,
        self ? workspace : nullptr, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ball_query_backward launch");
    return POINTOPS_OK;
}
