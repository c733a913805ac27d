// Uniform-grid helpers shared by the kNN grid search and the Ball Query grid
// pass: the cell mapping, the sorted copies and boxes the build writes, the
// box lower bound of s32 and a sorted list of 64-bit keys.
//
// Build (knn_grid.hip): per cloud, the references' bounding box, a uniform grid
// of 2^L cells per axis over it, counting-sorted copies (x, y, z, original
// index) of references and queries in Morton order of their cells, a box for
// every kGridBlk consecutive sorted references and one for every 64 blocks
// (each with the range of its references' original indices). The cell formula
// only decides the order: no result depends on it.
#pragma once

#include "common.h"

namespace pointops {

constexpr int kGridBlk = 16;  // sorted references per block (per box)

struct GridParams {
    float lo[3];
    float inv[3];  // cells per unit length
    float pad[2];
};

__device__ __forceinline__ uint32_t spread3(uint32_t v) {
    // bit b of v -> bit 3b
    v &= 0x3FF;
    v = (v | (v << 16)) & 0x030000FF;
    v = (v | (v << 8)) & 0x0300F00F;
    v = (v | (v << 4)) & 0x030C30C3;
    v = (v | (v << 2)) & 0x09249249;
    return v;
}

__device__ __forceinline__ uint32_t cell_code(const GridParams& g, float x, float y, float z,
                                              int L) {
    // clamped in float first, so points outside the box (queries) convert safely
    const float top = (float)((1 << L) - 1);
    const int cx = (int)fminf(fmaxf((x - g.lo[0]) * g.inv[0], 0.0f), top);
    const int cy = (int)fminf(fmaxf((y - g.lo[1]) * g.inv[1], 0.0f), top);
    const int cz = (int)fminf(fmaxf((z - g.lo[2]) * g.inv[2], 0.0f), top);
    return spread3((uint32_t)cx) | (spread3((uint32_t)cy) << 1) | (spread3((uint32_t)cz) << 2);
}

template <int KCAP>
struct TopK64 {
    uint64_t key[KCAP];  // ascending; front sentinels 0, empty slots ~0

    __device__ __forceinline__ void init(int k) {
#pragma unroll
        for (int p = 0; p < KCAP; ++p) key[p] = p < KCAP - k ? 0ull : ~0ull;
    }

    // True if kk is already in the list.
    __device__ __forceinline__ bool contains(uint64_t kk) const {
        bool f = false;
#pragma unroll
        for (int p = 0; p < KCAP; ++p) f |= key[p] == kk;
        return f;
    }

    // Insert kk (~0 inserts nothing); the largest key drops out.
    __device__ __forceinline__ void insert(uint64_t kk) {
#pragma unroll
        for (int p = KCAP - 1; p >= 1; --p) {
            const uint64_t hi = key[p - 1] > kk ? key[p - 1] : kk;
            key[p] = hi < key[p] ? hi : key[p];
        }
        key[0] = kk < key[0] ? kk : key[0];
    }

    __device__ __forceinline__ uint32_t last_hi() const { return (uint32_t)(key[KCAP - 1] >> 32); }
};

// Lower bound of s32 between a point and a box (see the file comment).
__device__ __forceinline__ float box_bound(const float* __restrict__ o, float qx, float qy,
                                           float qz) {
    const float gx = fmaxf(fmaxf(o[0] - qx, qx - o[3]), 0.0f);
    const float gy = fmaxf(fmaxf(o[1] - qy, qy - o[4]), 0.0f);
    const float gz = fmaxf(fmaxf(o[2] - qz, qz - o[5]), 0.0f);
    return (gx * gx + gy * gy) + gz * gz;
}

// Ragged batches: the build and the kNN search can take a table of kGcWords
// words per cloud in device memory. Cloud b's references are then rows
// [ROff, ROff + RCnt) of the reference buffer and its queries rows
// [QOff, QOff + QCnt) of the query buffer; its sorted copies keep the slots
// [b * P, b * P + RCnt) and [b * Q, b * Q + QCnt), P and Q being the largest
// counts of the batch. The search writes a query's row QOff + its index in
// the cloud and reports reference indices IdxBase + index in the cloud.
enum GridCloud { kGcROff = 0, kGcRCnt, kGcQOff, kGcQCnt, kGcIdxBase };
constexpr int kGcWords = 8;

// The build's outputs inside its workspace.
struct GridView {
    GridParams* gp;      // per cloud
    uint32_t* ref_start; // per cloud and cell: first sorted reference
    float4* sref;        // (B, P) sorted references (x, y, z, original index bits)
    float4* squery;      // (B, Q) sorted queries
    float* box;          // (B, nblk) x 8: min x, y, z, max x, y, z of each block, then
                         // its smallest and largest original index (int32 bits)
    float* sbox;         // (B, nsb) x 8: the same for every 64 blocks
    int L, nblk, nsb;
};

// Cells per axis 2^L, 2 <= L <= 7: the kNN grid search's choice for P
// references per cloud.
int knn_grid_level(int64_t P);
size_t grid_workspace_bytes(int64_t B, int64_t Q, int64_t P, int L);
// Builds the grid (2^L cells per axis) of B clouds of P references and Q
// queries into `workspace` (grid_workspace_bytes(B, Q, P, L) bytes). With
// `gate` non-null every build kernel reads *gate first and does nothing when
// it is 0 (the caller decides on the device whether the grid is needed).
// With `clouds` non-null (a ragged batch, see GridCloud) P and Q are the
// largest counts and every cloud takes its points from its table record.
hipError_t launch_grid_build(const float* query, const float* ref, int64_t B, int64_t Q,
                             int64_t P, int L, void* workspace, const uint32_t* gate,
                             const int64_t* clouds, hipStream_t stream, GridView* view);

}  // namespace pointops
