// Device helpers shared by the pointops kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

// Every translation unit is also built with -ffp-contract=off; the pragma makes
// the rule local to the code that needs it.
#pragma clang fp contract(off)

namespace pointops {

constexpr int kWave = 64;

// Squared distance in the fixed float32 order ((dx*dx + dy*dy) + dz*dz),
// dx = fl32(q.x - x.x): the project page, "The operators in equations" (the
// sum over three coordinates) and "How the kernels work" (that order, no FMA).
// fl32(a - b) = -fl32(b - a) under round-to-nearest-even, so the direction of
// the differences does not change the result.
__device__ __forceinline__ float s32(float qx, float qy, float qz, float x, float y, float z) {
    float dx = qx - x;
    float dy = qy - y;
    float dz = qz - z;
    float sx = dx * dx;
    float sy = dy * dy;
    float sz = dz * dz;
    float sxy = sx + sy;
    return sxy + sz;
}

__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

// Wave-uniform 64-bit predicate mask of the active lanes (bit l = lane l).
__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Lane 0's value of a 32-bit integer (a float would be converted: pass its bits).
template <typename T> __device__ __forceinline__ T uniform(T v) {
    static_assert(std::is_integral<T>::value && sizeof(T) == 4, "32-bit integers only");
    return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Maximum of a 32-bit value over the 64 lanes of a wave, returned wave-uniform.
__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, kWave));
    return __builtin_amdgcn_readfirstlane(v);
}

// DPP lane movement (gfx9 encodings): quad_perm, row mirrors, row broadcasts.
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t src) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, ROW_MASK, 0xF, false);
}

// Maximum of an unsigned 32-bit value over the 64 lanes of a wave, returned
// wave-uniform. Lanes exchange through DPP (no LDS traffic): butterflies inside
// each row of 16 lanes, then row broadcasts carry rows 0-1 and 0-2 into the
// last row, whose lane 63 holds the maximum.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    // 0 (the identity of max) stands in for lanes a row mask leaves out, which
    // also lets the compiler fold each lane move into the max instruction
    v = max(v, dpp_u32<kDppQuadSwap1>(0u, v));
    v = max(v, dpp_u32<kDppQuadSwap2>(0u, v));
    v = max(v, dpp_u32<kDppRowHalfMirror>(0u, v));
    v = max(v, dpp_u32<kDppRowMirror>(0u, v));
    v = max(v, dpp_u32<kDppRowBcast15, 0xA>(0u, v));
    v = max(v, dpp_u32<kDppRowBcast31, 0xC>(0u, v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Value of `v` in lane `l` (l wave-uniform).
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int l) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Lane-wise maximum of an unsigned 64-bit key over the 64 lanes of a wave;
// every lane gets the result.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
        uint32_t olo = __shfl_xor(lo, off, kWave);
        uint32_t ohi = __shfl_xor(hi, off, kWave);
        uint64_t o = ((uint64_t)ohi << 32) | olo;
        v = o > v ? o : v;
    }
    return v;
}

}  // namespace pointops
