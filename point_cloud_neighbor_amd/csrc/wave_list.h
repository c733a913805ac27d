// A wave's sorted list of its 32 (or 16) smallest 64-bit keys, fed with
// candidates in batches of 32 (or 48) and merged by a bitonic network of lane
// moves: used by the
// one-query-per-wave kNN scan and grid search (keys (bits(s) << 32) | index)
// and the Ball Query grid pass (keys (index << 32) | bits(s)).
//
// Lanes 0..31 hold the list, ascending. Candidates go, in ballot order, to a
// 32-entry buffer of the query in LDS; when it fills (and at the end) lanes
// 32..63 load it and a bitonic network in the mirror formulation (every
// compare-exchange keeps the smaller key in the lower lane) sorts lanes 32..63
// and then merges the two sorted halves: 21 steps, each two lane moves (DPP
// inside rows, ds_swizzle or ds_bpermute across them), one 64-bit compare and
// two selects. The bound for new candidates is the high word of lane k-1's key:
// callers offer a candidate only when its high word is strictly below it
// (each caller states why that is exact for its keys).
#pragma once

#include "common.h"

namespace pointops {

constexpr int kKwBuf = 32;               // candidate buffer entries per wave
constexpr uint64_t kKwEmpty = ~0ull;     // an empty list slot (sorts last)

// Lanes of a wave whose lane-index bit D is clear: the lower lane of every
// pair a step at distance D (or a mirror step of half-size D) compares.
template <int D>
constexpr uint64_t kw_lower_lanes() {
    uint64_t m = 0;
    for (int l = 0; l < kWave; ++l)
        if (!(l & D)) m |= 1ull << l;
    return m;
}

__device__ __forceinline__ uint64_t kw_join(uint32_t lo, uint32_t hi) {
    return ((uint64_t)hi << 32) | lo;
}

// Partner values. DPP: quad_perm (xor 1, xor 2, mirror of 4), row_half_mirror
// (mirror of 8), row_mirror (mirror of 16), row_ror:8 (xor 8); ds_swizzle in
// bit-mask mode (xor 4, xor 16, mirror of 32); ds_bpermute (mirror of 64).
// Every lane of these permutations reads a lane of its own row, so no lane
// keeps an old value and none needs initialising.
template <int CTRL>
__device__ __forceinline__ uint64_t kw_dpp(uint64_t v) {
    return kw_join((uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false),
                   (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF,
                                                      false));
}
template <int XOR>
__device__ __forceinline__ uint64_t kw_swizzle(uint64_t v) {
    constexpr int pattern = (XOR << 10) | 0x1F;  // and 31, or 0, xor XOR
    return kw_join((uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)v, pattern),
                   (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)(v >> 32), pattern));
}
__device__ __forceinline__ uint64_t kw_mirror64(uint64_t v, int lane) {
    const int addr = (63 - lane) * 4;
    return kw_join((uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)v),
                   (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)(v >> 32)));
}

// One compare-exchange step: lanes in LOWER keep min(v, p), the others
// max(v, p). Equal keys are only empty slots, for which either choice is the
// same.
template <uint64_t LOWER>
__device__ __forceinline__ uint64_t kw_ce(uint64_t v, uint64_t p) {
    const uint64_t lt = ballot(p < v);
    return __builtin_amdgcn_inverse_ballot_w64(~(lt ^ LOWER)) ? p : v;
}

constexpr int kDppQuadMirror = 0x1B;  // quad_perm [3,2,1,0]
constexpr int kDppRowRor8 = 0x128;    // row_ror:8 = xor 8 inside a row

// Sorts each 32-lane half ascending (the lower half, already sorted, passes
// through unchanged), then merges the halves: lanes 0..31 end up holding the
// 32 smallest keys of the wave, ascending.
__device__ __forceinline__ uint64_t kw_sort_merge(uint64_t v, int lane) {
    // blocks of 2
    v = kw_ce<kw_lower_lanes<1>()>(v, kw_dpp<kDppQuadSwap1>(v));
    // blocks of 4
    v = kw_ce<kw_lower_lanes<2>()>(v, kw_dpp<kDppQuadMirror>(v));
    v = kw_ce<kw_lower_lanes<1>()>(v, kw_dpp<kDppQuadSwap1>(v));
    // blocks of 8
    v = kw_ce<kw_lower_lanes<4>()>(v, kw_dpp<kDppRowHalfMirror>(v));
    v = kw_ce<kw_lower_lanes<2>()>(v, kw_dpp<kDppQuadSwap2>(v));
    v = kw_ce<kw_lower_lanes<1>()>(v, kw_dpp<kDppQuadSwap1>(v));
    // blocks of 16
    v = kw_ce<kw_lower_lanes<8>()>(v, kw_dpp<kDppRowMirror>(v));
    v = kw_ce<kw_lower_lanes<4>()>(v, kw_swizzle<4>(v));
    v = kw_ce<kw_lower_lanes<2>()>(v, kw_dpp<kDppQuadSwap2>(v));
    v = kw_ce<kw_lower_lanes<1>()>(v, kw_dpp<kDppQuadSwap1>(v));
    // blocks of 32
    v = kw_ce<kw_lower_lanes<16>()>(v, kw_swizzle<31>(v));
    v = kw_ce<kw_lower_lanes<8>()>(v, kw_dpp<kDppRowRor8>(v));
    v = kw_ce<kw_lower_lanes<4>()>(v, kw_swizzle<4>(v));
    v = kw_ce<kw_lower_lanes<2>()>(v, kw_dpp<kDppQuadSwap2>(v));
    v = kw_ce<kw_lower_lanes<1>()>(v, kw_dpp<kDppQuadSwap1>(v));
    // merge the halves: the mirror step leaves the 32 smallest keys, bitonic,
    // in lanes 0..31; the rest sorts them
    v = kw_ce<kw_lower_lanes<32>()>(v, kw_mirror64(v, lane));
    v = kw_ce<kw_lower_lanes<16>()>(v, kw_swizzle<16>(v));
    v = kw_ce<kw_lower_lanes<8>()>(v, kw_dpp<kDppRowRor8>(v));
    v = kw_ce<kw_lower_lanes<4>()>(v, kw_swizzle<4>(v));
    v = kw_ce<kw_lower_lanes<2>()>(v, kw_dpp<kDppQuadSwap2>(v));
    v = kw_ce<kw_lower_lanes<1>()>(v, kw_dpp<kDppQuadSwap1>(v));
    return v;
}

// The running answer of one query: its best keys (lanes 0..31, ascending), the
// candidate bound (high word of lane k-1's key), the candidates buffered in
// LDS and their count (wave-uniform).
struct KwQuery {
    uint64_t list;
    uint32_t bound;
    int cnt;
    uint64_t* buf;
};

// Merges the buffered candidates into the list. L is the number of list lanes
// kept (32, or 16 when k <= 16); the buffer holds cnt <= 64 - L candidates,
// which lanes L..63 load. The network sorts all 64 keys, so lanes 0..L-1 end
// up holding the L smallest, ascending.
template <int L = kKwBuf>
__device__ __forceinline__ void kw_merge(KwQuery& st, int lane, int k) {
    static_assert(L == 16 || L == 32, "list lanes");
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int e = lane - L;
    uint64_t v = st.list;
    if (e >= 0) v = e < st.cnt ? st.buf[e] : kKwEmpty;  // e < 64 - L: in bounds
    st.list = kw_sort_merge(v, lane);
    st.bound = lane_value((uint32_t)(st.list >> 32), k - 1);
    st.cnt = 0;
    // the next candidates overwrite the buffer only after this wave's loads
    // of it (LDS executes a wave's operations in order)
    __builtin_amdgcn_wave_barrier();
}

// Appends this lane's candidate key (u << 32) | j if `cand`; merges whenever
// the buffer fills and re-tests what did not fit against the new bound
// (u < bound; with INCL u <= bound, for callers that visit keys out of the
// order of their low words, where a key with the bound's high word can still
// enter by a smaller low word).
template <bool INCL = false, int L = kKwBuf>
__device__ __forceinline__ void kw_offer(KwQuery& st, bool cand, uint32_t u, int j, int lane,
                                         int k) {
    constexpr int CAP = kWave - L;  // buffer entries
    uint64_t m = ballot(cand);
    while (m) {
        const int pos = st.cnt + (int)lanes_below(m);
        if (cand && pos < CAP) st.buf[pos] = ((uint64_t)u << 32) | (uint32_t)j;
        st.cnt += (int)__builtin_popcountll(m);
        if (st.cnt < CAP) break;
        st.cnt = CAP;
        kw_merge<L>(st, lane, k);
        cand = cand && pos >= CAP && (INCL ? u <= st.bound : u < st.bound);
        m = ballot(cand);
    }
}

}  // namespace pointops
