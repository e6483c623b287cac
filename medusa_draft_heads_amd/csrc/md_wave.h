// Wave-wide max and argmax without LDS traffic.
//
// A lane exchange through __shfl_xor becomes ds_bpermute, an LDS-routed
// instruction whose latency (on the order of a hundred cycles) every level
// of a reduction waits for. Here the levels are DPP moves inside rows of 16
// lanes (quad permutes for lanes 1 and 2 apart, the half-row and row
// mirrors) and gfx950's row swaps (v_permlane16_swap, v_permlane32_swap)
// across rows, all register-to-register. Each level pairs every lane with
// exactly one partner, so after the six levels all 64 lanes hold the result.
// Max and argmax are exact, so the pairing order does not change any bit.
#pragma once

#include <hip/hip_runtime.h>

namespace md_wave {

// Immediate of s_waitcnt that waits until at most n vector-memory operations
// of this wave are outstanding and leaves the other counters alone (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7: no wait), lgkmcnt
// 11:8 (15: no wait)). The staged pipelines compute n from the same constants
// their issue loops use, so a change to the number of loads a stage issues
// changes the wait with it; the build rejects scratch use (spills are vector
// memory operations too) in the kernels that rely on it.
constexpr unsigned waitcnt_vm(int n) {
    return (unsigned)(n & 15) | ((unsigned)(n >> 4) << 14) | (0x7u << 4) | (0xFu << 8);
}
static_assert(waitcnt_vm(0) == 0x0F70u && waitcnt_vm(6) == 0x0F76u && waitcnt_vm(63) == 0xCF7Fu,
              "s_waitcnt vmcnt encoding");

constexpr int kXor1 = 0xB1;        // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kXor2 = 0x4E;        // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kHalfMirror = 0x141;  // lane i <-> 7 - i within each 8
constexpr int kMirror = 0x140;      // lane i <-> 15 - i within each 16

// Every control used here reads a lane inside the same row, so no lane is
// out of range; bound_ctrl lets the compiler fold the move into the
// instruction that consumes it (one DPP-modified max per level).
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
// The value of the lane 16 (32) apart: swapping a register with itself
// leaves rows (r & ~1, r | 1) -- halves (0, 1) -- in the two results.
__device__ __forceinline__ int swap16(int v) {
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((__lane_id() & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ int swap32(int v) {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((__lane_id() & 32) ? r[0] : r[1]);
}

// partner's value at level L (0..5)
template <int L>
__device__ __forceinline__ int partner(int v) {
    if constexpr (L == 0) return dpp<kXor1>(v);
    else if constexpr (L == 1) return dpp<kXor2>(v);
    else if constexpr (L == 2) return dpp<kHalfMirror>(v);
    else if constexpr (L == 3) return dpp<kMirror>(v);
    else if constexpr (L == 4) return swap16(v);
    else return swap32(v);
}
template <int L>
__device__ __forceinline__ float partner(float v) {
    return __int_as_float(partner<L>(__float_as_int(v)));
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, partner<0>(v));
    v = fmaxf(v, partner<1>(v));
    v = fmaxf(v, partner<2>(v));
    v = fmaxf(v, partner<3>(v));
    v = fmaxf(v, partner<4>(v));
    return fmaxf(v, partner<5>(v));
}
__device__ __forceinline__ int wave_max(int v) {
    v = max(v, partner<0>(v));
    v = max(v, partner<1>(v));
    v = max(v, partner<2>(v));
    v = max(v, partner<3>(v));
    v = max(v, partner<4>(v));
    return max(v, partner<5>(v));
}

// (v, i) of the lane ranking first by value descending, then index
// ascending (a total order when indices are distinct); p travels along.
template <int L>
__device__ __forceinline__ void argmax_level(float& v, int& i, int& p) {
    const float tv = partner<L>(v);
    const int ti = partner<L>(i), tp = partner<L>(p);
    if (tv > v || (tv == v && ti < i)) {
        v = tv;
        i = ti;
        p = tp;
    }
}
__device__ __forceinline__ void wave_argmax(float& v, int& i, int& p) {
    argmax_level<0>(v, i, p);
    argmax_level<1>(v, i, p);
    argmax_level<2>(v, i, p);
    argmax_level<3>(v, i, p);
    argmax_level<4>(v, i, p);
    argmax_level<5>(v, i, p);
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    int p = 0;
    wave_argmax(v, i, p);
}

}  // namespace md_wave
