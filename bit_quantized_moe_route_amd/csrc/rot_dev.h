// Device helpers of the online rotations, shared by the rotation kernels and
// the rotated layer's combine (the same butterflies in the same order, so
// both give the same bits).
#pragma once

#include "dev_common.h"

namespace moeq {
namespace {

// The value of lane L ^ (1 << S) (S < 5: inside the lane's half-wave): DPP
// moves for S = 0, 1 (quad_perm [1,0,3,2] / [2,3,0,1]), 2 (row_shl:4 into
// banks 0 and 2 of each 16-lane row, row_shr:4 into banks 1 and 3) and 3
// (row_ror:8); a lane permute for S = 4.
template <int CTRL, int BANKS>
__device__ __forceinline__ float dpp_mov(float old, float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, BANKS, false));
}
template <int S>
__device__ __forceinline__ float xor_partner(float v) {
    if constexpr (S == 0)
        return dpp_mov<0xB1, 0xF>(0.f, v);
    else if constexpr (S == 1)
        return dpp_mov<0x4E, 0xF>(0.f, v);
    else if constexpr (S == 2)
        return dpp_mov<0x114, 0xA>(dpp_mov<0x104, 0x5>(0.f, v), v);
    else if constexpr (S == 3)
        return dpp_mov<0x128, 0xF>(0.f, v);
    else
        return __shfl_xor(v, 16);
}

// One butterfly stage over lane bit S: the lower lane of a pair keeps
// v + p, the upper one p - v (p: the partner's value), written p + (+-v).
template <int S>
__device__ __forceinline__ void fwht_stage(f32x4& v, int lane) {
    const bool hi = (lane >> S) & 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float p = xor_partner<S>(v[q]);
        v[q] = p + (hi ? -v[q] : v[q]);
    }
}

// Unnormalised Walsh-Hadamard transform of each half-wave's 128 values
// (Sylvester order: out[i] = sum_j (-1)^popcount(i & j) in[j]), lane L
// holding elements 4 (L & 31) + q: two in-lane stages, then one per lane bit.
__device__ __forceinline__ void fwht128(f32x4& v, int lane) {
    float a = v[0] + v[1], b = v[0] - v[1], c = v[2] + v[3], d = v[2] - v[3];
    v = f32x4{a + c, b + d, a - c, b - d};
    fwht_stage<0>(v, lane);
    fwht_stage<1>(v, lane);
    fwht_stage<2>(v, lane);
    fwht_stage<3>(v, lane);
    fwht_stage<4>(v, lane);
}

// +1 / -1 of 4 elements from their sign bits (bit set = -1).
__device__ __forceinline__ f32x4 signs_of(uint32_t bits) {
    return f32x4{bits & 1 ? -1.f : 1.f, bits & 2 ? -1.f : 1.f, bits & 4 ? -1.f : 1.f,
                 bits & 8 ? -1.f : 1.f};
}

// The byte of a section holding the sign bits of the lane's 4 elements of
// span s (its nibble: lane & 1).
__device__ __forceinline__ const uint8_t* sign_byte(const uint8_t* sec, int s, int lane) {
    return sec + 32 * s + (lane >> 1);
}

// Signs of the lane's 4 elements of span s of a section (bit set = -1);
// +1 for a lane outside the row.
__device__ __forceinline__ f32x4 signs4(const uint8_t* sec, int s, int lane, bool in) {
    const uint32_t bits = in ? *sign_byte(sec, s, lane) >> (4 * (lane & 1)) : 0u;
    return signs_of(bits);
}

__device__ __forceinline__ f32x4 bf16x4_to_f32(uint2 v) {
    return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                 __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
}

__device__ __forceinline__ f16x4 to_f16x4(f32x4 v, float sc) {
    return f16x4{(_Float16)(v[0] * sc), (_Float16)(v[1] * sc), (_Float16)(v[2] * sc),
                 (_Float16)(v[3] * sc)};
}

// silu(g) * u of the middle rotation step.
__device__ __forceinline__ float silu_mul_r(float g, float u) {
    return g * u / (1.0f + expf(-g));
}

}  // namespace
}  // namespace moeq
