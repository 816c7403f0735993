// Device routine of the router top-k (shared by the route kernel, the fused
// route + permute kernel and the small-batch fused layer kernels).
//
// One wavefront per token.  Each lane holds E/64 (rounded up) logits.  k
// rounds of a wave-wide argmax pick the experts in rank order: larger logit
// first, equal logits -> lower expert id first, -0.0 == +0.0.  The softmax
// over the chosen logits is taken in fp32.
// (8 of 256 experts per token: "GLM-5-NVFP4-MTP", Model Description.)
//
// The order is carried by one 64-bit key per candidate:
//   key = (monotone bits of (logit + 0.0)) << 32 | (0xffffffff - id)
// so the best candidate is the largest key (key 0 = empty or taken; a real
// key is never 0, even for -inf).  Wave maxima use DPP row permutes inside
// each row of 16 lanes and four readlanes across the rows, on 32-bit halves.
#pragma once

#include "dev_common.h"

namespace moeq {

// float -> uint32 preserving order (adding +0.0 first turns -0.0 into +0.0)
__device__ __forceinline__ uint32_t mono_bits(float v) {
    const uint32_t u = __float_as_uint(v + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float mono_float(uint32_t m) {
    return __uint_as_float((m & 0x80000000u) ? (m & 0x7fffffffu) : ~m);
}

__device__ __forceinline__ uint64_t make_key(float v, int id) {
    return ((uint64_t)mono_bits(v) << 32) | (uint64_t)(0xffffffffu - (uint32_t)id);
}

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Largest 32-bit value (unsigned) over the wave, the same in every lane: DPP
// row permutes inside each row of 16 lanes, then the four rows' maxima.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xf, 0xf, false));
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xf, 0xf, false));
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x141, 0xf, 0xf, false));
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x140, 0xf, 0xf, false));
    const uint32_t a = umax32((uint32_t)__builtin_amdgcn_readlane(v, 0),
                              (uint32_t)__builtin_amdgcn_readlane(v, 16));
    const uint32_t b = umax32((uint32_t)__builtin_amdgcn_readlane(v, 32),
                              (uint32_t)__builtin_amdgcn_readlane(v, 48));
    return umax32(a, b);
}

// Top-k of one token's logits row, the same in every lane: top_i[j] / top_v[j]
// = id and logit of rank j (j < k).
// Each round takes the wave's largest remaining key: first the largest
// high half (the logit's monotone bits) over the lanes' best keys, then,
// only if several lanes hold that logit, the largest low half (the lowest
// id) among them.  The lane that owns the winner clears that key.
template <int VPL>
__device__ __forceinline__ void topk_select(const float* __restrict__ row, int E, int k, int lane,
                                            float (&top_v)[MOE_MAX_K], int (&top_i)[MOE_MAX_K]) {
    uint64_t key[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < E ? make_key(row[e], e) : 0ull;
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
        top_v[j] = 0.f;
        top_i[j] = 0;
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
        if (j < k) {
            // the lane's best remaining key and its slot
            uint64_t mine = key[0];
            int slot = 0;
#pragma unroll
            for (int i = 1; i < VPL; ++i)
                if (key[i] > mine) {
                    mine = key[i];
                    slot = i;
                }
            const uint32_t hi = (uint32_t)(mine >> 32);
            const uint32_t lo = (uint32_t)mine;
            const uint32_t best_hi = wave_max_u32(hi);
            const uint64_t tied = __ballot(hi == best_hi);
            uint32_t best_lo;
            if (__popcll(tied) == 1)
                best_lo = (uint32_t)__builtin_amdgcn_readlane(lo, __ffsll((unsigned long long)tied) - 1);
            else
                best_lo = wave_max_u32(hi == best_hi ? lo : 0u);
            top_i[j] = (int)(0xffffffffu - best_lo);
            top_v[j] = mono_float(best_hi);
            // keys are unique (ids differ): exactly one lane holds the winner
            if (hi == best_hi && lo == best_lo) {
#pragma unroll
                for (int i = 0; i < VPL; ++i)
                    if (i == slot) key[i] = 0ull;
            }
        }
    }
}

// The softmax weights of the chosen logits (fp32): w[j] = exp(v_j - v_0) /
// sum_{i<k} exp(v_i - v_0).
__device__ __forceinline__ void topk_weights(const float (&top_v)[MOE_MAX_K], int k,
                                             float (&w)[MOE_MAX_K]) {
    float sum = 0.f;
    float ex[MOE_MAX_K];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
        ex[j] = j < k ? expf(top_v[j] - top_v[0]) : 0.f;
        sum += ex[j];
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) w[j] = ex[j] / sum;
}

// Top-k of one token's logits row; lane 0 writes ids[0..k) and w[0..k), and
// the ids also to lds_ids[0..k) if that is not null.
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int lane,
                                            int32_t* __restrict__ ids, float* __restrict__ wout,
                                            int* lds_ids = nullptr) {
    float top_v[MOE_MAX_K];
    int top_i[MOE_MAX_K];
    topk_select<VPL>(row, E, k, lane, top_v, top_i);
    if (lane == 0) {
        float w[MOE_MAX_K];
        topk_weights(top_v, k, w);
#pragma unroll
        for (int j = 0; j < MOE_MAX_K; ++j) {
            if (j < k) {
                ids[j] = top_i[j];
                wout[j] = w[j];
                if (lds_ids) lds_ids[j] = top_i[j];
            }
        }
    }
}

}  // namespace moeq
