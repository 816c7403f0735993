// Device routine of the router top-k (shared by the route kernel and the
// fused route + permute kernel).
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
// key is never 0, even for -inf).  The wave maximum uses DPP row permutes
// inside each row of 16 lanes and four readlanes across the rows.
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

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max(uint64_t k) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)k, CTRL, 0xf, 0xf, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(k >> 32), CTRL, 0xf, 0xf, false);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > k ? o : k;
}

// Largest key over the wave (the same value in every lane).
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
    k = dpp_max<0xB1>(k);    // quad_perm [1,0,3,2]
    k = dpp_max<0x4E>(k);    // quad_perm [2,3,0,1]
    k = dpp_max<0x141>(k);   // row_half_mirror
    k = dpp_max<0x140>(k);   // row_mirror: every lane holds its row's maximum
    uint64_t best = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)k, 16 * r);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(k >> 32), 16 * r);
        const uint64_t v = ((uint64_t)hi << 32) | lo;
        best = v > best ? v : best;
    }
    return best;
}

// Top-k of one token's logits row; lane 0 writes ids[0..k) and w[0..k), and
// the ids also to lds_ids[0..k) if that is not null.
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int lane,
                                            int32_t* __restrict__ ids, float* __restrict__ wout,
                                            int* lds_ids = nullptr) {
    uint64_t key[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < E ? make_key(row[e], e) : 0ull;
    }
    float top_v[MOE_MAX_K];
    int top_i[MOE_MAX_K];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
        top_v[j] = 0.f;
        top_i[j] = 0;
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
        if (j < k) {
            uint64_t mine = 0;
#pragma unroll
            for (int i = 0; i < VPL; ++i) mine = key[i] > mine ? key[i] : mine;
            const uint64_t best = wave_max_key(mine);
            top_i[j] = (int)(0xffffffffu - (uint32_t)best);
            top_v[j] = mono_float((uint32_t)(best >> 32));
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (key[i] == best) key[i] = 0ull;   // taken (keys are unique: ids differ)
        }
    }
    if (lane == 0) {
        float sum = 0.f;
        float ex[MOE_MAX_K];
#pragma unroll
        for (int j = 0; j < MOE_MAX_K; ++j) {
            ex[j] = j < k ? expf(top_v[j] - top_v[0]) : 0.f;
            sum += ex[j];
        }
#pragma unroll
        for (int j = 0; j < MOE_MAX_K; ++j) {
            if (j < k) {
                ids[j] = top_i[j];
                wout[j] = ex[j] / sum;
                if (lds_ids) lds_ids[j] = top_i[j];
            }
        }
    }
}

}  // namespace moeq
