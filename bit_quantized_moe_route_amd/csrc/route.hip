// Router top-k: one wavefront per token.
//
// Each lane holds E/64 (rounded up) logits of the token.  k rounds of a
// wave-wide argmax pick the experts in rank order: larger logit first, equal
// logits -> lower expert id first (-0.0 == +0.0 under float compare).  The
// softmax over the chosen logits is then taken in fp32.
// (8 of 256 experts per token: "GLM-5-NVFP4-MTP", Model Description.)
#include "dev_common.h"

namespace moeq {

namespace {

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

template <int VPL>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits,
                                                    int64_t T, int E, int k,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ wout) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* row = logits + t * E;

    float v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        int e = lane + 64 * i;
        v[i] = e < E ? row[e] : -__builtin_inff();
    }
    uint32_t taken = 0;
    // slots beyond E never win: mark them taken
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        if (lane + 64 * i >= E) taken |= 1u << i;

    // fully unrolled over the rank so top_v/top_i stay in registers
    float top_v[MOE_MAX_K];
    int top_i[MOE_MAX_K];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
        if (j >= k) break;
        // lane-local best among the not-taken slots
        float bv = -__builtin_inff();
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            int e = lane + 64 * i;
            if (!(taken & (1u << i)) && better(v[i], e, bv, bi)) {
                bv = v[i];
                bi = e;
            }
        }
        // wave-wide argmax with the same order
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            float ov = __shfl_xor(bv, off);
            int oi = __shfl_xor(bi, off);
            if (better(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        top_v[j] = bv;
        top_i[j] = bi;
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    }
    if (lane == 0) {
        float sum = 0.f;
        float ex[MOE_MAX_K];
#pragma unroll
        for (int j = 0; j < MOE_MAX_K; ++j) {
            if (j >= k) break;
            ex[j] = expf(top_v[j] - top_v[0]);
            sum += ex[j];
        }
#pragma unroll
        for (int j = 0; j < MOE_MAX_K; ++j) {
            if (j >= k) break;
            ids[t * k + j] = top_i[j];
            wout[t * k + j] = ex[j] / sum;
        }
    }
}

}  // namespace

int launch_route_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                      int32_t* ids, float* w, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    dim3 grid((unsigned)((T + 3) / 4)), block(256);
    if (E <= 256)
        k_route_topk<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
    else
        k_route_topk<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

}  // namespace moeq
