// Router top-k kernel: one wavefront per token (see topk_dev.h).
#include "topk_dev.h"

namespace moeq {

namespace {

template <int VPL>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits,
                                                    int64_t T, int E, int k,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ wout) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    route_token<VPL>(logits + t * E, E, k, lane, ids + t * k, wout + t * k);
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
