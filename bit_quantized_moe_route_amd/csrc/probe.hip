// Measurement aid: the rate at which the chip streams a buffer from HBM with
// the same kind of loads the weight-streaming kernels issue (16-byte
// non-temporal loads, several in flight per lane), as context for their
// roofline fraction.
#include "dev_common.h"

namespace moeq {

namespace {

constexpr int kProbeUnroll = 4;

// Workgroup w reads 16-byte chunks w*256 + tid, + grid*256, ... ; the XOR of
// everything it read goes to sink[w] (so the loads cannot be dropped).
__global__ __launch_bounds__(256) void k_probe_read(const u32x4* __restrict__ buf, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t acc = 0;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    // one value per workgroup: the XOR over its four waves
    __shared__ uint32_t red[4];
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

int launch_probe_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    k_probe_read<<<(unsigned)blocks, 256, 0, s>>>(reinterpret_cast<const u32x4*>(buf),
                                                   (int64_t)(bytes / 16), sink);
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

}  // namespace moeq
