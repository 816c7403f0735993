// Gated combine and the activation conversion.
//
// out[t] = sum_{j=0}^{k-1} w[t, j] * y_perm[inv_perm[t*k + j]], summed in
// ascending j in fp32, plus the shared expert's y_shared[t] after the sum when
// there is one.  Every output element has exactly one writer, so no
// atomics are needed and the bits do not depend on scheduling.
// (The combine order changes the bits: "GLM-5.3-Flash-TR3-8bpw (K8)",
// Fidelity / Excess over control.)
#include "dev_common.h"

namespace moeq {

namespace {

template <bool SHARED>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y_perm,
                                                 const int32_t* __restrict__ inv_perm,
                                                 const float* __restrict__ w,
                                                 const float* __restrict__ y_shared, int k, int H,
                                                 int nbh, float* __restrict__ out) {
    const int64_t t = blockIdx.x / nbh;
    const int h = ((blockIdx.x % nbh) * 256 + threadIdx.x) * 4;
    if (h >= H) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
        const int64_t row = inv_perm[t * k + j];
        const float wj = w[t * k + j];
        f32x4 y = *reinterpret_cast<const f32x4*>(y_perm + row * H + h);
        acc = acc + wj * y;
    }
    if constexpr (SHARED) acc = acc + *reinterpret_cast<const f32x4*>(y_shared + t * H + h);
    *reinterpret_cast<f32x4*>(out + t * H + h) = acc;
}

// bf16 -> fp16, 8 elements per thread (exact for 2^-14 <= |x| <= 65504).
__global__ __launch_bounds__(256) void k_x_to_f16(const uint16_t* __restrict__ x, int64_t n8,
                                                  uint16_t* __restrict__ x16) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const f16x8 o = bf16x8_to_f16x8(*reinterpret_cast<const u32x4*>(x + i * 8));
    *reinterpret_cast<f16x8*>(x16 + i * 8) = o;
}

}  // namespace

int launch_combine(const float* y_perm, const int32_t* inv_perm, const float* w,
                   const float* y_shared, int64_t T, int32_t k, int32_t H, float* out,
                   void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int nbh = (H / 4 + 255) / 256;
    if (y_shared)
        k_combine<true><<<(unsigned)(T * nbh), 256, 0, s>>>(y_perm, inv_perm, w, y_shared, k, H,
                                                            nbh, out);
    else
        k_combine<false><<<(unsigned)(T * nbh), 256, 0, s>>>(y_perm, inv_perm, w, nullptr, k, H,
                                                             nbh, out);
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

int launch_x_to_f16(const uint16_t* x, int64_t n, uint16_t* x16, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int64_t n8 = n / 8;
    k_x_to_f16<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(x, n8, x16);
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

}  // namespace moeq
