// Gated combine and the activation conversion.
//
// out[t] = sum_{j=0}^{k-1} w[t, j] * y_perm[inv_perm[t*k + j]], summed in
// ascending j in fp32, plus the shared expert's y_shared[t] after the sum when
// there is one.  Every output element has exactly one writer, so no
// atomics are needed and the bits do not depend on scheduling.
// (The combine order changes the bits: "GLM-5.3-Flash-TR3-8bpw (K8)",
// Fidelity / Excess over control.)
//
// A rotated layer's one-call forward folds the down output's rotation back
// into the combine ("GLM-5.3 Vision NestQuant 1.75-4 bit", Method): slot j of
// token t contributes w[t, j] * y_j with y_j = s_o2[e] * H y'_j / 8 (e =
// topk_ids[t, j], y'_j = y_perm[inv_perm[t*k + j]] as the down product left
// it), the same butterflies and the same operation order as the separate
// rotation pass followed by the plain combine, so the same bits, without
// writing y back and reading it again.  A wave takes a 256-element span of
// the row (lane L: elements 4L .. 4L+3, one 128-block per half-wave); a span
// of a row ending in half a span has its upper half-wave idle.
#include "rot_dev.h"

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

struct CombineRotArgs {
    const float* y_perm;
    const int32_t* inv_perm;   // NULL: slot (t, j) is row t*k + j
    const int32_t* ids;
    const float* w;
    const float* y_shared;
    const uint8_t* s_o2;     // the first expert's down-output sign bits
    int64_t sign_stride;     // bytes per expert
    float* out;
    int k, H;
    int nspan, half_tail;    // 256-element spans of a row, the last maybe half
    int nbh;                 // workgroups per row (4 spans each)
};

template <bool SHARED>
__global__ __launch_bounds__(256) void k_combine_rot(CombineRotArgs A) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t t = blockIdx.x / A.nbh;
    const int sp = (int)(blockIdx.x % A.nbh) * 4 + wave;
    if (sp >= A.nspan) return;
    const bool in = !A.half_tail || sp + 1 < A.nspan || lane < 32;
    const int h = sp * 256 + 4 * lane;
    // slots in groups of 8: every load of a group (rows, experts, weights,
    // the y' spans, the sign bytes) is issued before its first transform,
    // from clamped slots and a lane's in-row address
    constexpr int UB = 8;
    const int hl = in ? h : h - 128;
    const int ll = in ? lane : lane - 32;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < A.k; j0 += UB) {
        f32x4 ys[UB];
        uint32_t sb[UB];
        float wj[UB];
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int64_t a = t * A.k + min(j0 + u, A.k - 1);
            const int64_t row = A.inv_perm ? A.inv_perm[a] : a;
            ys[u] = *reinterpret_cast<const f32x4*>(A.y_perm + row * A.H + hl);
            sb[u] = *sign_byte(A.s_o2 + (int64_t)A.ids[a] * A.sign_stride, sp, ll);
            wj[u] = A.w[a];
        }
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            if (j0 + u >= A.k) break;
            f32x4 y = ys[u];
            fwht128(y, lane);
            y = y * signs_of(in ? sb[u] >> (4 * (lane & 1)) : 0u) * 0.125f;
            acc = acc + wj[u] * y;
        }
    }
    if (!in) return;
    if constexpr (SHARED) acc = acc + *reinterpret_cast<const f32x4*>(A.y_shared + t * A.H + h);
    *reinterpret_cast<f32x4*>(A.out + t * A.H + h) = acc;
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

int launch_combine_rot(const LayerView& L, const float* y_perm, const int32_t* inv_perm,
                       const int32_t* ids, const float* w, const float* y_shared, int64_t T,
                       int32_t k, float* out, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    CombineRotArgs a{};
    a.y_perm = y_perm;
    a.inv_perm = inv_perm;
    a.ids = ids;
    a.w = w;
    a.y_shared = y_shared;
    a.s_o2 = L.rot + L.H / 8 + 3 * (L.I / 8);
    a.sign_stride = L.rot_stride;
    a.out = out;
    a.k = k;
    a.H = L.H;
    a.nspan = (L.H + 255) / 256;
    a.half_tail = L.H % 256 != 0;
    a.nbh = (a.nspan + 3) / 4;
    if (T == 0) return MOE_OK;
    const unsigned grid = (unsigned)(T * a.nbh);
    if (y_shared)
        k_combine_rot<true><<<grid, 256, 0, s>>>(a);
    else
        k_combine_rot<false><<<grid, 256, 0, s>>>(a);
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
