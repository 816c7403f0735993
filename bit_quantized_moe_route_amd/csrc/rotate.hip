// Online rotations of a rotated layer ("GLM-5.3 Vision NestQuant 1.75-4 bit",
// Method: random signs + Hadamard-128 on both sides of each weight matrix).
//
// A stored matrix is W_rot = R_out W R_in^T with R = blockdiag(H/sqrt(128))
// diag(s) (H the 128 x 128 Hadamard matrix, entries +-1), so
// W x = R_out^T W_rot R_in x.  The kernels apply the unnormalised transform
// and fold the two 1/sqrt(128) factors of a matrix into exact powers of two:
// the input side scales by 1/16 and the output side by 1/8 (16 * 8 = 128).
//
//   k_rot<0> (gate/up input):  x'[r]  = H (s_in13[e] * x[t]) / 16         -> fp16
//   k_rot<1> (middle):         g = s_og[e] * H g'[r] / 8, u likewise,
//                              h = silu(g) * u,
//                              h'[r] = H (s_in2[e] * h) / 16               -> fp16
//   k_rot<2> (down output):    y[r]  = s_o2[e] * H y'[r] / 8               (in place)
//
// for every permuted row r of expert e and token t = perm_src[r] / k, one
// 128-wide block per wave: lane L holds elements 2L and 2L+1 and the seven
// butterfly stages are one in-lane stage and six lane exchanges.
#include "dev_common.h"

namespace moeq {

namespace {

// Unnormalised Walsh-Hadamard transform of the wave's 128 values (Sylvester
// order: out[i] = sum_j (-1)^popcount(i & j) in[j]).
__device__ __forceinline__ void fwht128(float& a, float& b, int lane) {
    float t = a + b;
    b = a - b;
    a = t;
#pragma unroll
    for (int s = 0; s < 6; ++s) {
        const float pa = __shfl_xor(a, 1 << s);
        const float pb = __shfl_xor(b, 1 << s);
        const bool hi = (lane >> s) & 1;
        a = hi ? pa - a : a + pa;
        b = hi ? pb - b : b + pb;
    }
}

// The expert whose permuted rows hold row r: the number of experts whose
// segment ends at or before r (offsets[E] = rows > r).  One round of loads.
__device__ __forceinline__ int row_expert(const int32_t* __restrict__ offsets, int E, int r,
                                          int lane) {
    int n = 0;
    for (int c0 = 0; c0 < E; c0 += 64) {
        const int e = c0 + lane;
        const bool le = e < E && offsets[e + 1] <= r;
        n += __popcll(__ballot(le));
    }
    return n;
}

// Signs of elements 2L, 2L+1 of 128-block b of a section (bit set = -1).
__device__ __forceinline__ void signs2(const uint8_t* sec, int b, int lane, float& sa, float& sb) {
    const uint32_t byte = sec[16 * b + (lane >> 2)];
    const int bit = (2 * lane) & 7;
    sa = (byte >> bit) & 1 ? -1.f : 1.f;
    sb = (byte >> (bit + 1)) & 1 ? -1.f : 1.f;
}

__device__ __forceinline__ float silu_mul_r(float g, float u) {
    return g * u / (1.0f + expf(-g));
}

struct RotArgs {
    const int32_t* offsets;
    const int32_t* perm_src;
    const uint8_t* signs;   // per expert: s_in13 | s_og | s_ou | s_in2 | s_o2
    int64_t sign_stride;
    const uint16_t* x;      // MODE 0: bf16 tokens [T, H]
    _Float16* xrot;         // MODE 0: out [rows, H]
    const float* gu;        // MODE 1: g' | u' [rows, 2I]
    _Float16* h16;          // MODE 1: out h' [rows, I]
    float* y;               // MODE 2: [rows, H] in place
    int E, H, I, k, rows;
    int nblk;               // 128-blocks per row (H or I / 128)
    int nbw;                // workgroups per row (nblk / 4, rounded up)
};

template <int MODE>
__global__ __launch_bounds__(256) void k_rot(RotArgs A) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x / A.nbw;
    const int b = (blockIdx.x % A.nbw) * 4 + (threadIdx.x >> 6);
    if (r >= A.rows || b >= A.nblk) return;
    const int e = row_expert(A.offsets, A.E, r, lane);
    const uint8_t* sg = A.signs + (int64_t)e * A.sign_stride;
    const int c = 128 * b + 2 * lane;                      // first element of the lane
    float sa, sb;
    if constexpr (MODE == 0) {
        const int t = A.perm_src[r] / A.k;
        const uint32_t v = *reinterpret_cast<const uint32_t*>(A.x + (int64_t)t * A.H + c);
        float a = __uint_as_float(v << 16), bb = __uint_as_float(v & 0xffff0000u);
        signs2(sg, b, lane, sa, sb);
        a *= sa;
        bb *= sb;
        fwht128(a, bb, lane);
        f16x2 o = {(_Float16)(a * 0.0625f), (_Float16)(bb * 0.0625f)};
        *reinterpret_cast<f16x2*>(A.xrot + (int64_t)r * A.H + c) = o;
    } else if constexpr (MODE == 1) {
        const float* gp = A.gu + (int64_t)r * (2 * A.I) + c;
        float2 g = *reinterpret_cast<const float2*>(gp);
        float2 u = *reinterpret_cast<const float2*>(gp + A.I);
        fwht128(g.x, g.y, lane);
        fwht128(u.x, u.y, lane);
        const uint8_t* s_og = sg + A.H / 8;
        const uint8_t* s_ou = s_og + A.I / 8;
        const uint8_t* s_i2 = s_ou + A.I / 8;
        signs2(s_og, b, lane, sa, sb);
        g.x *= sa * 0.125f;
        g.y *= sb * 0.125f;
        signs2(s_ou, b, lane, sa, sb);
        u.x *= sa * 0.125f;
        u.y *= sb * 0.125f;
        float h0 = silu_mul_r(g.x, u.x), h1 = silu_mul_r(g.y, u.y);
        signs2(s_i2, b, lane, sa, sb);
        h0 *= sa;
        h1 *= sb;
        fwht128(h0, h1, lane);
        f16x2 o = {(_Float16)(h0 * 0.0625f), (_Float16)(h1 * 0.0625f)};
        *reinterpret_cast<f16x2*>(A.h16 + (int64_t)r * A.I + c) = o;
    } else {
        float2* yp = reinterpret_cast<float2*>(A.y + (int64_t)r * A.H + c);
        float2 y = *yp;
        fwht128(y.x, y.y, lane);
        const uint8_t* s_o2 = sg + A.H / 8 + 3 * (A.I / 8);
        signs2(s_o2, b, lane, sa, sb);
        y.x *= sa * 0.125f;
        y.y *= sb * 0.125f;
        *yp = y;
    }
}

template <int MODE>
int launch_rot(RotArgs a, int n, hipStream_t s) {
    a.nblk = n / 128;
    a.nbw = (a.nblk + 3) / 4;
    if (a.rows == 0) return MOE_OK;
    k_rot<MODE><<<(unsigned)((int64_t)a.rows * a.nbw), 256, 0, s>>>(a);
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

RotArgs rot_args(const LayerView& L, const int32_t* offsets, int64_t rows) {
    RotArgs a{};
    a.offsets = offsets;
    a.signs = L.rot;
    a.sign_stride = L.rot_stride;
    a.E = L.E;
    a.H = L.H;
    a.I = L.I;
    a.rows = (int)rows;
    return a;
}

}  // namespace

int launch_rot_in(const LayerView& L, const uint16_t* x_bf16, const int32_t* perm_src,
                  const int32_t* offsets, int64_t T, int32_t k, uint16_t* xrot, void* stream) {
    RotArgs a = rot_args(L, offsets, T * k);
    a.perm_src = perm_src;
    a.x = x_bf16;
    a.xrot = reinterpret_cast<_Float16*>(xrot);
    a.k = k;
    return launch_rot<0>(a, L.H, reinterpret_cast<hipStream_t>(stream));
}

int launch_rot_mid(const LayerView& L, const float* gu, const int32_t* offsets, int64_t rows,
                   uint16_t* h16, void* stream) {
    RotArgs a = rot_args(L, offsets, rows);
    a.gu = gu;
    a.h16 = reinterpret_cast<_Float16*>(h16);
    return launch_rot<1>(a, L.I, reinterpret_cast<hipStream_t>(stream));
}

int launch_rot_out(const LayerView& L, float* y, const int32_t* offsets, int64_t rows,
                   void* stream) {
    RotArgs a = rot_args(L, offsets, rows);
    a.y = y;
    return launch_rot<2>(a, L.H, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace moeq
