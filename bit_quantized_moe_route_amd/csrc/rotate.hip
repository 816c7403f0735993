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
//   k_rot<3> (middle, wide):   as k_rot<1> with h'[r] = H_512 (s_in2[e] * h) / 32
//
// for every permuted row r of expert e and token t = perm_src[r] / k.
// k_rot<3> serves the same Method's wide variant of the down projection's
// input side (random signs and one Hadamard-512 per 512 intermediate
// channels): the factors 1/sqrt(512) and 1/sqrt(128) of that matrix fold into
// 1/32 and 1/8 (32 * 8 = 256), so the down output step stays k_rot<2>.  A
// workgroup of 4 waves owns 4 spw 256-element spans of a row (all of it for
// many rows, 4 spans for few, so that a decode step still has enough
// workgroups); wave w takes spans w, w + 4, ...: lane L holds elements
// 4L .. 4L+3 of a span, i.e.
// half L >> 5 of the span's two 128-blocks, so each wave access is a
// contiguous 16-byte-per-lane load or store, and a block's seven butterfly
// stages are two in-lane stages and five lane exchanges inside a half-wave.
// The next span's loads are issued before the current span is transformed.
// k_rot<3>'s unit is a 512-block, two adjacent spans in one wave (lane L
// holds elements 4L .. 4L+3 of each): Sylvester's H_512 = H_4 (x) H_128 adds
// two stages to the spans' 128-point transforms, one across the half-waves
// (element bit 7) and one between the two spans in-lane (bit 8).
// A row of an odd number of 128-blocks ends with a half span: its upper
// half-wave neither loads nor stores (its butterflies never mix with the
// lower half's).
#include "rot_dev.h"

namespace moeq {

namespace {

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

struct RotArgs {
    const int32_t* offsets;
    const int32_t* row_ids;   // MODE 1, 3: row r is of expert row_ids[r] (NULL: from offsets)
    const int32_t* perm_src;
    const uint8_t* signs;   // per expert: s_in13 | s_og | s_ou | s_in2 | s_o2
    int64_t sign_stride;
    const uint16_t* x;      // MODE 0: bf16 tokens [T, H]
    _Float16* xrot;         // MODE 0: out [rows, H]
    const float* gu;        // MODE 1, 3: g' | u' [rows, 2I]
    _Float16* h16;          // MODE 1, 3: out h' [rows, I]
    float* y;               // MODE 2: [rows, H] in place
    int E, H, I, k, rows;
    int nspan;              // 256-element spans per row, the last maybe half
                            // (MODE 3: 512-blocks)
    int half_tail;          // the row ends with a half span
    int spw;                // spans (MODE 3: 512-blocks) per wave
    int nwg;                // workgroups per row
};

template <int MODE>
__global__ __launch_bounds__(256) void k_rot(RotArgs A) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = blockIdx.x / A.nwg;
    const int s0 = (blockIdx.x % A.nwg) * 4 * A.spw + wave;   // first span of the wave
    const int send = min(A.nspan, s0 - wave + 4 * A.spw);     // end of the workgroup's spans
    if (s0 >= send) return;
    const int e = A.row_ids ? A.row_ids[r] : row_expert(A.offsets, A.E, r, lane);
    const uint8_t* sg = A.signs + (int64_t)e * A.sign_stride;
    const int o = 4 * lane;                                   // lane's offset in a span
    // does the lane's part of span s lie inside the row?
    auto in = [&](int s) { return !A.half_tail || s + 1 < A.nspan || lane < 32; };
    if constexpr (MODE == 0) {
        const uint16_t* xr = A.x + (int64_t)(A.perm_src[r] / A.k) * A.H + o;
        _Float16* dst = A.xrot + (int64_t)r * A.H + o;
        uint2 cur = make_uint2(0u, 0u);
        if (in(s0)) cur = *reinterpret_cast<const uint2*>(xr + 256 * s0);
        for (int s = s0; s < send; s += 4) {
            uint2 nxt = cur;
            if (s + 4 < send && in(s + 4))
                nxt = *reinterpret_cast<const uint2*>(xr + 256 * (s + 4));
            f32x4 v = bf16x4_to_f32(cur) * signs4(sg, s, lane, in(s));
            fwht128(v, lane);
            if (in(s)) *reinterpret_cast<f16x4*>(dst + 256 * s) = to_f16x4(v, 0.0625f);
            cur = nxt;
        }
    } else if constexpr (MODE == 1) {
        const float* gp = A.gu + (int64_t)r * (2 * A.I) + o;
        _Float16* dst = A.h16 + (int64_t)r * A.I + o;
        const uint8_t* s_og = sg + A.H / 8;
        const uint8_t* s_ou = s_og + A.I / 8;
        const uint8_t* s_i2 = s_ou + A.I / 8;
        f32x4 g = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
        if (in(s0)) {
            g = *reinterpret_cast<const f32x4*>(gp + 256 * s0);
            u = *reinterpret_cast<const f32x4*>(gp + A.I + 256 * s0);
        }
        for (int s = s0; s < send; s += 4) {
            f32x4 gn = g, un = u;
            if (s + 4 < send && in(s + 4)) {
                gn = *reinterpret_cast<const f32x4*>(gp + 256 * (s + 4));
                un = *reinterpret_cast<const f32x4*>(gp + A.I + 256 * (s + 4));
            }
            const bool ok = in(s);
            fwht128(g, lane);
            fwht128(u, lane);
            g = g * signs4(s_og, s, lane, ok) * 0.125f;
            u = u * signs4(s_ou, s, lane, ok) * 0.125f;
            f32x4 h;
#pragma unroll
            for (int q = 0; q < 4; ++q) h[q] = silu_mul_r(g[q], u[q]);
            h = h * signs4(s_i2, s, lane, ok);
            fwht128(h, lane);
            if (ok) *reinterpret_cast<f16x4*>(dst + 256 * s) = to_f16x4(h, 0.0625f);
            g = gn;
            u = un;
        }
    } else if constexpr (MODE == 3) {
        // unit p = spans 2p and 2p + 1 (I is a multiple of 512: no tail)
        const float* gp = A.gu + (int64_t)r * (2 * A.I) + o;
        _Float16* dst = A.h16 + (int64_t)r * A.I + o;
        const uint8_t* s_og = sg + A.H / 8;
        const uint8_t* s_ou = s_og + A.I / 8;
        const uint8_t* s_i2 = s_ou + A.I / 8;
        const bool hi = lane >= 32;
        f32x4 g[2], u[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            g[j] = *reinterpret_cast<const f32x4*>(gp + 256 * (2 * s0 + j));
            u[j] = *reinterpret_cast<const f32x4*>(gp + A.I + 256 * (2 * s0 + j));
        }
        for (int p = s0; p < send; p += 4) {
            f32x4 gn[2] = {g[0], g[1]}, un[2] = {u[0], u[1]};
            if (p + 4 < send) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    gn[j] = *reinterpret_cast<const f32x4*>(gp + 256 * (2 * (p + 4) + j));
                    un[j] = *reinterpret_cast<const f32x4*>(gp + A.I + 256 * (2 * (p + 4) + j));
                }
            }
            f32x4 h[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int s = 2 * p + j;
                fwht128(g[j], lane);
                fwht128(u[j], lane);
                const f32x4 gj = g[j] * signs4(s_og, s, lane, true) * 0.125f;
                const f32x4 uj = u[j] * signs4(s_ou, s, lane, true) * 0.125f;
#pragma unroll
                for (int q = 0; q < 4; ++q) h[j][q] = silu_mul_r(gj[q], uj[q]);
                h[j] = h[j] * signs4(s_i2, s, lane, true);
                fwht128(h[j], lane);
#pragma unroll
                for (int q = 0; q < 4; ++q) {   // element bit 7: the other half-wave
                    const float t = __shfl_xor(h[j][q], 32);
                    h[j][q] = hi ? t - h[j][q] : h[j][q] + t;
                }
            }
            // element bit 8: the two spans
            *reinterpret_cast<f16x4*>(dst + 256 * (2 * p)) = to_f16x4(h[0] + h[1], 0.03125f);
            *reinterpret_cast<f16x4*>(dst + 256 * (2 * p + 1)) = to_f16x4(h[0] - h[1], 0.03125f);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                g[j] = gn[j];
                u[j] = un[j];
            }
        }
    } else {
        float* yp = A.y + (int64_t)r * A.H + o;
        const uint8_t* s_o2 = sg + A.H / 8 + 3 * (A.I / 8);
        f32x4 cur = {0.f, 0.f, 0.f, 0.f};
        if (in(s0)) cur = *reinterpret_cast<const f32x4*>(yp + 256 * s0);
        for (int s = s0; s < send; s += 4) {
            f32x4 nxt = cur;
            if (s + 4 < send && in(s + 4))
                nxt = *reinterpret_cast<const f32x4*>(yp + 256 * (s + 4));
            const bool ok = in(s);
            fwht128(cur, lane);
            if (ok)
                *reinterpret_cast<f32x4*>(yp + 256 * s) =
                    cur * signs4(s_o2, s, lane, ok) * 0.125f;
            cur = nxt;
        }
    }
}

constexpr int kRotWholeRowMin = 1024;   // rows from which a workgroup takes a whole row

template <int MODE>
int launch_rot(RotArgs a, int n, hipStream_t s) {
    // units of a row: 256-element spans (the last maybe half), or 512-blocks
    // for the wide middle step (n a multiple of 512)
    const int unit = MODE == 3 ? 512 : 256;
    a.nspan = (n + unit - 1) / unit;
    a.half_tail = n % unit != 0;
    // whole rows per workgroup once there are enough rows to fill the chip
    a.spw = a.rows >= kRotWholeRowMin ? (a.nspan + 3) / 4 : 1;
    a.nwg = (a.nspan + 4 * a.spw - 1) / (4 * a.spw);
    if (a.rows == 0) return MOE_OK;
    k_rot<MODE><<<(unsigned)((int64_t)a.rows * a.nwg), 256, 0, s>>>(a);
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
                   uint16_t* h16, void* stream, const int32_t* row_ids) {
    RotArgs a = rot_args(L, offsets, rows);
    a.row_ids = row_ids;
    a.gu = gu;
    a.h16 = reinterpret_cast<_Float16*>(h16);
    if (L.rot_in2 == MOE_ROT_BLOCK_WIDE) {
        if (L.I % MOE_ROT_BLOCK_WIDE) return fail(MOE_EUNSUPPORTED, "rotation: I % 512 != 0");
        return launch_rot<3>(a, L.I, reinterpret_cast<hipStream_t>(stream));
    }
    return launch_rot<1>(a, L.I, reinterpret_cast<hipStream_t>(stream));
}

int launch_rot_out(const LayerView& L, float* y, const int32_t* offsets, int64_t rows,
                   void* stream) {
    RotArgs a = rot_args(L, offsets, rows);
    a.y = y;
    return launch_rot<2>(a, L.H, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace moeq
