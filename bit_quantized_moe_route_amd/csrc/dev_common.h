// Device-side helpers shared by the HIP kernels: vector types, the NVFP4 and
// VQ decode routines and the 16x16x32 fp16 MFMA wrapper.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "internal.h"

namespace moeq {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define MOEQ_CHECK_LAUNCH()                                                   \
    do {                                                                      \
        hipError_t _e = hipGetLastError();                                    \
        if (_e != hipSuccess)                                                 \
            return ::moeq::fail(MOE_EHIP, std::string("HIP launch: ") +       \
                                              hipGetErrorString(_e));         \
    } while (0)

// D += A * B over one 16x16x32 fp16 tile (fp32 accumulate).
// Lane L holds A[row L&15][k (L>>4)*8 + 0..7], B[k (L>>4)*8 + 0..7][col L&15],
// D[row (L>>4)*4 + i][col L&15], i = 0..3.
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}

// ---------------------------------------------------------------- NVFP4
// The two E4M3 scale bytes of a lane (low byte = first 16 inputs), decoded to
// fp16 and broadcast to pairs.  E4M3 -> fp16 is exact (every E4M3 value is a
// normal fp16).
__device__ __forceinline__ void nv_scales(uint32_t two_bytes, f16x2& s0, f16x2& s1) {
    f16x2 s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two_bytes, 1.0f, false);
    s0 = f16x2{s[0], s[0]};
    s1 = f16x2{s[1], s[1]};
}

// Eight weights from four code bytes (element 2i in the low nibble of byte i)
// times their block scale.  The E2M1 -> fp16 conversion is exact, and so is
// the fp16 product: an E2M1 value (2 significant bits) times an E4M3 scale
// (4 bits) has at most 6 significant bits and lies in [2^-10, 2688].  (The
// scale operand of the conversion instruction only takes a power of two, so
// the scale is applied with a packed fp16 multiply.)
__device__ __forceinline__ f16x8 nv_dequant8(uint32_t w, f16x2 s) {
    f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
    f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
    f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
    f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
    return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// One lane's 32 decoded weights of an NVFP4 tile: a[s] covers inputs
// (L>>4)*32 + 8s + 0..7 of the tile, s = 0..3.
struct NvFrag {
    u32x4 codes;
    uint32_t scales;
};

__device__ __forceinline__ NvFrag nv_load(const uint8_t* tile, int lane) {
    NvFrag f;
    f.codes = *reinterpret_cast<const u32x4*>(tile + lane * 16);
    f.scales = *reinterpret_cast<const uint16_t*>(tile + kNvScaleOff + lane * 2);
    return f;
}

__device__ __forceinline__ void nv_decode(const NvFrag& f, f16x8 a[4]) {
    f16x2 s0, s1;
    nv_scales(f.scales, s0, s1);
    a[0] = nv_dequant8(f.codes[0], s0);
    a[1] = nv_dequant8(f.codes[1], s0);
    a[2] = nv_dequant8(f.codes[2], s1);
    a[3] = nv_dequant8(f.codes[3], s1);
}

// ---------------------------------------------------------------- VQ
// Codebook row of a uint16 code: 8 fp16 values (16 bytes).
__device__ __forceinline__ f16x8 vq_row(const uint8_t* cb, uint32_t code) {
    return *reinterpret_cast<const f16x8*>(cb + (size_t)code * 16);
}

// 8 bf16 values (bits, two per dword, low half first) to fp16: bf16 -> fp32
// is exact, fp32 -> fp16 rounds to nearest even (exact for
// 2^-14 <= |x| <= 65504).
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(u32x4 v) {
    f16x8 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        o[2 * q] = (_Float16)__uint_as_float(v[q] << 16);
        o[2 * q + 1] = (_Float16)__uint_as_float(v[q] & 0xffff0000u);
    }
    return o;
}

// Non-temporal 16-byte load for streamed weight bytes (read once per call),
// so they do not push the shared VQ codebooks out of the caches.
__device__ __forceinline__ u32x4 load_stream16(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------- experts
struct ActiveExpert {
    int e;      // expert id, -1 if there is no s-th active expert
    int r0;     // first permuted row of the expert (offsets[e])
    int me;     // number of rows (assignments) of the expert
    int ridx;   // record index within its format's pool
};

// The s-th expert (ascending id) with at least one assignment and format
// `fmt`.  All loads are issued up front (one memory round trip); the answer
// is broadcast from the owning lane, so every lane gets the same result.
// E <= 64 * 16.
__device__ __forceinline__ ActiveExpert find_active_expert(const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ rec,
                                                           int E, int fmt, int s, int lane) {
    // groups of 4 chunks of 64 experts: one memory round trip per group
    constexpr int kG = 4;
    ActiveExpert r{-1, 0, 0, 0};
    int seen = 0;
    for (int g0 = 0; g0 < E; g0 += 64 * kG) {
        int o0[kG], o1[kG], rc[kG];
#pragma unroll
        for (int c = 0; c < kG; ++c) {
            const int e = g0 + 64 * c + lane;
            const bool in = e < E;
            o0[c] = in ? offsets[e] : 0;
            o1[c] = in ? offsets[e + 1] : 0;
            rc[c] = in ? rec[e] : 0;
        }
#pragma unroll
        for (int c = 0; c < kG; ++c) {
            const bool act = o1[c] > o0[c] && (rc[c] >> 24) == fmt;
            uint64_t m = __ballot(act);
            const int n = __popcll(m);
            if (r.e < 0 && s < seen + n) {
                for (int i = 0; i < s - seen; ++i) m &= m - 1;   // drop lower set bits
                const int owner = __ffsll((unsigned long long)m) - 1;
                r.e = g0 + 64 * c + owner;
                r.r0 = __builtin_amdgcn_readlane(o0[c], owner);
                r.me = __builtin_amdgcn_readlane(o1[c], owner) - r.r0;
                r.ridx = __builtin_amdgcn_readlane(rc[c], owner) & 0xffffff;
            }
            seen += n;
        }
        if (r.e >= 0) break;
    }
    return r;
}

}  // namespace moeq
