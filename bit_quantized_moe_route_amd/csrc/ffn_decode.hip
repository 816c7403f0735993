// Expert FFN for small token batches (decode): a weight-streaming, skinny
// matrix-core product per active expert.
//
// For each active expert e (rows r0 .. r0+M_e of the permuted order):
//   gate/up kernel: g = W_gate x, u = W_up x, h = silu(g) * u  -> h (fp16)
//   down kernel:    y = W_down h                                -> y_perm (fp32)
// ("GLM-5-NVFP4-MTP", What's quantized: gate, up and down projections of the
// routed experts are the low-bit part.)
//
// Work decomposition (gfx950, wave64):
//   * one workgroup = 4 waves = one 16-row group of output channels (gate/up:
//     16 gate rows + the 16 matching up rows) of one active expert;
//   * the 4 waves split the input dimension (tile kb goes to wave kb % 4) and
//     reduce their 16x16 fp32 partial tiles through LDS in a fixed order;
//   * each wave streams its weight tiles straight from HBM into registers
//     (16-byte loads per lane, one tile = 1 KB of codes per wave-load),
//     decodes them in registers to fp16 (exact) and feeds
//     v_mfma_f32_16x16x32_f16 with the weights as the A operand and up to
//     16 tokens per B operand (tokens of the expert beyond 16 use further
//     B tiles; lanes of absent tokens carry zeros).
// The tokens' activations are fp16 copies of x made once per call.
#include "dev_common.h"

namespace moeq {

namespace {

constexpr int kWaves = 4;

// Per-format tile traits ----------------------------------------------------
struct NvFmt {
    static constexpr bool kVq = false;
    static constexpr int TK = kNvTileK;       // inputs per tile
    static constexpr int TB = kNvTileBytes;   // bytes per tile
    static constexpr int STEPS = 4;           // MFMA K-steps per tile
    static constexpr int KSPAN = 32;          // inputs per lane per tile
    struct Frag {
        NvFrag f;
    };
    __device__ __forceinline__ static void load(Frag& fr, const uint8_t* tile, int lane) {
        fr.f.codes = load_stream16(tile + lane * 16);
        fr.f.scales = *reinterpret_cast<const uint16_t*>(tile + kNvScaleOff + lane * 2);
    }
    __device__ __forceinline__ static void decode(const Frag& fr, const uint8_t*, f16x8 a[STEPS]) {
        nv_decode(fr.f, a);
    }
};

struct VqFmt {
    static constexpr bool kVq = true;
    static constexpr int TK = kVqTileK;
    static constexpr int TB = kVqTileBytes;
    static constexpr int STEPS = 8;
    static constexpr int KSPAN = 64;
    struct Frag {
        u32x4 codes;
    };
    __device__ __forceinline__ static void load(Frag& fr, const uint8_t* tile, int lane) {
        fr.codes = load_stream16(tile + lane * 16);
    }
    __device__ __forceinline__ static void decode(const Frag& fr, const uint8_t* cb,
                                                  f16x8 a[STEPS]) {
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            uint32_t c = (fr.codes[s >> 1] >> (16 * (s & 1))) & 0xffffu;
            a[s] = vq_row(cb, c);
        }
    }
};

template <class F>
__device__ __forceinline__ int64_t tiles_k(int kin) {
    return (kin + F::TK - 1) / F::TK;
}

// B operand fragments of one tile for NTT token tiles: lane L holds token
// (L & 15) + 16 tt, inputs k0 + 8 s .. +7 with k0 = kb*TK + (L>>4)*KSPAN.
template <class F, int NTT>
__device__ __forceinline__ void load_b(const _Float16* const xrow[NTT], int k0, int K,
                                       f16x8 b[NTT][F::STEPS]) {
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
        for (int s = 0; s < F::STEPS; ++s) {
            const int kk = k0 + 8 * s;
            if (xrow[tt] != nullptr && kk < K)
                b[tt][s] = *reinterpret_cast<const f16x8*>(xrow[tt] + kk);
            else
                b[tt][s] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
}

struct DecodeArgs {
    const uint8_t* pool13;
    const uint8_t* pool2;
    int64_t stride13;
    int64_t stride2;
    const uint8_t* cb_gate;
    const uint8_t* cb_up;
    const uint8_t* cb_down;
    int64_t cb_stride;
    const int32_t* rec;
    const int32_t* offsets;
    const int32_t* perm_src;
    const _Float16* x16;
    _Float16* h16;
    float* y_perm;
    int E, H, I, k, fmt;
};

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * u / (1.0f + expf(-g));
}

// gate/up + SwiGLU.  grid: x = row-pair group j (I/16), y = active-expert slot,
// z = chunk of 16*NTT rows of the expert.
template <class F, int NTT>
__global__ __launch_bounds__(256) void k_gateup(DecodeArgs A) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = blockIdx.x;
    const int e = find_active_expert(A.offsets, A.rec, A.E, A.fmt, blockIdx.y, lane);
    if (e < 0) return;
    const int r0 = A.offsets[e];
    const int me = A.offsets[e + 1] - r0;
    const int c0 = blockIdx.z * 16 * NTT;
    if (c0 >= me) return;
    const int ridx = A.rec[e] & 0xffffff;
    const uint8_t* base = A.pool13 + (int64_t)ridx * A.stride13;
    const int64_t nkb = tiles_k<F>(A.H);
    const uint8_t* tg = base + (int64_t)(2 * j) * nkb * F::TB;
    const uint8_t* tu = tg + nkb * F::TB;
    const uint8_t* cbg = A.cb_gate + (int64_t)ridx * A.cb_stride;
    const uint8_t* cbu = A.cb_up + (int64_t)ridx * A.cb_stride;

    const _Float16* xrow[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        const int c = c0 + (lane & 15) + 16 * tt;
        xrow[tt] = c < me ? A.x16 + (int64_t)(A.perm_src[r0 + c] / A.k) * A.H : nullptr;
    }

    f32x4 accg[NTT], accu[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        accg[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        accu[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int64_t kb = wave; kb < nkb; kb += kWaves) {
        typename F::Frag fg, fu;
        F::load(fg, tg + kb * F::TB, lane);
        F::load(fu, tu + kb * F::TB, lane);
        f16x8 b[NTT][F::STEPS];
        load_b<F, NTT>(xrow, (int)(kb * F::TK) + (lane >> 4) * F::KSPAN, A.H, b);
        f16x8 a[F::STEPS];
        F::decode(fg, cbg, a);
#pragma unroll
        for (int s = 0; s < F::STEPS; ++s)
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) accg[tt] = mfma16(a[s], b[tt][s], accg[tt]);
        F::decode(fu, cbu, a);
#pragma unroll
        for (int s = 0; s < F::STEPS; ++s)
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) accu[tt] = mfma16(a[s], b[tt][s], accu[tt]);
    }

    __shared__ f32x4 red[kWaves][2][NTT][64];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        red[wave][0][tt][lane] = accg[tt];
        red[wave][1][tt][lane] = accu[tt];
    }
    __syncthreads();
    if (wave < NTT) {
        const int tt = wave;
        f32x4 g = red[0][0][tt][lane], u = red[0][1][tt][lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            g = g + red[w][0][tt][lane];
            u = u + red[w][1][tt][lane];
        }
        const int c = c0 + (lane & 15) + 16 * tt;
        if (c < me) {
            const int n0 = 16 * j + (lane >> 4) * 4;
            if constexpr (F::kVq) {
                // VQ: per-output-channel fp16 scales after the dot product
                const uint8_t* sc = base + (int64_t)(2 * (A.I / 16)) * nkb * F::TB;
                const _Float16* sg = reinterpret_cast<const _Float16*>(sc);
                const _Float16* su = sg + A.I;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    g[i] *= (float)sg[n0 + i];
                    u[i] *= (float)su[n0 + i];
                }
            }
            f16x4 h;
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = (_Float16)silu_mul(g[i], u[i]);
            *reinterpret_cast<f16x4*>(A.h16 + (int64_t)(r0 + c) * A.I + n0) = h;
        }
    }
}

// down.  grid: x = row group j (H/16), y = active-expert slot, z = row chunk.
template <class F, int NTT>
__global__ __launch_bounds__(256) void k_down(DecodeArgs A) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = blockIdx.x;
    const int e = find_active_expert(A.offsets, A.rec, A.E, A.fmt, blockIdx.y, lane);
    if (e < 0) return;
    const int r0 = A.offsets[e];
    const int me = A.offsets[e + 1] - r0;
    const int c0 = blockIdx.z * 16 * NTT;
    if (c0 >= me) return;
    const int ridx = A.rec[e] & 0xffffff;
    const uint8_t* base = A.pool2 + (int64_t)ridx * A.stride2;
    const int64_t nkb = tiles_k<F>(A.I);
    const uint8_t* tw = base + (int64_t)j * nkb * F::TB;
    const uint8_t* cbd = A.cb_down + (int64_t)ridx * A.cb_stride;

    const _Float16* xrow[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        const int c = c0 + (lane & 15) + 16 * tt;
        xrow[tt] = c < me ? A.h16 + (int64_t)(r0 + c) * A.I : nullptr;
    }
    f32x4 acc[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t kb = wave; kb < nkb; kb += kWaves) {
        typename F::Frag fw;
        F::load(fw, tw + kb * F::TB, lane);
        f16x8 b[NTT][F::STEPS];
        load_b<F, NTT>(xrow, (int)(kb * F::TK) + (lane >> 4) * F::KSPAN, A.I, b);
        f16x8 a[F::STEPS];
        F::decode(fw, cbd, a);
#pragma unroll
        for (int s = 0; s < F::STEPS; ++s)
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) acc[tt] = mfma16(a[s], b[tt][s], acc[tt]);
    }

    __shared__ f32x4 red[kWaves][NTT][64];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) red[wave][tt][lane] = acc[tt];
    __syncthreads();
    if (wave < NTT) {
        const int tt = wave;
        f32x4 y = red[0][tt][lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) y = y + red[w][tt][lane];
        const int c = c0 + (lane & 15) + 16 * tt;
        if (c < me) {
            const int n0 = 16 * j + (lane >> 4) * 4;
            if constexpr (F::kVq) {
                const _Float16* sd = reinterpret_cast<const _Float16*>(
                    base + (int64_t)(A.H / 16) * nkb * F::TB);
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] *= (float)sd[n0 + i];
            }
            *reinterpret_cast<f32x4*>(A.y_perm + (int64_t)(r0 + c) * A.H + n0) = y;
        }
    }
}

template <class F, int NTT>
int launch_fmt(const DecodeArgs& a, int slots, int chunks, int phase, hipStream_t s) {
    if (phase == 0) {
        dim3 grid((unsigned)(a.I / 16), (unsigned)slots, (unsigned)chunks);
        k_gateup<F, NTT><<<grid, 256, 0, s>>>(a);
    } else {
        dim3 grid((unsigned)(a.H / 16), (unsigned)slots, (unsigned)chunks);
        k_down<F, NTT><<<grid, 256, 0, s>>>(a);
    }
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

template <class F>
int launch_ntt(const DecodeArgs& a, int64_t T, int slots, int phase, hipStream_t s) {
    // an expert has at most T rows (the k experts of a token are distinct)
    if (T <= 16) return launch_fmt<F, 1>(a, slots, 1, phase, s);
    if (T <= 32) return launch_fmt<F, 2>(a, slots, 1, phase, s);
    const int chunks = (int)((T + 63) / 64);
    return launch_fmt<F, 4>(a, slots, chunks, phase, s);
}

}  // namespace

int launch_ffn_decode(const LayerView& L, int fmt, int n_fmt, const uint16_t* x16,
                      const int32_t* perm_src, const int32_t* offsets, int64_t T, int32_t k,
                      uint16_t* h16, float* y_perm, int phase, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    DecodeArgs a;
    a.pool13 = L.pool13[fmt];
    a.pool2 = L.pool2[fmt];
    a.stride13 = L.stride13[fmt];
    a.stride2 = L.stride2[fmt];
    a.cb_gate = L.cb[0];
    a.cb_up = L.cb[1];
    a.cb_down = L.cb[2];
    a.cb_stride = L.cb_stride;
    a.rec = L.rec;
    a.offsets = offsets;
    a.perm_src = perm_src;
    a.x16 = reinterpret_cast<const _Float16*>(x16);
    a.h16 = reinterpret_cast<_Float16*>(h16);
    a.y_perm = y_perm;
    a.E = L.E;
    a.H = L.H;
    a.I = L.I;
    a.k = k;
    a.fmt = fmt;
    const int64_t tk = T * k;
    const int slots = (int)(tk < n_fmt ? tk : n_fmt);
    if (slots == 0) return MOE_OK;
    if (fmt == MOE_FMT_NVFP4) return launch_ntt<NvFmt>(a, T, slots, phase, s);
    return launch_ntt<VqFmt>(a, T, slots, phase, s);
}

}  // namespace moeq
