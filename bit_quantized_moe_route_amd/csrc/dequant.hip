// Test hook: decode one projection of one expert from its device record to
// fp32 with the same decode routines as the FFN kernels.  NVFP4 and VQ values
// are exact (NVFP4: an E2M1 value times an E4M3 scale, exact in fp16; VQ: an
// fp16 codebook entry times an fp16 scale, exact in fp32), so the output can
// be compared bit for bit with a plain decode of the canonical bytes.  VQ8
// with one code per group is exact too; with two or three it is
// fp32(fp32(C_0 + .. + C_{m-1}) * S).  BF16 gives the kernels' fp16 operand: the
// stored weight rounded to fp16 (equal to it for |w| >= 2^-17).  Nested
// two-level NVFP4 gives fp32(base + residual * 2^-shift).
#include "dev_common.h"

namespace moeq {

namespace {

// one wave per tile; grid.x = row groups of the projection, grid.y = tiles
// along the input dimension
// res != 0 (MOE_FMT_NVFP4R): plus the residual plane res bytes further on
// times rscale, summed in fp32.
__global__ __launch_bounds__(64) void k_dequant_nv(const uint8_t* __restrict__ rec, int rg_step,
                                                   int rg_off, int n, int kin, int64_t res,
                                                   float rscale, float* __restrict__ out) {
    const int lane = threadIdx.x;
    const int g = blockIdx.x;
    const int kb = blockIdx.y;
    const int nkb = gridDim.y;
    const uint8_t* tile = rec + ((int64_t)(g * rg_step + rg_off) * nkb + kb) * kNvTileBytes;
    NvFrag f = nv_load(tile, lane);
    f16x8 a[4];
    nv_decode(f, a);
    float v[4][8];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[s][i] = (float)a[s][i];
    if (res) {
        NvFrag fr = nv_load(tile + res, lane);
        nv_decode(fr, a);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) v[s][i] += (float)a[s][i] * rscale;
    }
    const int row = 16 * g + (lane & 15);
    const int k0 = kb * kNvTileK + (lane >> 4) * 32;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int k = k0 + 8 * s + i;
            if (row < n && k < kin) out[(int64_t)row * kin + k] = v[s][i];
        }
}

__global__ __launch_bounds__(64) void k_dequant_vq(const uint8_t* __restrict__ rec, int rg_step,
                                                   int rg_off, int n, int kin,
                                                   const uint8_t* __restrict__ cb,
                                                   const _Float16* __restrict__ scales,
                                                   float* __restrict__ out) {
    const int lane = threadIdx.x;
    const int g = blockIdx.x;
    const int kb = blockIdx.y;
    const int nkb = gridDim.y;
    const uint8_t* tile = rec + ((int64_t)(g * rg_step + rg_off) * nkb + kb) * kVqTileBytes;
    u32x4 codes = *reinterpret_cast<const u32x4*>(tile + lane * 16);
    const int row = 16 * g + (lane & 15);
    const int k0 = kb * kVqTileK + (lane >> 4) * 64;
    const float sc = row < n ? (float)scales[row] : 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        uint32_t c = (codes[s >> 1] >> (16 * (s & 1))) & 0xffffu;
        f16x8 a = vq_row(cb, c);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int k = k0 + 8 * s + i;
            if (row < n && k < kin) out[(int64_t)row * kin + k] = sc * (float)a[i];
        }
    }
}

__global__ __launch_bounds__(64) void k_dequant_bf16(const uint8_t* __restrict__ rec,
                                                     int rg_step, int rg_off, int n, int kin,
                                                     float* __restrict__ out) {
    const int lane = threadIdx.x;
    const int g = blockIdx.x;
    const int kb = blockIdx.y;
    const int nkb = gridDim.y;
    const uint8_t* tile = rec + ((int64_t)(g * rg_step + rg_off) * nkb + kb) * kBf16TileBytes;
    const int row = 16 * g + (lane & 15);
    const int k0 = kb * kBf16TileK + (lane >> 4) * 32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f16x8 a =
            bf16x8_to_f16x8(*reinterpret_cast<const u32x4*>(tile + 1024 * j + lane * 16));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int k = k0 + 8 * j + i;
            if (row < n && k < kin) out[(int64_t)row * kin + k] = (float)a[i];
        }
    }
}

// VQ8: the M small codebooks of the projection, [M][256][8] fp16
template <int M>
__global__ __launch_bounds__(64) void k_dequant_vq8(const uint8_t* __restrict__ rec, int rg_step,
                                                    int rg_off, int n, int kin,
                                                    const uint8_t* __restrict__ cb,
                                                    const _Float16* __restrict__ scales,
                                                    float* __restrict__ out) {
    const int lane = threadIdx.x;
    const int g = blockIdx.x;
    const int kb = blockIdx.y;
    const int nkb = gridDim.y;
    const uint8_t* tile =
        rec + ((int64_t)(g * rg_step + rg_off) * nkb + kb) * (kVq8TileBytesPerCode * M);
    const uint8_t* lc = tile + lane * 8 * M;
    const int row = 16 * g + (lane & 15);
    const int k0 = kb * kVq8TileK + (lane >> 4) * 64;
    const float sc = row < n ? (float)scales[row] : 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const f16x8 a = vq_row(cb + m * (MOE_VQ8_NCODE * 16), lc[M * s + m]);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] += (float)a[i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int k = k0 + 8 * s + i;
            if (row < n && k < kin) out[(int64_t)row * kin + k] = sc * v[i];
        }
    }
}

}  // namespace

int launch_dequant(const LayerView& L, int fmt, int32_t ridx, int32_t proj, float* out,
                   void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool down = proj == MOE_PROJ_DOWN;
    const int n = down ? L.H : L.I;
    const int kin = down ? L.I : L.H;
    const int rg_step = down ? 1 : 2;
    const int rg_off = proj == MOE_PROJ_UP ? 1 : 0;
    const uint8_t* rec = down ? L.pool2[fmt] + (int64_t)ridx * L.stride2[fmt]
                              : L.pool13[fmt] + (int64_t)ridx * L.stride13[fmt];
    if (fmt == MOE_FMT_NVFP4 || fmt == MOE_FMT_NVFP4R) {
        dim3 grid((unsigned)(n / 16), (unsigned)nv_tiles_k(kin));
        const int64_t res = fmt == MOE_FMT_NVFP4 ? 0 : down ? L.res2 : L.res13;
        k_dequant_nv<<<grid, 64, 0, s>>>(rec, rg_step, rg_off, n, kin, res, L.res_scale, out);
    } else if (fmt == MOE_FMT_BF16) {
        dim3 grid((unsigned)(n / 16), (unsigned)bf16_tiles_k(kin));
        k_dequant_bf16<<<grid, 64, 0, s>>>(rec, rg_step, rg_off, n, kin, out);
    } else if (is_vq8(fmt)) {
        const int m = vq8_rate(fmt, L.vq8_m);
        const int64_t nkb = vq_tiles_k(kin);
        const int groups = down ? L.H / 16 : 2 * (L.I / 16);
        const int64_t tb = (int64_t)kVq8TileBytesPerCode * m;
        const _Float16* sc = reinterpret_cast<const _Float16*>(rec + (int64_t)groups * nkb * tb);
        if (proj == MOE_PROJ_UP) sc += L.I;
        dim3 grid((unsigned)(n / 16), (unsigned)nkb);
        if (m == 1)
            k_dequant_vq8<1><<<grid, 64, 0, s>>>(rec, rg_step, rg_off, n, kin, L.cb8[proj], sc, out);
        else if (m == 3)
            k_dequant_vq8<3><<<grid, 64, 0, s>>>(rec, rg_step, rg_off, n, kin, L.cb8[proj], sc, out);
        else
            k_dequant_vq8<2><<<grid, 64, 0, s>>>(rec, rg_step, rg_off, n, kin, L.cb8[proj], sc, out);
    } else {
        const int64_t nkb = vq_tiles_k(kin);
        const int groups = down ? L.H / 16 : 2 * (L.I / 16);
        const _Float16* sc = reinterpret_cast<const _Float16*>(rec + (int64_t)groups * nkb * kVqTileBytes);
        if (proj == MOE_PROJ_UP) sc += L.I;
        const uint8_t* cb = L.cb[proj] + (int64_t)ridx * L.cb_stride;
        dim3 grid((unsigned)(n / 16), (unsigned)nkb);
        k_dequant_vq<<<grid, 64, 0, s>>>(rec, rg_step, rg_off, n, kin, cb, sc, out);
    }
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

}  // namespace moeq
