// Expert FFN for small token batches (decode): a weight-streaming, skinny
// matrix-core product per active expert.
//
// For each active expert e (rows r0 .. r0+M_e of the permuted order):
//   gate/up kernel: g = W_gate x, u = W_up x, h = silu(g) * u  -> h (fp16)
//   down kernel:    y = W_down h                                -> y_perm (fp32)
// ("GLM-5-NVFP4-MTP", What's quantized: gate, up and down projections of the
// routed experts are the low-bit part.)
//
// Work decomposition (gfx950, wave64, 4 waves per workgroup):
//   * a wave owns one 16-row group of output channels (gate/up: 16 gate rows
//     and the 16 matching up rows) and a share of the input dimension: with
//     KS waves per row group, tile kb goes to wave kb % KS of the group; the
//     KS partial 16x16 fp32 tiles are summed through LDS in a fixed order;
//   * the wave streams its weight tiles from HBM straight into registers with
//     16-byte loads (one tile = 1 KB of codes per wave-wide load), keeping the
//     next tile's loads in flight while it decodes the current one to fp16
//     (exact) and feeds v_mfma_f32_16x16x32_f16: weights are the A operand,
//     up to 16 tokens of the expert the B operand (further tokens use further
//     B tiles; only the tiles the expert needs are computed);
//   * the B operand is read straight from the bf16 tokens x (gate/up; each
//     8-element fragment converted to fp16 in registers, exact for
//     2^-14 <= |x| <= 65504) or from the fp16 activations h (down).
#include <type_traits>

#include "rot_dev.h"
#include "topk_dev.h"

namespace moeq {

namespace {



// Per-format tile traits ----------------------------------------------------
struct NvFmt {
    static constexpr int PLANES = 1;
    static constexpr bool kVq = false;
    static constexpr bool kVq8 = false;
    static constexpr int TK = kNvTileK;       // inputs per tile
    static constexpr int TB = kNvTileBytes;   // bytes per tile
    static constexpr int STEPS = 4;           // MFMA K-steps per tile
    static constexpr int KSPAN = 32;          // inputs per lane per tile
    // The two scale bytes are held as the 16-bit value the load returns: a
    // 32-bit field makes the compiler zero-extend it right after the load,
    // inside the conditional prefetch, which waits for the prefetch to land.
    struct Frag {
        u32x4 codes;
        uint16_t scales;
    };
    __device__ __forceinline__ static void load(Frag& fr, const uint8_t* tile, int lane) {
        fr.codes = load_stream16(tile + lane * 16);
        fr.scales = *reinterpret_cast<const uint16_t*>(tile + kNvScaleOff + lane * 2);
    }
    __device__ __forceinline__ static void decode(const Frag& fr, const uint8_t*, f16x8 a[STEPS]) {
        NvFrag f{fr.codes, fr.scales};
        nv_decode(f, a);
    }
};

struct VqFmt {
    static constexpr int PLANES = 1;
    static constexpr bool kVq = true;
    static constexpr bool kVq8 = false;
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

// Small-codebook VQ: M uint8 codes per 8-weight group into M 256-entry fp16
// codebooks shared by the layer (rows summed).  The kernel's codebooks sit
// in LDS (M x 4 KB per projection), so a lookup is an LDS read, not an L2
// gather; each codebook's row is its own MFMA A fragment (the sum of the M
// exact products is taken in the fp32 accumulator; adding the fp16 rows
// first would round).  Per-row scales as for VQ.
template <int M>
struct Vq8Fmt {
    static constexpr int PLANES = 1;
    static constexpr bool kVq = true;
    static constexpr bool kVq8 = true;
    static constexpr int CODES = M;
    static constexpr int TK = kVq8TileK;
    static constexpr int TB = kVq8TileBytesPerCode * M;
    static constexpr int STEPS = 8;
    static constexpr int KSPAN = 64;
};

// BF16 weights as stored: a lane's 32 weights of a tile are four contiguous
// 1 KB slices' 16-byte chunks; each chunk converts to one fp16 A fragment
// (bf16 -> fp32 exact, fp32 -> fp16 nearest even: exact for
// 2^-17 <= |w| <= 65504, since a bf16 value has 8 significant bits).
struct Bf16Fmt {
    static constexpr int PLANES = 1;
    static constexpr bool kVq = false;
    static constexpr bool kVq8 = false;
    static constexpr int TK = kBf16TileK;
    static constexpr int TB = kBf16TileBytes;
    static constexpr int STEPS = 4;
    static constexpr int KSPAN = 32;
    struct Frag {
        u32x4 c[4];
    };
    __device__ __forceinline__ static void load(Frag& fr, const uint8_t* tile, int lane) {
#pragma unroll
        for (int j = 0; j < 4; ++j) fr.c[j] = load_stream16(tile + 1024 * j + lane * 16);
    }
    __device__ __forceinline__ static void decode(const Frag& fr, const uint8_t*, f16x8 a[STEPS]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = bf16x8_to_f16x8(fr.c[j]);
    }
};

// Nested two-level NVFP4 (MOE_FMT_NVFP4R): a tile of the base plane and the
// tile at the same place of the residual plane, poff bytes further on, whose
// scales are multiplied by the layer's power of two pscale; each plane's
// decoded fragment is its own MFMA A operand (both products exact, summed in
// the fp32 accumulator).  ("GLM-5.3 Vision NestQuant 1.75-4 bit",
// introduction: a base plus a residual plane that lifts it.)
struct Nv2Fmt : NvFmt {
    static constexpr int PLANES = 2;
    struct Frag {
        NvFmt::Frag p[2];
    };
    __device__ __forceinline__ static void load(Frag& fr, const uint8_t* tile, int lane,
                                                int64_t poff) {
        NvFmt::load(fr.p[0], tile, lane);
        NvFmt::load(fr.p[1], tile + poff, lane);
    }
    __device__ __forceinline__ static void decode2(const Frag& fr, f16x8 a0[STEPS],
                                                   f16x8 a1[STEPS], _Float16 ps) {
        NvFmt::decode(fr.p[0], nullptr, a0);
        f16x2 s0, s1;
        nv_scales(fr.p[1].scales, s0, s1);
        const f16x2 p2 = {ps, ps};
        s0 = s0 * p2;
        s1 = s1 * p2;
        a1[0] = nv_dequant8(fr.p[1].codes[0], s0);
        a1[1] = nv_dequant8(fr.p[1].codes[1], s0);
        a1[2] = nv_dequant8(fr.p[1].codes[2], s1);
        a1[3] = nv_dequant8(fr.p[1].codes[3], s1);
    }
};

template <class F>
__device__ __forceinline__ int tiles_k(int kin) {
    return (kin + F::TK - 1) / F::TK;
}

// 8 activations (raw 16-bit words) as fp16: bf16 bits converted (BF) or
// fp16 bits as they are.  Fragments are loaded raw and converted right
// before their MFMA, so a load in flight is never waited for early.
template <bool BF>
__device__ __forceinline__ f16x8 act_f16(u32x4 v) {
    if constexpr (BF)
        return bf16x8_to_f16x8(v);
    else
        return __builtin_bit_cast(f16x8, v);
}

// B operand fragments of one tile for the NTT token tiles: lane L holds
// token (L & 15) + 16 tt, inputs k0 + 8 s .. +7 with k0 = kb*TK + (L>>4)*KSPAN.
// Every lane loads, always from a valid address, so that no load sits on a
// branch (a load on a branch makes the compiler wait for all loads in flight
// before the next use, which defeats the prefetch): rows past the expert's
// rows come in as a valid row of it (xrow holds one; their output columns are
// never stored) and inputs past K as inputs K-8..K-1 of the row (the weights
// of those inputs are zero codes, so their products are zero).
template <class F, int NTT>
__device__ __forceinline__ void load_b(const uint16_t* const xrow[NTT], int k0, int K,
                                       u32x4 b[NTT][F::STEPS]) {
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
        for (int s = 0; s < F::STEPS; ++s) {
            const int kk = min(k0 + 8 * s, K - 8);
            b[tt][s] = *reinterpret_cast<const u32x4*>(xrow[tt] + kk);
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
    const uint8_t* cb8[3];   // VQ8 codebooks per projection, [M][256][8] fp16
    const int32_t* rec;
    const int32_t* offsets;
    const int32_t* perm_src;
    const uint16_t* xbf;   // tokens, bf16 bits [T, H]
    _Float16* h16;
    float* y_perm;
    int E, H, I, k, fmt;
    int rows;              // offsets == NULL: rows of the identity map
    int64_t res13, res2;   // MOE_FMT_NVFP4R: residual plane offset in a record
    float res_scale;       // ... and its decode factor
    int nsplit;            // PART kernels: workgroups splitting the input dimension
    float* part;           // PART kernels: fp32 [nsplit][rows][2I] partial g | u
    // small-batch fused layer (ROUTE gate/up, k_down_combine)
    const float* logits;   // fp32 [T, E]
    int32_t* topk_ids;     // [T, k]: written by the gate/up kernel, read by down
    float* topk_w;
    const float* y_shared; // NULL or fp32 [T, H], added after the routed sum
    float* out;            // fp32 [T, H]
    const uint8_t* rot;    // rotated layers: sign bits per expert (rot_stride bytes each)
    int64_t rot_stride;
};

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * u / (1.0f + expf(-g));
}

// Streams NM matrices' tiles (gate/up: NM = 2, down: NM = 1) of one 16-row
// group over tiles kb = kpart, kpart + KS, ... and accumulates
// acc[m][tt] += W_m[rows, tile] * B[tile, tokens of tile tt].
// The loads of the next D tiles stay in flight (a register ring of D + 1
// stages) while a tile is decoded and multiplied.
template <class F, int NTT, int NM, int D, bool BF>
__device__ __forceinline__ void stream_tiles(const uint8_t* const tbase[NM],
                                             const uint8_t* const cb[NM],
                                             const uint16_t* const xrow[NTT], int ntt, int K,
                                             int kpart, int KS, int lane,
                                             f32x4 acc[NM][NTT], int64_t poff = 0,
                                             float pscale = 1.f) {
    const int nkb = tiles_k<F>(K);
    const int ksub = (lane >> 4) * F::KSPAN;
    const int niter = kpart < nkb ? (nkb - kpart + KS - 1) / KS : 0;   // tiles of this wave
    if (niter == 0) return;
    typename F::Frag wr[D + 1][NM];
    u32x4 br[D + 1][NTT][F::STEPS];
    // the loads of tile i; past the last tile the last one is loaded again
    // (from the caches; never used), so that the prefetch is not on a branch
    auto issue = [&](int i, typename F::Frag (&w)[NM], u32x4 (&b)[NTT][F::STEPS]) {
        const int kb = kpart + min(i, niter - 1) * KS;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if constexpr (F::PLANES == 2)
                F::load(w[m], tbase[m] + (int64_t)kb * F::TB, lane, poff);
            else
                F::load(w[m], tbase[m] + (int64_t)kb * F::TB, lane);
        }
        load_b<F, NTT>(xrow, kb * F::TK + ksub, K, b);
    };
#pragma unroll
    for (int u = 0; u < D; ++u) issue(u, wr[u], br[u]);
    // the trip count rounded up to the unroll: every pass issues its loads,
    // only the decode and the products are skipped past the last tile
    const int nround = (niter + D) / (D + 1) * (D + 1);
    for (int it = 0; it < nround; it += D + 1) {
#pragma unroll
        for (int u = 0; u <= D; ++u) {
            const int i = it + u;
            issue(i + D, wr[(u + D) % (D + 1)], br[(u + D) % (D + 1)]);
            if (i >= niter) continue;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                if constexpr (F::PLANES == 2) {
                    f16x8 a0[F::STEPS], a1[F::STEPS];
                    F::decode2(wr[u][m], a0, a1, (_Float16)pscale);
#pragma unroll
                    for (int s = 0; s < F::STEPS; ++s)
#pragma unroll
                        for (int tt = 0; tt < NTT; ++tt)
                            if (tt < ntt) {
                                const f16x8 bb = act_f16<BF>(br[u][tt][s]);
                                acc[m][tt] = mfma16(a0[s], bb, acc[m][tt]);
                                acc[m][tt] = mfma16(a1[s], bb, acc[m][tt]);
                            }
                } else {
                    f16x8 a[F::STEPS];
                    F::decode(wr[u][m], cb[m], a);
#pragma unroll
                    for (int s = 0; s < F::STEPS; ++s)
#pragma unroll
                        for (int tt = 0; tt < NTT; ++tt)
                            if (tt < ntt)
                                acc[m][tt] = mfma16(a[s], act_f16<BF>(br[u][tt][s]), acc[m][tt]);
                }
            }
        }
    }
}

// VQ tiles.  Every 16-byte codebook row a tile needs is a gather whose
// address comes from the tile's codes, and each gathered row is one MFMA A
// fragment.  All NM x 8 gathers of a tile (and its activation fragments) are
// issued before the tile's first MFMA, and the next tile's codes are loaded
// behind them, so a wave keeps NM * 8 gathers in flight.  The scheduling
// barrier stops the compiler from moving each gather next to its MFMA, which
// leaves one gather in flight per wave and a full wait per MFMA.
// Lanes of tokens past the expert's rows read the row `xsafe` (their output
// columns are never stored); inputs past K are zero.
#ifndef MOEQ_VQ_CODES_AHEAD
#define MOEQ_VQ_CODES_AHEAD 1
#endif
constexpr int kVqCodesAhead = MOEQ_VQ_CODES_AHEAD;

template <int NTT, int NM, bool BF>
__device__ __forceinline__ void stream_tiles_vq(const uint8_t* const tbase[NM],
                                                const uint8_t* const cb[NM],
                                                const uint16_t* const xrow[NTT],
                                                const uint16_t* xsafe, int ntt, int K, int kpart,
                                                int KS, int lane, f32x4 acc[NM][NTT]) {
    using F = VqFmt;
    const int nkb = tiles_k<F>(K);
    const int ksub = (lane >> 4) * F::KSPAN;
    const int niter = kpart < nkb ? (nkb - kpart + KS - 1) / KS : 0;
    if (niter == 0) return;
    const uint16_t* xr[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) xr[tt] = xrow[tt] != nullptr ? xrow[tt] : xsafe;
    // codes of tiles i .. i + kVqCodesAhead (HBM latency is longer than a
    // tile's gather round trip)
    u32x4 codes[NM], ahead[kVqCodesAhead][NM];
#pragma unroll
    for (int m = 0; m < NM; ++m)
        codes[m] = load_stream16(tbase[m] + (int64_t)kpart * F::TB + lane * 16);
#pragma unroll
    for (int d = 0; d < kVqCodesAhead; ++d)
        if (d + 1 < niter) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
                ahead[d][m] =
                    load_stream16(tbase[m] + (int64_t)(kpart + (d + 1) * KS) * F::TB + lane * 16);
        }
    for (int i = 0; i < niter; ++i) {
        const int kb = kpart + i * KS;
        const int k0 = kb * F::TK + ksub;
        f16x8 a[NM][F::STEPS];
        u32x4 b[NTT][F::STEPS];
#pragma unroll
        for (int s = 0; s < F::STEPS; ++s) {
            const int kk = k0 + 8 * s;
            const int kc = kk < K ? kk : K - 8;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
                if (tt < ntt) b[tt][s] = *reinterpret_cast<const u32x4*>(xr[tt] + kc);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const uint32_t c = (codes[m][s >> 1] >> (16 * (s & 1))) & 0xffffu;
                a[m][s] = vq_row(cb[m], c);
            }
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            codes[m] = ahead[0][m];
#pragma unroll
            for (int d = 0; d + 1 < kVqCodesAhead; ++d) ahead[d][m] = ahead[d + 1][m];
        }
        if (i + 1 + kVqCodesAhead < niter) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
                ahead[kVqCodesAhead - 1][m] = load_stream16(
                    tbase[m] + (int64_t)(kb + (1 + kVqCodesAhead) * KS) * F::TB + lane * 16);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < F::STEPS; ++s) {
            const bool kin = k0 + 8 * s < K;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                if (tt >= ntt) break;
                const f16x8 bb = kin ? act_f16<BF>(b[tt][s]) : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
                for (int m = 0; m < NM; ++m) acc[m][tt] = mfma16(a[m][s], bb, acc[m][tt]);
            }
        }
    }
}

// VQ8 tiles: codes (8M bytes per lane per tile) stream from HBM with the
// next tile's codes and activations in flight (as stream_tiles); lcb[m] is
// the LDS copy of matrix m's codebooks ([M][256][8] fp16).
template <int NTT, int NM, int M, bool BF>
__device__ __forceinline__ void stream_tiles_vq8(const uint8_t* const tbase[NM],
                                                 const _Float16* const lcb[NM],
                                                 const uint16_t* const xrow[NTT], int ntt,
                                                 int K, int kpart, int KS, int lane,
                                                 f32x4 acc[NM][NTT]) {
    using F = Vq8Fmt<M>;
    constexpr int CW = 2 * M;   // code dwords per lane per tile
    const int nkb = tiles_k<F>(K);
    const int ksub = (lane >> 4) * F::KSPAN;
    const int niter = kpart < nkb ? (nkb - kpart + KS - 1) / KS : 0;
    uint32_t cw[2][NM][CW];
    u32x4 br[2][NTT][F::STEPS];
    auto issue = [&](int i, uint32_t (&c)[NM][CW], u32x4 (&b)[NTT][F::STEPS]) {
        const int kb = kpart + i * KS;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const uint8_t* p = tbase[m] + (int64_t)kb * F::TB + lane * 8 * M;
            if constexpr (M == 1 || M == 3) {
                // 8 bytes per load (3 codes per group: 24 bytes, 8-byte aligned)
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
                for (int q = 0; q < M; ++q) {
                    const u32x2 v =
                        __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p + 8 * q));
                    c[m][2 * q] = v[0];
                    c[m][2 * q + 1] = v[1];
                }
            } else {
                const u32x4 v = load_stream16(p);
#pragma unroll
                for (int q = 0; q < 4; ++q) c[m][q] = v[q];
            }
        }
        load_b<F, NTT>(xrow, kb * F::TK + ksub, K, b);
    };
    if (niter == 0) return;
    issue(0, cw[0], br[0]);
    // the trip count rounded up to the unroll; past the last tile the last
    // one is loaded again (never used): no load on a branch
    const int nround = (niter + 1) / 2 * 2;
    for (int it = 0; it < nround; it += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = it + u;
            issue(min(i + 1, niter - 1), cw[u ^ 1], br[u ^ 1]);
            if (i >= niter) continue;
            {
                // the tile holding the end of K: its groups past K carry zero
                // codes, which still select a codebook row, so their
                // activations are zeroed here (after the wait, not at the load)
                const int kb = kpart + i * KS;
                if (kb * F::TK + F::TK > K) {
                    const int k0 = kb * F::TK + ksub;
#pragma unroll
                    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                        for (int s = 0; s < F::STEPS; ++s)
                            if (k0 + 8 * s >= K) br[u][tt][s] = u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int s = 0; s < F::STEPS; ++s)
#pragma unroll
                    for (int j = 0; j < M; ++j) {
                        const int byte = M * s + j;
                        const uint32_t code = (cw[u][m][byte >> 2] >> (8 * (byte & 3))) & 0xffu;
                        const f16x8 a = *reinterpret_cast<const f16x8*>(
                            lcb[m] + (j * MOE_VQ8_NCODE + code) * 8);
#pragma unroll
                        for (int tt = 0; tt < NTT; ++tt)
                            if (tt < ntt)
                                acc[m][tt] = mfma16(a, act_f16<BF>(br[u][tt][s]), acc[m][tt]);
                    }
        }
    }
}

#ifndef MOEQ_VQ_GATHER_AHEAD
#define MOEQ_VQ_GATHER_AHEAD 1
#endif

// Row groups per wave: gate/up 2 row-pair groups (4 weight tiles per input
// tile), down 4 row groups.
constexpr int kRpwGateup = 2;
constexpr int kRpwDown = 4;
// Tiles kept in flight ahead of the one being used.
#ifndef MOEQ_PREFETCH
#define MOEQ_PREFETCH 1
#endif
constexpr int kPrefetch = MOEQ_PREFETCH;
// ... for the one expert of a shared-expert layer, whose waves have only a
// few tiles each (the whole expert is spread over the chip).  (Measured: 2
// and 3 are no faster at one token and spill at 32.)
#ifndef MOEQ_SH_PREFETCH
#define MOEQ_SH_PREFETCH 1
#endif
constexpr int kPrefetchShared = MOEQ_SH_PREFETCH;
// ... for the routed gate/up kernel of the small-batch fused layer.
#ifndef MOEQ_ROUTE_PREFETCH
#define MOEQ_ROUTE_PREFETCH 1
#endif
constexpr int kPrefetchRoute = MOEQ_ROUTE_PREFETCH;
// Waves per SIMD the register budget is sized for (latency hiding).
#ifndef MOEQ_MIN_WAVES
#define MOEQ_MIN_WAVES 2
#endif
constexpr int kMinWaves = MOEQ_MIN_WAVES;

// Dynamic LDS of the small-codebook VQ kernels: the codebooks of the
// projections a pass reads (gate and up, or down).
template <class F>
constexpr size_t codebook_lds_bytes(int phase) {
    if constexpr (F::kVq8)
        return (size_t)(phase == 0 ? 2 : 1) * F::CODES * MOE_VQ8_NCODE * 16;
    else
        return 0;
}

// One kernel for both halves.  PHASE 0 (gate/up + SwiGLU): a wave owns RPW
// row-pair groups (RPW gate tiles and RPW up tiles per input tile); PHASE 1
// (down): a wave owns RPW row groups of W_down.  KS waves split the input
// dimension of the same rows.  The B fragments (activations) are loaded once
// per input tile and used for all 2*RPW (or RPW) weight tiles of the wave.
// grid: x = sets of (4/KS) waves' rows, y = active-expert slot, z = chunk of
// 16*NTT rows of the expert.
// ID: offsets / perm_src are the identity map of a one-expert layer (a
// shared expert: its rows are the tokens).  PART (gate/up only): the input
// dimension is also split over A.nsplit workgroups (blockIdx.x % nsplit),
// which write fp32 partial g and u to A.part instead of h; k_swiglu_parts
// sums them and applies SwiGLU.  (One expert alone has too few row groups to
// fill the chip.)  ROT (gate/up of a rotated layer, with PART and nsplit = 1):
// the B operand is the fp16 rotated row of each assignment (A.xbf points to
// [rows, H] in permuted order) and the raw products go to A.part.
// ROUTE (gate/up of the small-batch fused layer): blockIdx.y is assignment
// a = t*k + j; each wave takes token t's top-k from the logits itself, the
// expert of rank j is its one "row", and h goes to row a (token order, no
// permutation); one workgroup per token writes the token's ids and weights.
// Single-format layers only (the record index of expert e is e).  ROUTE with
// ROT (and PART): the workgroup first rotates its assignment's x row into
// LDS (after the codebooks), the B operand is read from there, and the raw
// products go to A.part row a.
// ADDOUT (down of a shared expert): y is added to A.out (the routed sum
// already there) instead of being stored to A.y_perm.
// The body is a device function of the workgroup's grid coordinates bid, so
// that one launch can run it beside another kernel's workgroups.
template <class F, int NTT, int KS, int RPW, int PHASE, int WV, bool ID, bool PART, bool ROT,
          bool ROUTE, bool ADDOUT = false>
__device__ __forceinline__ void ffn_body(const DecodeArgs& A, const uint3 bid) {
    static_assert(!ROT || (PART && PHASE == 0 && !ID), "rotated gate/up writes raw products");
    static_assert(!ROUTE || (PHASE == 0 && !ID && PART == ROT), "routed gate/up only");
    static_assert(!ADDOUT || (PHASE == 1 && ID), "the down pass of a shared expert");
    constexpr bool XBF = PHASE == 0 && !ROT;        // B operand is bf16
    constexpr int NM = PHASE == 0 ? 2 * RPW : RPW;   // weight tiles per input tile
    constexpr int SETS = WV / KS;                    // row sets per workgroup
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    ActiveExpert ae;
    if constexpr (ROUTE) {
        const int a = bid.y;
        const int t = a / A.k, j = a % A.k;
        float top_v[MOE_MAX_K];
        int top_i[MOE_MAX_K];
        topk_select<4>(A.logits + (int64_t)t * A.E, A.E, A.k, lane, top_v, top_i);
        int e = top_i[0];
#pragma unroll
        for (int jj = 1; jj < MOE_MAX_K; ++jj)
            if (jj == j) e = top_i[jj];
        if (j == 0 && bid.x == 0 && wave == 0 && lane == 0) {
            float w[MOE_MAX_K];
            topk_weights(top_v, A.k, w);
#pragma unroll
            for (int jj = 0; jj < MOE_MAX_K; ++jj)
                if (jj < A.k) {
                    A.topk_ids[(int64_t)t * A.k + jj] = top_i[jj];
                    A.topk_w[(int64_t)t * A.k + jj] = w[jj];
                }
        }
        ae = ActiveExpert{e, a, 1, e};
    } else {
        ae = ID ? ActiveExpert{bid.y == 0 ? 0 : -1, 0, A.rows, 0}
                : find_active_expert(A.offsets, A.rec, A.E, A.fmt, bid.y, lane);
    }
    if (ae.e < 0) return;
    const int c0 = bid.z * 16 * NTT;
    if (c0 >= ae.me) return;
    const int ntt = min(NTT, (ae.me - c0 + 15) / 16);
    // VQ8: the codebooks of this kernel's projections into LDS (dynamic LDS:
    // gate and up for PHASE 0, down for PHASE 1)
    extern __shared__ _Float16 lds_cb[];
    if constexpr (F::kVq8) {
        constexpr int NP = PHASE == 0 ? 2 : 1;
        constexpr int CHUNKS = F::CODES * MOE_VQ8_NCODE;   // 16-byte rows per projection
        for (int i = threadIdx.x; i < NP * CHUNKS; i += 64 * WV) {
            const int pj = i / CHUNKS;
            const uint8_t* src = A.cb8[PHASE == 0 ? pj : 2] + (int64_t)(i % CHUNKS) * 16;
            *reinterpret_cast<u32x4*>(lds_cb + (int64_t)i * 8) =
                *reinterpret_cast<const u32x4*>(src);
        }
        __syncthreads();
    }
    if constexpr (ROUTE && ROT) {
        // the rotated row of this assignment, x' = H (s_in13[e] * x_t) / 16 in
        // fp16, into LDS after the codebooks: the separate rotation pass's
        // arithmetic (the same bits), 256-element spans per wave, lane L
        // holding elements 4L .. 4L+3 (the upper half-wave idle in a half span)
        // The loads of up to 8 spans per wave are issued before the first is
        // transformed (from clamped addresses: a lane outside the row reads
        // the lower half-wave's elements, which it never stores).
        constexpr int UB = 8;
        _Float16* xs = lds_cb + codebook_lds_bytes<F>(0) / 2;
        const uint16_t* xt = A.xbf + (int64_t)(ae.r0 / A.k) * A.H + 4 * lane;
        const uint8_t* s_in = A.rot + (int64_t)ae.e * A.rot_stride;
        const int nspan = (A.H + 255) / 256;
        const bool half = A.H % 256 != 0;
        for (int sp0 = wave; sp0 < nspan; sp0 += WV * UB) {
            uint2 raw[UB];
            uint32_t sb[UB];
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const int sp = min(sp0 + WV * u, nspan - 1);
                const bool in = !half || sp + 1 < nspan || lane < 32;
                raw[u] = *reinterpret_cast<const uint2*>(xt + 256 * sp - (in ? 0 : 128));
                sb[u] = *sign_byte(s_in, sp, in ? lane : lane - 32);
            }
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const int sp = sp0 + WV * u;
                if (sp >= nspan) break;
                const bool in = !half || sp + 1 < nspan || lane < 32;
                f32x4 v = bf16x4_to_f32(raw[u]) *
                          signs_of(in ? sb[u] >> (4 * (lane & 1)) : 0u);
                fwht128(v, lane);
                if (in)
                    *reinterpret_cast<f16x4*>(xs + 256 * sp + 4 * lane) = to_f16x4(v, 0.0625f);
            }
        }
        __syncthreads();
    }
    const int kloc = wave % KS;                      // part of the workgroup's inputs
    const int split = PART ? (int)bid.x % A.nsplit : 0;
    const int set = (PART ? (int)bid.x / A.nsplit : (int)bid.x) * SETS + wave / KS;
    const int kpart = split * KS + kloc;             // first input tile of this wave
    const int kstride = PART ? KS * A.nsplit : KS;   // ... and the stride between its tiles
    const int K = PHASE == 0 ? A.H : A.I;
    const int nrg = (PHASE == 0 ? A.I : A.H) / 16;   // row (pair) groups
    const int g0 = set * RPW;                        // first row (pair) group
    const int nlive = min(RPW, nrg - g0);            // groups of this wave in range
    const int nkb = tiles_k<F>(K);
    const uint8_t* base = PHASE == 0 ? A.pool13 + (int64_t)ae.ridx * A.stride13
                                     : A.pool2 + (int64_t)ae.ridx * A.stride2;
    const uint8_t* tb[NM];
    const uint8_t* cb[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        // gate/up records interleave row groups: 2j = gate, 2j+1 = up
        const int g = PHASE == 0 ? 2 * min(g0 + m / 2, nrg - 1) + (m & 1) : min(g0 + m, nrg - 1);
        tb[m] = base + (int64_t)g * nkb * F::TB;
        cb[m] = PHASE == 0 ? ((m & 1) ? A.cb_up : A.cb_gate) + (int64_t)ae.ridx * A.cb_stride
                           : A.cb_down + (int64_t)ae.ridx * A.cb_stride;
    }

    // B rows of the lanes' tokens; a lane past the expert's rows takes row c0
    // (its output column is never stored)
    const uint16_t* xrow[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        const int c0l = c0 + (lane & 15) + 16 * tt;
        const int c = c0l < ae.me ? c0l : c0;
        if (ROUTE && ROT)   // the assignment's rotated row in LDS (every column)
            xrow[tt] = reinterpret_cast<const uint16_t*>(lds_cb + codebook_lds_bytes<F>(0) / 2);
        else if (F::kVq && !F::kVq8 && c0l >= ae.me)
            xrow[tt] = nullptr;     // 16-bit VQ: stream_tiles_vq substitutes its safe row
        else if (PHASE == 0)
            xrow[tt] = A.xbf + (int64_t)(ROT     ? ae.r0 + c
                                         : ROUTE ? ae.r0 / A.k
                                         : ID    ? c
                                                 : A.perm_src[ae.r0 + c] / A.k) * A.H;
        else
            xrow[tt] = reinterpret_cast<const uint16_t*>(A.h16) + (int64_t)(ae.r0 + c) * A.I;
    }
    f32x4 acc[NM][NTT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[m][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nlive > 0) {
        if constexpr (F::kVq8) {
            const _Float16* lcb[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m)
                lcb[m] = lds_cb + (PHASE == 0 ? (m & 1) : 0) * (F::CODES * MOE_VQ8_NCODE * 8);
            stream_tiles_vq8<NTT, NM, F::CODES, XBF>(tb, lcb, xrow, ntt, K, kpart, kstride, lane,
                                                     acc);
        } else if constexpr (F::kVq && MOEQ_VQ_GATHER_AHEAD) {
            // row c0 of the expert exists: a safe row for lanes past its rows
            const uint16_t* xsafe =
                ROUTE && ROT ? xrow[0]
                : PHASE == 0
                    ? A.xbf + (int64_t)(ROT     ? ae.r0 + c0
                                        : ROUTE ? ae.r0 / A.k
                                        : ID    ? c0
                                                : A.perm_src[ae.r0 + c0] / A.k) * A.H
                    : reinterpret_cast<const uint16_t*>(A.h16) + (int64_t)(ae.r0 + c0) * A.I;
            stream_tiles_vq<NTT, NM, XBF>(tb, cb, xrow, xsafe, ntt, K, kpart, kstride, lane, acc);
        } else {
            stream_tiles<F, NTT, NM, ID ? kPrefetchShared : ROUTE ? kPrefetchRoute : kPrefetch, XBF>(
                tb, cb, xrow, ntt, K, kpart, kstride, lane, acc, PHASE == 0 ? A.res13 : A.res2,
                A.res_scale);
        }
    }

    if constexpr (KS > 1) {
        // sum the KS partial tiles of a row set in a fixed order (wave order)
        __shared__ f32x4 red[WV][NM][64];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            if (tt >= ntt) break;
            __syncthreads();
#pragma unroll
            for (int m = 0; m < NM; ++m) red[wave][m][lane] = acc[m][tt];
            __syncthreads();
            if (kloc == 0) {
#pragma unroll
                for (int w = 1; w < KS; ++w)
#pragma unroll
                    for (int m = 0; m < NM; ++m) acc[m][tt] = acc[m][tt] + red[wave + w][m][lane];
            }
        }
        if (kloc != 0) return;
    }
    const int r4 = (lane >> 4) * 4;
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
        if (q >= nlive) break;
        const int n0 = 16 * (g0 + q) + r4;            // first output channel of this lane
        if constexpr (PHASE == 0) {
            float sg[4] = {1.f, 1.f, 1.f, 1.f}, su[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (F::kVq) {
                // VQ: per-output-channel fp16 scales, applied after the dot product
                const _Float16* sp =
                    reinterpret_cast<const _Float16*>(base + (int64_t)(2 * nrg) * nkb * F::TB);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sg[i] = (float)sp[n0 + i];
                    su[i] = (float)sp[A.I + n0 + i];
                }
            }
            if constexpr (PART) {
                // fp32 partial sums of this workgroup's inputs: g at [.., n],
                // u at [.., I + n] of row (split, r0 + c)
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) {
                    const int c = c0 + (lane & 15) + 16 * tt;
                    if (tt < ntt && c < ae.me) {
                        f32x4 g, u;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            g[i] = acc[2 * q][tt][i] * sg[i];
                            u[i] = acc[2 * q + 1][tt][i] * su[i];
                        }
                        float* pp =
                            A.part + ((int64_t)split * A.rows + ae.r0 + c) * (2 * A.I) + n0;
                        *reinterpret_cast<f32x4*>(pp) = g;
                        *reinterpret_cast<f32x4*>(pp + A.I) = u;
                    }
                }
                continue;
            }
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                const int c = c0 + (lane & 15) + 16 * tt;
                if (tt < ntt && c < ae.me) {
                    f16x4 h;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        h[i] = (_Float16)silu_mul(acc[2 * q][tt][i] * sg[i],
                                                  acc[2 * q + 1][tt][i] * su[i]);
                    *reinterpret_cast<f16x4*>(A.h16 + (int64_t)(ae.r0 + c) * A.I + n0) = h;
                }
            }
        } else {
            float sd[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (F::kVq) {
                const _Float16* sp =
                    reinterpret_cast<const _Float16*>(base + (int64_t)nrg * nkb * F::TB);
#pragma unroll
                for (int i = 0; i < 4; ++i) sd[i] = (float)sp[n0 + i];
            }
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                const int c = c0 + (lane & 15) + 16 * tt;
                if (tt < ntt && c < ae.me) {
                    f32x4 y = acc[q][tt];
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[i] *= sd[i];
                    if constexpr (ADDOUT) {
                        // the combine's last addition: out = routed sum + y
                        float* op = A.out + (int64_t)(ae.r0 + c) * A.H + n0;
                        const f32x4 o = *reinterpret_cast<const f32x4*>(op);
#pragma unroll
                        for (int i = 0; i < 4; ++i) y[i] = __fadd_rn(o[i], y[i]);
                        *reinterpret_cast<f32x4*>(op) = y;
                    } else {
                        *reinterpret_cast<f32x4*>(A.y_perm + (int64_t)(ae.r0 + c) * A.H + n0) = y;
                    }
                }
            }
        }
    }
}


template <class F, int NTT, int KS, int RPW, int PHASE, int WV, bool ID, bool PART = false,
          bool ROT = false, bool ROUTE = false>
__global__ __launch_bounds__(64 * WV, kMinWaves) void k_ffn(DecodeArgs A) {
    ffn_body<F, NTT, KS, RPW, PHASE, WV, ID, PART, ROT, ROUTE>(
        A, uint3{blockIdx.x, blockIdx.y, blockIdx.z});
}

// h[c, n..n+3] = silu(g) * u with g, u the sums over the nsplit partials in
// ascending split order (one thread per 4 channels of a row).
__device__ __forceinline__ void swiglu_parts_body(const float* __restrict__ part, int nsplit,
                                                  int rows, int I, _Float16* __restrict__ h16,
                                                  const int64_t i) {
    const int nq = I / 4;
    if (i >= (int64_t)rows * nq) return;
    const int c = (int)(i / nq);
    const int n = (int)(i % nq) * 4;
    f32x4 g = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < nsplit; ++sp) {
        const float* pp = part + ((int64_t)sp * rows + c) * (2 * I) + n;
        g = g + *reinterpret_cast<const f32x4*>(pp);
        u = u + *reinterpret_cast<const f32x4*>(pp + I);
    }
    f16x4 h;
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q] = (_Float16)silu_mul(g[q], u[q]);
    *reinterpret_cast<f16x4*>(h16 + (int64_t)c * I + n) = h;
}

__global__ __launch_bounds__(256) void k_swiglu_parts(const float* __restrict__ part, int nsplit,
                                                      int rows, int I, _Float16* __restrict__ h16) {
    swiglu_parts_body(part, nsplit, rows, I, h16, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// Down projection and gated combine of the small-batch fused layer, for one
// token t (blockIdx.y) and one 16-row group g of the output (blockIdx.x):
//   out[t, rows of g] = sum_{j<k} w[t, j] * (W_down[e_j] h[t*k + j])[rows of g]
//                       (+ y_shared[t, rows of g])
// in ascending j in fp32, e_j / w[t, j] as the routed gate/up kernel wrote
// them.  Wave (sg, kloc) = (slot group, input part): it streams the tiles
// kloc, kloc + 4, ... of W_down[e_j] for the NSL slots j of group sg, with
// the h rows of those slots as the B operand's columns (column m = slot
// NSL sg + m, so one B load serves every slot and column m of the m-th
// product is the wanted one).  The 4 input parts are summed through LDS in
// wave order and wave 0 takes the weighted sum over the slots, so each y_j
// and the sum are the bits of the unfused down kernel and combine for the
// same batch.  (Fixed combine order: "GLM-5.3-Flash-TR3-8bpw (K8)", Fidelity.)
// NSL = 8 (NVFP4, VQ8: one group of 4-wave workgroups, two per CU) or 4
// (BF16 and 16-bit VQ, whose A fragments take more registers: NG groups).
constexpr int kDcKS = 4;     // waves splitting the input dimension of a slot group
constexpr int kDcMaxK = 8;   // k of the fused path
// SLOTS: each slot's output rows y'[t*k + j] go to y_perm (a rotated layer:
// the combine rotates them back per slot) instead of the weighted sum.
template <class F, int NSL, int NG, bool SLOTS = false>
__device__ __forceinline__ void down_combine_body(const DecodeArgs& A, const uint3 bid) {
    constexpr int KS = kDcKS, NM = NSL, WV = KS * NG;
    static_assert(NSL * NG <= 16, "slots are B columns");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kloc = wave % KS;
    const int sg = wave / KS;
    const int t = bid.y;
    const int g = bid.x;
    extern __shared__ _Float16 lds_cb[];
    if constexpr (F::kVq8) {
        constexpr int CHUNKS = F::CODES * MOE_VQ8_NCODE;
        for (int i = threadIdx.x; i < CHUNKS; i += 64 * WV)
            *reinterpret_cast<u32x4*>(lds_cb + (int64_t)i * 8) =
                *reinterpret_cast<const u32x4*>(A.cb8[2] + (int64_t)i * 16);
        __syncthreads();
    }
    const int K = A.I;
    const int nrg = A.H / 16;
    const int nkb = tiles_k<F>(K);
    const int j0 = sg * NM;                        // first slot of the group
    const int nsl = min(NM, A.k - j0);             // its live slots (>= 1)
    const int32_t* ids = A.topk_ids + (int64_t)t * A.k;
    // the gate weights, loaded now for the epilogue (uniform: scalar loads)
    float wts[kDcMaxK];
#pragma unroll
    for (int j = 0; j < kDcMaxK; ++j) wts[j] = j < A.k ? A.topk_w[(int64_t)t * A.k + j] : 0.f;
    const uint8_t* tb[NM];
    const uint8_t* cb[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        // slots past k repeat the last live one (same addresses: no new HBM bytes)
        const int e = ids[j0 + min(m, nsl - 1)];
        tb[m] = A.pool2 + (int64_t)e * A.stride2 + (int64_t)g * nkb * F::TB;
        cb[m] = A.cb_down + (int64_t)e * A.cb_stride;
    }
    const int col = lane & 15;                     // B column = slot j0 + col
    // columns past the live slots read the last live slot's h row (those
    // columns are never part of the sum)
    const uint16_t* xrow[1];
    if constexpr (F::kVq && !F::kVq8) {
        // 16-bit VQ: stream_tiles_vq substitutes its safe row for NULL
        xrow[0] = col < nsl ? reinterpret_cast<const uint16_t*>(A.h16) +
                                  ((int64_t)t * A.k + j0 + col) * A.I
                            : nullptr;
    } else {
        const int cs = col < nsl ? col : nsl - 1;
        xrow[0] = reinterpret_cast<const uint16_t*>(A.h16) + ((int64_t)t * A.k + j0 + cs) * A.I;
    }
    f32x4 acc[NM][1];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (F::kVq8) {
        const _Float16* lcb[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) lcb[m] = lds_cb;
        stream_tiles_vq8<1, NM, F::CODES, false>(tb, lcb, xrow, 1, K, kloc, KS, lane, acc);
    } else if constexpr (F::kVq && MOEQ_VQ_GATHER_AHEAD) {
        const uint16_t* xsafe =
            reinterpret_cast<const uint16_t*>(A.h16) + ((int64_t)t * A.k + j0) * A.I;
        stream_tiles_vq<1, NM, false>(tb, cb, xrow, xsafe, 1, K, kloc, KS, lane, acc);
    } else {
        stream_tiles<F, 1, NM, kPrefetch, false>(tb, cb, xrow, 1, K, kloc, KS, lane, acc, A.res2,
                                                 A.res_scale);
    }
    // the KS input parts of each slot group, summed in wave order
    __shared__ f32x4 red[WV][NM][64];
    __shared__ f32x4 ys[NG][64];
#pragma unroll
    for (int m = 0; m < NM; ++m) red[wave][m][lane] = acc[m][0];
    __syncthreads();
    if (kloc == 0) {
#pragma unroll
        for (int w = 1; w < KS; ++w)
#pragma unroll
            for (int m = 0; m < NM; ++m) acc[m][0] = acc[m][0] + red[wave + w][m][lane];
        // this lane's slot: column col of product col
        f32x4 y = acc[0][0];
#pragma unroll
        for (int m = 1; m < NM; ++m)
            if (col == m) y = acc[m][0];
        if constexpr (F::kVq) {
            // per-output-channel scales of the slot's expert
            const int e = ids[j0 + min(col, nsl - 1)];
            const _Float16* sp = reinterpret_cast<const _Float16*>(
                A.pool2 + (int64_t)e * A.stride2 + (int64_t)nrg * nkb * F::TB);
            const int n0 = 16 * g + (lane >> 4) * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] *= (float)sp[n0 + i];
        }
        if constexpr (SLOTS) {
            if (col < nsl)
                *reinterpret_cast<f32x4*>(A.y_perm + ((int64_t)t * A.k + j0 + col) * A.H +
                                          16 * g + (lane >> 4) * 4) = y;
        } else {
            ys[sg][lane] = y;
        }
    }
    if constexpr (SLOTS) return;
    __syncthreads();
    if (wave != 0) return;
    // lane 16q + c of ys[sg] holds rows 4q .. 4q+3 of the group for slot NSL sg + c
    const int q16 = lane & 48;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kDcMaxK; ++j) {
        if (j >= A.k) break;
        const f32x4 y = ys[j / NM][q16 + j % NM];
        o = o + wts[j] * y;
    }
    if (col != 0) return;
    const int64_t n = (int64_t)t * A.H + 16 * g + (lane >> 4) * 4;
    if (A.y_shared) o = o + *reinterpret_cast<const f32x4*>(A.y_shared + n);
    *reinterpret_cast<f32x4*>(A.out + n) = o;
}

template <class F, int NSL, int NG, bool SLOTS = false>
__global__ __launch_bounds__(64 * kDcKS * NG, kMinWaves) void k_down_combine(DecodeArgs A) {
    down_combine_body<F, NSL, NG, SLOTS>(A, uint3{blockIdx.x, blockIdx.y, 0u});
}

template <class F, int NTT, int KS, int WV>
int launch_ks(const DecodeArgs& a, int slots, int chunks, int phase, hipStream_t s) {
    constexpr int SETS = WV / KS;
    if (phase == 0) {
        const int nsets = (a.I / 16 + kRpwGateup - 1) / kRpwGateup;
        dim3 grid((unsigned)((nsets + SETS - 1) / SETS), (unsigned)slots, (unsigned)chunks);
        if (a.part)   // a rotated layer: raw products
            k_ffn<F, NTT, KS, kRpwGateup, 0, WV, false, true, true>
                <<<grid, 64 * WV, codebook_lds_bytes<F>(0), s>>>(a);
        else
            k_ffn<F, NTT, KS, kRpwGateup, 0, WV, false>
                <<<grid, 64 * WV, codebook_lds_bytes<F>(0), s>>>(a);
    } else {
        const int nsets = (a.H / 16 + kRpwDown - 1) / kRpwDown;
        dim3 grid((unsigned)((nsets + SETS - 1) / SETS), (unsigned)slots, (unsigned)chunks);
        k_ffn<F, NTT, KS, kRpwDown, 1, WV, false>
            <<<grid, 64 * WV, codebook_lds_bytes<F>(1), s>>>(a);
    }
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

// Few active experts -> split the input dimension over more waves so the
// whole chip streams; many -> one wave per row set.  (An 8-way split in
// 8-wave workgroups measured slower at one token than this 4-way split.)
template <class F, int NTT>
int launch_fmt(const DecodeArgs& a, int slots, int chunks, int phase, hipStream_t s) {
    if (slots <= 16) return launch_ks<F, NTT, 4, 4>(a, slots, chunks, phase, s);
    if (slots <= 64) return launch_ks<F, NTT, 2, 4>(a, slots, chunks, phase, s);
    return launch_ks<F, NTT, 1, 4>(a, slots, chunks, phase, s);
}

// The identity map of a one-expert layer (a shared expert): one 16-row group
// (pair) per wave, 4 waves splitting the inputs of a workgroup, and for
// gate/up a further split of the inputs over nsplit workgroups (partials
// summed by k_swiglu_parts), so that one expert's rows fill the chip.  Up to
// 16 NTT tokens per wave pass (NTT = 2 for batches past 16 tokens, 1 for
// VQ8, whose LDS lookups need the registers; more tokens take further chunks
// of the grid's z dimension).
#ifndef MOEQ_SH_KS13
#define MOEQ_SH_KS13 4      // waves of a workgroup splitting the gate/up inputs
#endif
#ifndef MOEQ_SH_RPW13
#define MOEQ_SH_RPW13 1     // gate/up row-pair groups per wave
#endif
#ifndef MOEQ_SH_KS2
#define MOEQ_SH_KS2 4
#endif
#ifndef MOEQ_SH_RPW2
#define MOEQ_SH_RPW2 2      // down row groups per wave
#endif
#ifndef MOEQ_SH_NTT
#define MOEQ_SH_NTT 2       // largest token tile count per wave pass
#endif
#ifndef MOEQ_SH_WV13
#define MOEQ_SH_WV13 4      // waves per gate/up workgroup
#endif
#ifndef MOEQ_SH_WV2
#define MOEQ_SH_WV2 4
#endif
#ifndef MOEQ_SH_PART
#define MOEQ_SH_PART 1      // split the gate/up inputs over workgroups too
#endif
// Workgroups over the row-pair groups of a shared expert's gate/up pass
// (nblk) and the number of workgroups splitting its inputs (nsplit), for
// input tiles of tk inputs.
void shared_split(int H, int I, int tk, int& nblk, int& nsplit) {
    constexpr int KS = MOEQ_SH_KS13, RPW = MOEQ_SH_RPW13, WV = MOEQ_SH_WV13, SETS = WV / KS;
    const int nsets = (I / 16 + RPW - 1) / RPW;
    nblk = (nsets + SETS - 1) / SETS;
    const int nkb = (H + tk - 1) / tk;
    nsplit = (kSharedTargetBlocks + nblk - 1) / nblk;
    nsplit = nsplit < kSharedMaxSplit ? nsplit : kSharedMaxSplit;
    nsplit = nsplit <= nkb / KS ? nsplit : (nkb / KS > 1 ? nkb / KS : 1);
}

template <class F>
void shared_gateup_split(const DecodeArgs& a, int& nblk, int& nsplit) {
    shared_split(a.H, a.I, F::TK, nblk, nsplit);
}

template <class F, int NTT>
int launch_shared_ntt(DecodeArgs a, int phase, hipStream_t s) {
    const int chunks = (a.rows + 16 * NTT - 1) / (16 * NTT);
    if (phase == 0) {
        constexpr int KS = MOEQ_SH_KS13, RPW = MOEQ_SH_RPW13, WV = MOEQ_SH_WV13, SETS = WV / KS;
        const int nsets = (a.I / 16 + RPW - 1) / RPW;
        const int nblk = (nsets + SETS - 1) / SETS;
        if constexpr (MOEQ_SH_PART) {
            int nblk_p = 0, nsplit = 1;
            shared_gateup_split<F>(a, nblk_p, nsplit);
            a.nsplit = nsplit;
            dim3 grid((unsigned)(nblk * nsplit), 1u, (unsigned)chunks);
            k_ffn<F, NTT, KS, RPW, 0, WV, true, true>
                <<<grid, 64 * WV, codebook_lds_bytes<F>(0), s>>>(a);
            MOEQ_CHECK_LAUNCH();
            const int64_t n = (int64_t)a.rows * (a.I / 4);
            k_swiglu_parts<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a.part, nsplit, a.rows,
                                                                       a.I, a.h16);
        } else {
            dim3 grid((unsigned)nblk, 1u, (unsigned)chunks);
            k_ffn<F, NTT, KS, RPW, 0, WV, true, false>
                <<<grid, 64 * WV, codebook_lds_bytes<F>(0), s>>>(a);
        }
    } else {
        constexpr int KS = MOEQ_SH_KS2, RPW = MOEQ_SH_RPW2, WV = MOEQ_SH_WV2, SETS = WV / KS;
        const int nsets = (a.H / 16 + RPW - 1) / RPW;
        dim3 grid((unsigned)((nsets + SETS - 1) / SETS), 1u, (unsigned)chunks);
        k_ffn<F, NTT, KS, RPW, 1, WV, true, false>
            <<<grid, 64 * WV, codebook_lds_bytes<F>(1), s>>>(a);
    }
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

template <class F>
int launch_shared_fmt(const DecodeArgs& a, int phase, hipStream_t s) {
    if constexpr (F::kVq8) {
        return launch_shared_ntt<F, 1>(a, phase, s);
    } else {
        if (MOEQ_SH_NTT < 2 || a.rows <= 16) return launch_shared_ntt<F, 1>(a, phase, s);
        return launch_shared_ntt<F, MOEQ_SH_NTT < 2 ? 1 : 2>(a, phase, s);
    }
}

template <class F>
int launch_ntt(const DecodeArgs& a, int64_t T, int slots, int phase, hipStream_t s) {
    // an expert has at most T rows (the k experts of a token are distinct:
    // a documented precondition of the ABI); tokens of an expert go 16 at a
    // time to the z dimension of the grid
    const int chunks = (int)((T + 15) / 16);
    return launch_fmt<F, 1>(a, slots, chunks, phase, s);
}

DecodeArgs decode_args(const LayerView& L, int fmt, const uint16_t* x_bf16,
                       const int32_t* perm_src, const int32_t* offsets, int64_t T, int32_t k,
                       uint16_t* h16, float* y_perm) {
    DecodeArgs a;
    a.pool13 = L.pool13[fmt];
    a.pool2 = L.pool2[fmt];
    a.stride13 = L.stride13[fmt];
    a.stride2 = L.stride2[fmt];
    a.cb_gate = L.cb[0];
    a.cb_up = L.cb[1];
    a.cb_down = L.cb[2];
    a.cb_stride = L.cb_stride;
    for (int p = 0; p < 3; ++p) a.cb8[p] = L.cb8[p];
    a.rec = L.rec;
    a.offsets = offsets;
    a.perm_src = perm_src;
    a.xbf = x_bf16;
    a.h16 = reinterpret_cast<_Float16*>(h16);
    a.y_perm = y_perm;
    a.E = L.E;
    a.H = L.H;
    a.I = L.I;
    a.k = k;
    a.fmt = fmt;
    a.rows = (int)T;
    a.res13 = L.res13;
    a.res2 = L.res2;
    a.res_scale = L.res_scale;
    a.nsplit = 1;
    a.part = nullptr;
    a.logits = nullptr;
    a.topk_ids = nullptr;
    a.topk_w = nullptr;
    a.y_shared = nullptr;
    a.out = nullptr;
    a.rot = L.rot;
    a.rot_stride = L.rot_stride;
    return a;
}

template <class F>
int launch_small_fmt(const DecodeArgs& a, int64_t T, hipStream_t s) {
    // gate/up: the shape of the unfused decode kernel for <= 16 assignments
    // (4 waves splitting the inputs of 2 row-pair groups), one grid row per
    // assignment
    const int nsets = (a.I / 16 + kRpwGateup - 1) / kRpwGateup;
    dim3 g1((unsigned)nsets, (unsigned)(T * a.k), 1u);
    k_ffn<F, 1, 4, kRpwGateup, 0, 4, false, false, false, true>
        <<<g1, 256, codebook_lds_bytes<F>(0), s>>>(a);
    MOEQ_CHECK_LAUNCH();
    dim3 g2((unsigned)(a.H / 16), (unsigned)T, 1u);
    // 8 slots per wave for small-codebook VQ (one LDS codebook copy serves
    // them all); NVFP4 takes two slot groups of 4 waves each (128 VGPRs: two
    // 8-wave workgroups per CU, so a token's 384 workgroups all fit at once;
    // 4% faster at one token than 8 slots per wave in 4-wave workgroups)
    constexpr bool kWide = F::kVq8;
    if (a.k <= 4)
        k_down_combine<F, 4, 1><<<g2, 64 * kDcKS, codebook_lds_bytes<F>(1), s>>>(a);
    else if constexpr (kWide)
        k_down_combine<F, 8, 1><<<g2, 64 * kDcKS, codebook_lds_bytes<F>(1), s>>>(a);
    else
        k_down_combine<F, 4, 2><<<g2, 128 * kDcKS, codebook_lds_bytes<F>(1), s>>>(a);
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

// The same for a rotated layer, in four launches: the routed gate/up with
// each workgroup rotating its assignment's x row into LDS and writing the raw
// products g' | u' (token order, no permutation); the middle rotation (g, u
// back, SwiGLU, h' for the down pass) with each row's expert from topk_ids;
// the down pass writing every slot's y' row; the combine rotating each slot
// back.  Every value is computed as on the step-by-step path (same input
// split, same products, same rotation arithmetic), so the output has the same
// bits.  gu [T*k, 2I] fp32, h16 [T*k, I] fp16 and y_perm [T*k, H] fp32 are
// workspace.
template <class F>
int launch_small_rot_fmt(const LayerView& L, DecodeArgs a, int64_t T, float* gu, float* y_perm,
                         hipStream_t s) {
    a.part = gu;
    a.nsplit = 1;
    a.y_perm = y_perm;
    const int nsets = (a.I / 16 + kRpwGateup - 1) / kRpwGateup;
    dim3 g1((unsigned)nsets, (unsigned)(T * a.k), 1u);
    k_ffn<F, 1, 4, kRpwGateup, 0, 4, false, true, true, true>
        <<<g1, 256, codebook_lds_bytes<F>(0) + (size_t)a.H * 2, s>>>(a);
    MOEQ_CHECK_LAUNCH();
    int st = launch_rot_mid(L, gu, nullptr, T * a.k, reinterpret_cast<uint16_t*>(a.h16), s,
                            a.topk_ids);
    if (st) return st;
    dim3 g2((unsigned)(a.H / 16), (unsigned)T, 1u);
    if (a.k <= 4)
        k_down_combine<F, 4, 1, true><<<g2, 64 * kDcKS, codebook_lds_bytes<F>(1), s>>>(a);
    else if constexpr (F::kVq8)
        k_down_combine<F, 8, 1, true><<<g2, 64 * kDcKS, codebook_lds_bytes<F>(1), s>>>(a);
    else
        k_down_combine<F, 4, 2, true><<<g2, 128 * kDcKS, codebook_lds_bytes<F>(1), s>>>(a);
    MOEQ_CHECK_LAUNCH();
    return launch_combine_rot(L, y_perm, nullptr, a.topk_ids, a.topk_w, a.y_shared, T, a.k,
                              a.out, s);
}

// The fused decode layer with a BF16 shared expert, in three launches:
//   1. k_gateup_routed_shared: workgroups [0, nr) run the routed gate/up
//      (ranking each token's experts itself) over grid gr, the rest the shared
//      expert's gate/up partial sums over grid gs -- the same work as the two
//      separate kernels, so one stream of weight bytes fills the chip;
//   2. k_down_combine_swiglu: workgroups [0, nd) run the routed down + combine
//      over grid gd (no shared term yet), the rest sum the shared partials and
//      apply SwiGLU (one thread per 4 channels);
//   3. k_shared_down_add: the shared expert's down pass, each output element
//      added to the routed sum in out -- the combine's last addition.
// Every value is computed by the same code, in the same order, as in the
// separate kernels, so the output has the same bits.
// (Shared experts: "GLM-5.3-EXL3-TR3-3.42bpw", What is quantized.)
template <class F>
__global__ __launch_bounds__(256, kMinWaves) void k_gateup_routed_shared(DecodeArgs R,
                                                                          DecodeArgs S, int nr,
                                                                          uint3 gr, uint3 gs) {
    static_assert(64 * MOEQ_SH_WV13 == 256, "both halves run 256-thread workgroups");
    unsigned b = blockIdx.x;
    if (b < (unsigned)nr) {
        ffn_body<F, 1, 4, kRpwGateup, 0, 4, false, false, false, true>(
            R, uint3{b % gr.x, (b / gr.x) % gr.y, b / (gr.x * gr.y)});
    } else {
        b -= (unsigned)nr;
        ffn_body<Bf16Fmt, 1, MOEQ_SH_KS13, MOEQ_SH_RPW13, 0, MOEQ_SH_WV13, true, true, false,
                 false>(S, uint3{b % gs.x, (b / gs.x) % gs.y, b / (gs.x * gs.y)});
    }
}

template <class F, int NSL, int NG>
__global__ __launch_bounds__(64 * kDcKS * NG, kMinWaves) void k_down_combine_swiglu(
    DecodeArgs R, int nd, unsigned gdx, const float* __restrict__ part, int nsplit, int rows,
    int I, _Float16* __restrict__ h16) {
    const unsigned b = blockIdx.x;
    if (b < (unsigned)nd)
        down_combine_body<F, NSL, NG>(R, uint3{b % gdx, b / gdx, 0u});
    else
        swiglu_parts_body(part, nsplit, rows, I, h16,
                          (int64_t)(b - (unsigned)nd) * (64 * kDcKS * NG) + threadIdx.x);
}

__global__ __launch_bounds__(64 * MOEQ_SH_WV2, kMinWaves) void k_shared_down_add(DecodeArgs S) {
    ffn_body<Bf16Fmt, 1, MOEQ_SH_KS2, MOEQ_SH_RPW2, 1, MOEQ_SH_WV2, true, false, false, false,
             true>(S, uint3{blockIdx.x, blockIdx.y, blockIdx.z});
}

template <class F>
int launch_small_shared_fmt(const DecodeArgs& a, DecodeArgs sa, int64_t T, hipStream_t s) {
    // 1. routed gate/up (as launch_small_fmt) + shared gate/up partials (as
    // launch_shared_ntt with NTT = 1: at most 16 tokens)
    const int nsets = (a.I / 16 + kRpwGateup - 1) / kRpwGateup;
    const uint3 gr{(unsigned)nsets, (unsigned)(T * a.k), 1u};
    int nblk = 0, nsplit = 1;
    shared_gateup_split<Bf16Fmt>(sa, nblk, nsplit);
    sa.nsplit = nsplit;
    const int chunks = (sa.rows + 15) / 16;
    const uint3 gs{(unsigned)(nblk * nsplit), 1u, (unsigned)chunks};
    const int nr = (int)(gr.x * gr.y);
    const int ns = (int)(gs.x * gs.z);
    k_gateup_routed_shared<F><<<(unsigned)(nr + ns), 256, codebook_lds_bytes<F>(0), s>>>(
        a, sa, nr, gr, gs);
    MOEQ_CHECK_LAUNCH();
    // 2. routed down + combine (as launch_small_fmt) + the shared SwiGLU
    const unsigned gdx = (unsigned)(a.H / 16);
    const int nd = (int)(gdx * T);
    const int64_t nsw = (int64_t)sa.rows * (sa.I / 4);
    constexpr bool kWide = F::kVq8;   // as launch_small_fmt
    if (a.k <= 4) {
        const int nb = nd + (int)((nsw + 64 * kDcKS - 1) / (64 * kDcKS));
        k_down_combine_swiglu<F, 4, 1><<<(unsigned)nb, 64 * kDcKS, codebook_lds_bytes<F>(1), s>>>(
            a, nd, gdx, sa.part, nsplit, sa.rows, sa.I, sa.h16);
    } else if constexpr (kWide) {
        const int nb = nd + (int)((nsw + 64 * kDcKS - 1) / (64 * kDcKS));
        k_down_combine_swiglu<F, 8, 1><<<(unsigned)nb, 64 * kDcKS, codebook_lds_bytes<F>(1), s>>>(
            a, nd, gdx, sa.part, nsplit, sa.rows, sa.I, sa.h16);
    } else {
        const int nb = nd + (int)((nsw + 128 * kDcKS - 1) / (128 * kDcKS));
        k_down_combine_swiglu<F, 4, 2><<<(unsigned)nb, 128 * kDcKS, codebook_lds_bytes<F>(1), s>>>(
            a, nd, gdx, sa.part, nsplit, sa.rows, sa.I, sa.h16);
    }
    MOEQ_CHECK_LAUNCH();
    // 3. shared down, added to out (as launch_shared_ntt's down pass, NTT = 1)
    constexpr int SETS2 = MOEQ_SH_WV2 / MOEQ_SH_KS2;
    const int nsets2 = (sa.H / 16 + MOEQ_SH_RPW2 - 1) / MOEQ_SH_RPW2;
    dim3 g3((unsigned)((nsets2 + SETS2 - 1) / SETS2), 1u, (unsigned)chunks);
    k_shared_down_add<<<g3, 64 * MOEQ_SH_WV2, 0, s>>>(sa);
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

// Two formats of a mixed layer in one launch (decode batches): workgroups
// [0, n2) run the second format's grid g2, the rest the first format's grid
// g1, each with the body of its own kernel (so the same bits).  The second
// format is a VQ form, whose gather-bound workgroups go first; the NVFP4
// weight stream then runs beside them instead of after them.
// ("GLM-5.3-EXL3-TR3-3.42bpw", What is quantized: layers that mix two
// per-expert tiers.)
template <class F1, class F2, int KS, int PHASE>
__global__ __launch_bounds__(256, kMinWaves) void k_ffn_pair(DecodeArgs A1, DecodeArgs A2,
                                                             int n2, uint3 g1, uint3 g2) {
    constexpr int RPW = PHASE == 0 ? kRpwGateup : kRpwDown;
    unsigned b = blockIdx.x;
    if (b < (unsigned)n2) {
        ffn_body<F2, 1, KS, RPW, PHASE, 4, false, false, false, false>(
            A2, uint3{b % g2.x, (b / g2.x) % g2.y, b / (g2.x * g2.y)});
    } else {
        b -= (unsigned)n2;
        ffn_body<F1, 1, KS, RPW, PHASE, 4, false, false, false, false>(
            A1, uint3{b % g1.x, (b / g1.x) % g1.y, b / (g1.x * g1.y)});
    }
}

// The input split launch_fmt picks for this many active-expert slots.
int decode_ks(int slots) { return slots <= 16 ? 4 : slots <= 64 ? 2 : 1; }

template <class F2, int KS>
int launch_pair_ks(const DecodeArgs& a1, int slots1, const DecodeArgs& a2, int slots2, int chunks,
                   int phase, hipStream_t s) {
    constexpr int SETS = 4 / KS;
    const int nrg = phase == 0 ? a1.I / 16 : a1.H / 16;
    const int rpw = phase == 0 ? kRpwGateup : kRpwDown;
    const int nsets = (nrg + rpw - 1) / rpw;
    const unsigned gx = (unsigned)((nsets + SETS - 1) / SETS);
    const uint3 g1{gx, (unsigned)slots1, (unsigned)chunks};
    const uint3 g2{gx, (unsigned)slots2, (unsigned)chunks};
    const int n2 = (int)(g2.x * g2.y * g2.z);
    const unsigned nb = (unsigned)n2 + g1.x * g1.y * g1.z;
    if (phase == 0)
        k_ffn_pair<NvFmt, F2, KS, 0><<<nb, 256, codebook_lds_bytes<F2>(0), s>>>(a1, a2, n2, g1, g2);
    else
        k_ffn_pair<NvFmt, F2, KS, 1><<<nb, 256, codebook_lds_bytes<F2>(1), s>>>(a1, a2, n2, g1, g2);
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

template <class F2>
int launch_pair_fmt(const DecodeArgs& a1, int slots1, const DecodeArgs& a2, int slots2,
                    int chunks, int phase, hipStream_t s) {
    switch (decode_ks(slots1)) {
        case 4: return launch_pair_ks<F2, 4>(a1, slots1, a2, slots2, chunks, phase, s);
        case 2: return launch_pair_ks<F2, 2>(a1, slots1, a2, slots2, chunks, phase, s);
        default: return launch_pair_ks<F2, 1>(a1, slots1, a2, slots2, chunks, phase, s);
    }
}

}  // namespace

bool ffn_decode_pair_ok(const LayerView& L, int fmt1, int n1, int fmt2, int n2, int64_t T,
                        int32_t k) {
    if (fmt1 != MOE_FMT_NVFP4 || !(fmt2 == MOE_FMT_VQ || is_vq8(fmt2)) || L.rot) return false;
    const int64_t tk = T * k;
    const int s1 = (int)(tk < n1 ? tk : n1), s2 = (int)(tk < n2 ? tk : n2);
    return s1 > 0 && s2 > 0 && decode_ks(s1) == decode_ks(s2);
}

int launch_ffn_decode_pair(const LayerView& L, int fmt1, int n1, int fmt2, int n2,
                           const uint16_t* x_bf16, const int32_t* perm_src,
                           const int32_t* offsets, int64_t T, int32_t k, uint16_t* h16,
                           float* y_perm, int phase, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const DecodeArgs a1 = decode_args(L, fmt1, x_bf16, perm_src, offsets, T, k, h16, y_perm);
    const DecodeArgs a2 = decode_args(L, fmt2, x_bf16, perm_src, offsets, T, k, h16, y_perm);
    const int64_t tk = T * k;
    const int s1 = (int)(tk < n1 ? tk : n1), s2 = (int)(tk < n2 ? tk : n2);
    const int chunks = (int)((T + 15) / 16);
    if (fmt2 == MOE_FMT_VQ) return launch_pair_fmt<VqFmt>(a1, s1, a2, s2, chunks, phase, s);
    const int m = vq8_rate(fmt2, L.vq8_m);
    if (m == 1) return launch_pair_fmt<Vq8Fmt<1>>(a1, s1, a2, s2, chunks, phase, s);
    if (m == 3) return launch_pair_fmt<Vq8Fmt<3>>(a1, s1, a2, s2, chunks, phase, s);
    return launch_pair_fmt<Vq8Fmt<2>>(a1, s1, a2, s2, chunks, phase, s);
}

int launch_layer_small(const LayerView& L, int fmt, const uint16_t* x_bf16, const float* logits,
                       int64_t T, int32_t k, int32_t* topk_ids, float* topk_w, uint16_t* h16,
                       const float* y_shared, float* out, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    DecodeArgs a = decode_args(L, fmt, x_bf16, nullptr, nullptr, T, k, h16, nullptr);
    a.logits = logits;
    a.topk_ids = topk_ids;
    a.topk_w = topk_w;
    a.y_shared = y_shared;
    a.out = out;
    if (T == 0) return MOE_OK;
    if (L.rot) {
        // workspace after h16 [T*k, I]: g' | u' [T*k, 2I], then y' [T*k, H]
        const int64_t tk = T * k;
        float* gu = reinterpret_cast<float*>(h16 + round_up(tk * L.I, 128));
        float* yp = gu + round_up(tk * 2 * L.I, 64);
        if (fmt == MOE_FMT_NVFP4) return launch_small_rot_fmt<NvFmt>(L, a, T, gu, yp, s);
        if (fmt == MOE_FMT_NVFP4R) return launch_small_rot_fmt<Nv2Fmt>(L, a, T, gu, yp, s);
        if (fmt == MOE_FMT_BF16) return launch_small_rot_fmt<Bf16Fmt>(L, a, T, gu, yp, s);
        if (is_vq8(fmt)) {
            const int m = vq8_rate(fmt, L.vq8_m);
            if (m == 1) return launch_small_rot_fmt<Vq8Fmt<1>>(L, a, T, gu, yp, s);
            if (m == 3) return launch_small_rot_fmt<Vq8Fmt<3>>(L, a, T, gu, yp, s);
            return launch_small_rot_fmt<Vq8Fmt<2>>(L, a, T, gu, yp, s);
        }
        return launch_small_rot_fmt<VqFmt>(L, a, T, gu, yp, s);
    }
    if (fmt == MOE_FMT_NVFP4) return launch_small_fmt<NvFmt>(a, T, s);
    if (fmt == MOE_FMT_NVFP4R) return launch_small_fmt<Nv2Fmt>(a, T, s);
    if (fmt == MOE_FMT_BF16) return launch_small_fmt<Bf16Fmt>(a, T, s);
    if (is_vq8(fmt)) {
        const int m = vq8_rate(fmt, L.vq8_m);
        if (m == 1) return launch_small_fmt<Vq8Fmt<1>>(a, T, s);
        if (m == 3) return launch_small_fmt<Vq8Fmt<3>>(a, T, s);
        return launch_small_fmt<Vq8Fmt<2>>(a, T, s);
    }
    return launch_small_fmt<VqFmt>(a, T, s);
}

int launch_layer_small_shared(const LayerView& L, int fmt, const LayerView& SL,
                              const uint16_t* x_bf16, const float* logits, int64_t T, int32_t k,
                              int32_t* topk_ids, float* topk_w, uint16_t* h16, uint16_t* sh_h16,
                              float* sh_part, float* out, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (T == 0) return MOE_OK;
    DecodeArgs a = decode_args(L, fmt, x_bf16, nullptr, nullptr, T, k, h16, nullptr);
    a.logits = logits;
    a.topk_ids = topk_ids;
    a.topk_w = topk_w;
    a.out = out;
    DecodeArgs sa = decode_args(SL, MOE_FMT_BF16, x_bf16, nullptr, nullptr, T, 1, sh_h16, nullptr);
    sa.part = sh_part;
    sa.out = out;
    if (fmt == MOE_FMT_NVFP4) return launch_small_shared_fmt<NvFmt>(a, sa, T, s);
    if (fmt == MOE_FMT_NVFP4R) return launch_small_shared_fmt<Nv2Fmt>(a, sa, T, s);
    if (fmt == MOE_FMT_BF16) return launch_small_shared_fmt<Bf16Fmt>(a, sa, T, s);
    if (is_vq8(fmt)) {
        const int m = vq8_rate(fmt, L.vq8_m);
        if (m == 1) return launch_small_shared_fmt<Vq8Fmt<1>>(a, sa, T, s);
        if (m == 3) return launch_small_shared_fmt<Vq8Fmt<3>>(a, sa, T, s);
        return launch_small_shared_fmt<Vq8Fmt<2>>(a, sa, T, s);
    }
    return launch_small_shared_fmt<VqFmt>(a, sa, T, s);
}

int launch_ffn_decode(const LayerView& L, int fmt, int n_fmt, const uint16_t* x_bf16,
                      const int32_t* perm_src, const int32_t* offsets, int64_t T, int32_t k,
                      uint16_t* h16, float* y_perm, int phase, void* stream, float* gu) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    DecodeArgs a = decode_args(L, fmt, x_bf16, perm_src, offsets, T, k, h16, y_perm);
    a.part = phase == 0 ? gu : nullptr;   // nsplit = 1
    const int64_t tk = T * k;
    const int slots = (int)(tk < n_fmt ? tk : n_fmt);
    if (slots == 0) return MOE_OK;
    if (fmt == MOE_FMT_NVFP4) return launch_ntt<NvFmt>(a, T, slots, phase, s);
    if (fmt == MOE_FMT_NVFP4R) return launch_ntt<Nv2Fmt>(a, T, slots, phase, s);
    if (fmt == MOE_FMT_BF16) return launch_ntt<Bf16Fmt>(a, T, slots, phase, s);
    if (is_vq8(fmt)) {
        const int m = vq8_rate(fmt, L.vq8_m);
        if (m == 1) return launch_ntt<Vq8Fmt<1>>(a, T, slots, phase, s);
        if (m == 3) return launch_ntt<Vq8Fmt<3>>(a, T, slots, phase, s);
        return launch_ntt<Vq8Fmt<2>>(a, T, slots, phase, s);
    }
    return launch_ntt<VqFmt>(a, T, slots, phase, s);
}

}  // namespace moeq

namespace moeq {

size_t shared_part_bytes(int fmt, int64_t T, int32_t H, int32_t I) {
    if (T <= 0 || H <= 0 || I <= 0) return 0;
    if (T >= kPrefillMinTokens && prefill_fmt(fmt, true)) return 0;   // the grouped GEMM
    if (!MOEQ_SH_PART) return 0;
    const bool known = fmt >= MOE_FMT_NVFP4 && fmt <= MOE_FMT_MAX;
    // input tile of the format (an unknown tag: the smaller tile, the larger split)
    const int tk = known && (fmt == MOE_FMT_VQ || is_vq8(fmt)) ? kVqTileK : kNvTileK;
    int nblk = 0, nsplit = 1;
    shared_split(H, I, tk, nblk, nsplit);
    return (size_t)nsplit * (size_t)T * 2 * (size_t)I * 4;
}

int launch_shared_decode(const LayerView& L, int fmt, const uint16_t* x_bf16, int64_t T,
                         uint16_t* h16, float* part, float* y, int phase, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    DecodeArgs a = decode_args(L, fmt, x_bf16, nullptr, nullptr, T, 1, h16, y);
    a.part = part;
    if (T == 0) return MOE_OK;
    if (fmt == MOE_FMT_NVFP4) return launch_shared_fmt<NvFmt>(a, phase, s);
    if (fmt == MOE_FMT_NVFP4R) return launch_shared_fmt<Nv2Fmt>(a, phase, s);
    if (fmt == MOE_FMT_BF16) return launch_shared_fmt<Bf16Fmt>(a, phase, s);
    if (is_vq8(fmt)) {
        const int m = vq8_rate(fmt, L.vq8_m);
        if (m == 1) return launch_shared_fmt<Vq8Fmt<1>>(a, phase, s);
        if (m == 3) return launch_shared_fmt<Vq8Fmt<3>>(a, phase, s);
        return launch_shared_fmt<Vq8Fmt<2>>(a, phase, s);
    }
    return launch_shared_fmt<VqFmt>(a, phase, s);
}

}  // namespace moeq
