// Expert FFN for large token batches (prefill): a grouped GEMM over the
// active experts with their weights decoded in registers (NVFP4, BF16, and
// VQ codes whose codebook rows come from LDS (small codebooks) or L2).
//
// Per active expert e with M_e rows (permuted order r0 .. r0+M_e):
//   gate/up:  [g | u] = W13[e] X_e^T,  h = silu(g) * u      -> h (fp16)
//   down:     Y_e = W_down[e] H_e^T                         -> y_perm (fp32)
// ("GLM-5-NVFP4-MTP", What's quantized: gate, up and down projections.)
//
// Work item = (expert, 64-row tile of its tokens) x (256 weight rows).  A
// workgroup of 4 waves owns one item; wave w owns 64 weight rows (two 32-row
// A tiles of v_mfma_f32_32x32x16_f16) and all 64 tokens (two 32-token B
// tiles), i.e. a 64 x 64 fp32 accumulator block.  (BF16 experts: 32
// weight rows per wave, since a raw bf16 A fragment takes four times the
// registers of an NVFP4 one.)
//   * weights: each wave loads its rows' packed NVFP4 tiles from HBM straight
//     into registers (the next 128-input tile is in flight while the current
//     one is used), decodes 8 weights at a time to fp16 (exact) right before
//     the MFMA that uses them;
//   * tokens: the 64 rows x 128 inputs fp16 tile is gathered (through
//     perm_src for gate/up) into LDS with direct-to-LDS loads (no register
//     round trip), double-buffered, XOR-swizzled against bank conflicts;
//   * gate/up: a 32-row A tile is 16 gate rows + the 16 matching up rows, so
//     each lane holds g and u of the same (channel, token) and SwiGLU is fused
//     in registers before the fp16 store of h.
// A workgroup finds its (expert, row tile, weight tile) from the offsets with
// a wave prefix scan; the grid is an upper bound on the work list (slots past
// its end exit at once), items dealt round-robin over the 8 XCDs.
#include <type_traits>

#include "dev_common.h"

namespace moeq {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Tokens per work item, per weight format (the trait's BM): 64 for NVFP4
// and small-codebook VQ, 128 for BF16 and 16-bit VQ.  (Measured at T = 4096:
// 64-token items, three waves per SIMD, ran the NVFP4 passes 2-4% faster and
// the small-codebook ones 5-15% faster than 128-token items at two waves per
// SIMD, although each decoded weight then feeds half as many MFMAs; 16-bit
// VQ, whose codebook rows are L2 gathers per item, ran 30% slower, and BF16
// 1% slower.)
constexpr int kBMMax = 128;
// Workgroup shape: waves of 64 weight rows each, and token-tile buffers.
// (Measured: 4 waves x 2 buffers beats 8 waves x 3 buffers and 8 x 2.)
#ifndef MOEQ_PF_WAVES
#define MOEQ_PF_WAVES 4
#endif
#ifndef MOEQ_PF_STAGES
#define MOEQ_PF_STAGES 2
#endif
#ifndef MOEQ_PF_ORDER
#define MOEQ_PF_ORDER 1
#endif
#ifndef MOEQ_PF_OCC
#define MOEQ_PF_OCC 2
#endif
constexpr int kPrefillWaves = MOEQ_PF_WAVES;
constexpr int kPrefillStages = MOEQ_PF_STAGES;
// s_waitcnt immediate for "vmcnt(0)", other counters unconstrained (gfx9 encoding:
// vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8]).
constexpr int kVmcnt0 = 0x0F70;

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
}

struct PrefillArgs {
    const uint8_t* pool;
    int64_t stride;
    const uint8_t* cb[3];      // VQ codebooks (gate, up, down), per record at cb_stride
    int64_t cb_stride;
    const uint8_t* cb8[3];     // VQ8 codebooks (gate, up, down): [M][256][8] fp16
    const int32_t* rec;
    const int32_t* offsets;    // NULL: one expert whose rows are the tokens
    const int32_t* perm_src;   // NULL: identity
    const _Float16* x16;
    _Float16* h16;
    float* y_perm;
    int E, H, I, k, fmt;
    int rows;                  // offsets == NULL: rows of the identity map
    float* gu;                 // rotated layers: raw g | u [rows, 2I] (gate/up)
    int64_t res;               // MOE_FMT_NVFP4R: residual plane offset in a record
    float res_scale;           // ... and its decode factor
};

struct WorkItem {
    int e, r0, me, ridx, m0;
};

// Locates work item w of the list (item-major, nnt weight tiles per item,
// items = (expert, BM-row tile) over the active experts of `fmt` in
// ascending expert id).  All offsets/record loads are issued up front (one
// memory round trip); the item count comes from the same registers.
// Returns e = -1 if w is past the end of the list.
// ID: the identity map of a one-expert layer (rows 0 .. rows-1 of expert 0).
template <int BM, bool ID>
__device__ __forceinline__ WorkItem locate_item(const int32_t* __restrict__ offsets,
                                                const int32_t* __restrict__ rec, int E, int fmt,
                                                int rows, int nnt, int blk, int lane,
                                                int& ntile) {
    if constexpr (ID) {
#if MOEQ_PF_ORDER == 0
        const int total = (rows + BM - 1) / BM;
        const int nwork = total * nnt;
        const int quota = (nwork + 7) / 8;
        const int slot = blk >> 3;
        const int w = (blk & 7) * quota + slot;
        ntile = w % nnt;
        const int want_item = (slot >= quota || w >= nwork) ? total : w / nnt;
#else
        const int slot = blk >> 3;
        const int want_item = (slot / nnt) * 8 + (blk & 7);
        ntile = slot % nnt;
#endif
        if (want_item * BM >= rows) return WorkItem{-1, 0, 0, 0, 0};
        return WorkItem{0, 0, rows, 0, want_item * BM};
    }
    constexpr int kMaxChunks = MOE_MAX_E / 64;
    int o0[kMaxChunks], o1[kMaxChunks], rc[kMaxChunks], cnt[kMaxChunks];
    const int nch = (E + 63) / 64;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        const int e = 64 * c + lane;
        const bool in = c < nch && e < E;
        o0[c] = in ? offsets[e] : 0;
        o1[c] = in ? offsets[e + 1] : 0;
        rc[c] = in ? rec[e] : 0;
    }
    int total = 0;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        cnt[c] = (o1[c] > o0[c] && (rc[c] >> 24) == fmt) ? (o1[c] - o0[c] + BM - 1) / BM : 0;
        int t = cnt[c];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
        total += t;
    }
    WorkItem r{-1, 0, 0, 0, 0};
#if MOEQ_PF_ORDER == 0
    // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs,
    // so XCD blk % 8 takes a contiguous slice of the work list.  The weight
    // tiles of one token tile, and the next few token tiles of the same
    // expert, then share that XCD's L2.
    const int nwork = total * nnt;
    const int quota = (nwork + 7) / 8;
    const int slot = blk >> 3;
    const int w = (blk & 7) * quota + slot;
    if (slot >= quota || w >= nwork) return r;
    ntile = w % nnt;
    const int want_item = w / nnt;
#else
    // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs
    // (XCD blk % 8); items are dealt to the XCDs round-robin too, and all
    // nnt weight tiles of an item run on its XCD, one after the other, so
    // they share the item's token tiles in that XCD's L2.  Dealing items
    // (rather than cutting the list into 8 slices) evens out the work per
    // XCD when expert sizes are skewed.
    const int slot = blk >> 3;
    const int want_item = (slot / nnt) * 8 + (blk & 7);
    ntile = slot % nnt;
    if (want_item >= total) return r;
#endif
    int before = 0;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        int incl = cnt[c];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off);
            if (lane >= off) incl += v;
        }
        const int tot = __shfl(incl, 63);
        const int want = want_item - before;
        if (r.e < 0 && want >= 0 && want < tot) {
            const bool mine = cnt[c] > 0 && want >= incl - cnt[c] && want < incl;
            const uint64_t m = __ballot(mine);
            const int owner = __ffsll((unsigned long long)m) - 1;
            r.e = 64 * c + owner;
            r.r0 = __shfl(o0[c], owner);
            r.me = __shfl(o1[c], owner) - r.r0;
            r.ridx = __shfl(rc[c], owner) & 0xffffff;
            r.m0 = (want - (__shfl(incl, owner) - __shfl(cnt[c], owner))) * BM;
        }
        before += tot;
    }
    return r;
}

// One lane's share of a 32-row A tile for one 128-input tile: rows
// (L & 31) of record groups ga (L < 16 of the 32) / ga + 1, inputs
// (L >> 5) * 64 .. +64 = two 16-byte code chunks and their 4 scales.
struct AFrag {
    u32x4 c0, c1;
    uint16_t s0, s1;
};

__device__ __forceinline__ void load_a(AFrag& f, const uint8_t* grp_base, int64_t gstride,
                                       int lane, bool valid) {
    if (!valid) {
        f.c0 = f.c1 = u32x4{0u, 0u, 0u, 0u};
        f.s0 = f.s1 = 0u;
        return;
    }
    const int row = lane & 31;
    const uint8_t* tile = grp_base + (row >> 4) * gstride;   // group ga or ga + 1
    const int l0 = (row & 15) + 32 * (lane >> 5);            // record lane of inputs 64h..
    const int l1 = l0 + 16;                                  // ... and 64h + 32..
    f.c0 = *reinterpret_cast<const u32x4*>(tile + l0 * 16);
    f.c1 = *reinterpret_cast<const u32x4*>(tile + l1 * 16);
    f.s0 = *reinterpret_cast<const uint16_t*>(tile + kNvScaleOff + l0 * 2);
    f.s1 = *reinterpret_cast<const uint16_t*>(tile + kNvScaleOff + l1 * 2);
}

// 8 decoded weights of K-step s (inputs 64h + 8s .. +7 of the tile).
__device__ __forceinline__ f16x8 a_step(const AFrag& f, int s) {
    const uint32_t sc = s < 4 ? f.s0 : f.s1;
    const u32x4 c = s < 4 ? f.c0 : f.c1;
    f16x2 s0, s1;
    nv_scales(sc, s0, s1);
    const f16x2 sv = ((s & 3) < 2) ? s0 : s1;
    return nv_dequant8(c[s & 3], sv);
}

// Weight formats of the grouped GEMM.  NA 32-row A tiles per wave; NSUB A
// operands (MFMAs) per K-step; group_bytes(K) bytes per 16-row record group;
// load() reads the lane's fragment of one A tile for the 128-input step kb
// (grp_base = the tile's first record group); step(f, s, j, ctx) is the fp16
// A operand j of K-step s (inputs 64h + 8s .. +7 of the step); kScales: fp16
// per-row scales follow the record's code tiles; cb_lds(phase): bytes of
// codebooks the workgroup keeps in LDS; ctx: the lane's codebook base.
#ifndef MOEQ_PF_NV_BM
#define MOEQ_PF_NV_BM 64
#endif
struct PfNv {
    static constexpr int BM = MOEQ_PF_NV_BM;
    static constexpr int NA = 2;
    static constexpr int NSUB = 1;
    static constexpr bool kScales = false;
    static constexpr int cb_lds(int) { return 0; }
    __device__ __forceinline__ static int64_t group_bytes(int K) {
        return (int64_t)((K + kNvTileK - 1) / kNvTileK) * kNvTileBytes;
    }
    using Frag = AFrag;
    __device__ __forceinline__ static void load(Frag& f, const uint8_t* grp_base, int64_t gstride,
                                                int kb, int K, int lane, bool valid,
                                                int64_t, float) {
        load_a(f, grp_base + (int64_t)kb * kNvTileBytes, gstride, lane, valid);
    }
    __device__ __forceinline__ static f16x8 step(const Frag& f, int s, int, const void*) {
        return a_step(f, s);
    }
};

// Nested two-level NVFP4 (MOE_FMT_NVFP4R): the base plane's tile and the
// residual plane's (poff bytes further on in the record, its scales times the
// layer's power of two pscale); sub-step j of a K-step is plane j, each its
// own exact MFMA A operand.
struct PfNv2 {
    static constexpr int BM = 64;
    static constexpr int NA = 2;
    static constexpr int NSUB = 2;
    static constexpr bool kScales = false;
    static constexpr int cb_lds(int) { return 0; }
    __device__ __forceinline__ static int64_t group_bytes(int K) { return PfNv::group_bytes(K); }
    struct Frag {
        AFrag p[2];
        _Float16 ps;
    };
    __device__ __forceinline__ static void load(Frag& f, const uint8_t* grp_base, int64_t gstride,
                                                int kb, int K, int lane, bool valid,
                                                int64_t poff, float pscale) {
        const uint8_t* t = grp_base + (int64_t)kb * kNvTileBytes;
        load_a(f.p[0], t, gstride, lane, valid);
        load_a(f.p[1], t + poff, gstride, lane, valid);
        f.ps = (_Float16)pscale;
    }
    __device__ __forceinline__ static f16x8 step(const Frag& f, int s, int j, const void*) {
        if (j == 0) return a_step(f.p[0], s);
        const uint32_t sc = s < 4 ? f.p[1].s0 : f.p[1].s1;
        const u32x4 c = s < 4 ? f.p[1].c0 : f.p[1].c1;
        f16x2 s0, s1;
        nv_scales(sc, s0, s1);
        const f16x2 sv = (((s & 3) < 2) ? s0 : s1) * f16x2{f.ps, f.ps};
        return nv_dequant8(c[s & 3], sv);
    }
};

// BF16: lane L (row L & 31, half h = L >> 5) needs inputs 64h + 8s .. +7,
// s = 0..7: record lane (row & 15) + 32h holds 64h + 8j (s = j < 4), record
// lane + 16 holds 64h + 32 + 8j (s = 4 + j), slice j of the tile.
struct PfBf16 {
    static constexpr int BM = 128;
    static constexpr int NA = 1;
    static constexpr int NSUB = 1;
    static constexpr bool kScales = false;
    static constexpr int cb_lds(int) { return 0; }
    __device__ __forceinline__ static int64_t group_bytes(int K) {
        return (int64_t)((K + kBf16TileK - 1) / kBf16TileK) * kBf16TileBytes;
    }
    struct Frag {
        u32x4 c[8];
    };
    __device__ __forceinline__ static void load(Frag& f, const uint8_t* grp_base, int64_t gstride,
                                                int kb, int K, int lane, bool valid,
                                                int64_t, float) {
        if (!valid) {
#pragma unroll
            for (int s = 0; s < 8; ++s) f.c[s] = u32x4{0u, 0u, 0u, 0u};
            return;
        }
        const int row = lane & 31;
        const uint8_t* tile = grp_base + (int64_t)kb * kBf16TileBytes + (row >> 4) * gstride;
        const int l0 = (row & 15) + 32 * (lane >> 5);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f.c[j] = *reinterpret_cast<const u32x4*>(tile + 1024 * j + l0 * 16);
            f.c[4 + j] = *reinterpret_cast<const u32x4*>(tile + 1024 * j + (l0 + 16) * 16);
        }
    }
    __device__ __forceinline__ static f16x8 step(const Frag& f, int s, int, const void*) {
        return bf16x8_to_f16x8(f.c[s]);
    }
};

// VQ codes (8 inputs per code) in 256-input record tiles: for the 128-input
// step kb, lane L (row L & 31, half h = L >> 5) needs the 8 groups of inputs
// (kb & 1) * 128 + 64h + 8s, s = 0..7, which record lane
// (row & 15) + 16 (2 (kb & 1) + h) holds.  Groups at or past K (the zero
// codes of the padding still select a codebook row) give a zero operand.
// Per-row fp16 scales are applied in the epilogue.
//
// M uint8 codes per group into M 256-entry codebooks held in LDS (one MFMA
// per codebook row: every product exact, as in the decode kernels).
// MOEQ_PF_VQ8_SUM: sum a group's codebook rows in fp32 and round once to fp16
// (one MFMA instead of M).  Measured 10-12% faster at M = 2 and 3 (the LDS
// lookups and occupancy limit these kernels, not the MFMAs); off, so that
// every product stays exact as in the decode kernels.
#ifndef MOEQ_PF_VQ8_SUM
#define MOEQ_PF_VQ8_SUM 0
#endif
template <int M>
struct PfVq8 {
    static constexpr int BM = 64;
    static constexpr int NA = 2;
    static constexpr int NSUB = MOEQ_PF_VQ8_SUM ? 1 : M;
    static constexpr bool kScales = true;
    static constexpr int cb_lds(int phase) { return (phase == 0 ? 2 : 1) * M * MOE_VQ8_NCODE * 16; }
    __device__ __forceinline__ static int64_t group_bytes(int K) {
        return (int64_t)((K + kVq8TileK - 1) / kVq8TileK) * kVq8TileBytesPerCode * M;
    }
    struct Frag {
        uint32_t c[2 * M];
        int nvalid;     // K-steps of the lane inside K
    };
    __device__ __forceinline__ static void load(Frag& f, const uint8_t* grp_base, int64_t gstride,
                                                int kb, int K, int lane, bool valid,
                                                int64_t, float) {
        const int row = lane & 31;
        const int h = lane >> 5;
        const int k0 = kb * 128 + 64 * h;
        f.nvalid = valid ? max(0, min(8, (K - k0) / 8)) : 0;
        const uint8_t* p = grp_base + (int64_t)(kb >> 1) * (kVq8TileBytesPerCode * M) +
                           (row >> 4) * gstride +
                           ((row & 15) + 16 * (2 * (kb & 1) + h)) * (8 * M);
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int q = 0; q < M; ++q) {
            u32x2 v = {0u, 0u};
            if (valid) v = *reinterpret_cast<const u32x2*>(p + 8 * q);
            f.c[2 * q] = v[0];
            f.c[2 * q + 1] = v[1];
        }
    }
    // ctx: the lane's projection codebooks in LDS ([M][256][8] fp16)
    __device__ __forceinline__ static f16x8 row(const Frag& f, int s, int j, const void* ctx) {
        const int byte = M * s + j;
        const uint32_t code = (f.c[byte >> 2] >> (8 * (byte & 3))) & 0xffu;
        return *(reinterpret_cast<const f16x8*>(ctx) + j * MOE_VQ8_NCODE + code);
    }
    __device__ __forceinline__ static f16x8 step(const Frag& f, int s, int j, const void* ctx) {
        f16x8 r;
        if constexpr (MOEQ_PF_VQ8_SUM && M > 1) {
            float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < M; ++jj) {
                const f16x8 c = row(f, s, jj, ctx);
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] += (float)c[i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) r[i] = (_Float16)v[i];
        } else {
            r = row(f, s, j, ctx);
        }
        return s < f.nvalid ? r : f16x8{};
    }
};

// 16-bit VQ codes into a 65536 x 8 fp16 codebook read from L2 (a gather per
// operand).
struct PfVq {
    static constexpr int BM = 128;
    static constexpr int NA = 2;
    static constexpr int NSUB = 1;
    static constexpr bool kScales = true;
    static constexpr int cb_lds(int) { return 0; }
    __device__ __forceinline__ static int64_t group_bytes(int K) {
        return (int64_t)((K + kVqTileK - 1) / kVqTileK) * kVqTileBytes;
    }
    struct Frag {
        u32x4 c;
        int nvalid;
    };
    __device__ __forceinline__ static void load(Frag& f, const uint8_t* grp_base, int64_t gstride,
                                                int kb, int K, int lane, bool valid,
                                                int64_t, float) {
        const int row = lane & 31;
        const int h = lane >> 5;
        const int k0 = kb * 128 + 64 * h;
        f.nvalid = valid ? max(0, min(8, (K - k0) / 8)) : 0;
        f.c = u32x4{0u, 0u, 0u, 0u};
        if (valid)
            f.c = *reinterpret_cast<const u32x4*>(grp_base + (int64_t)(kb >> 1) * kVqTileBytes +
                                                  (row >> 4) * gstride +
                                                  ((row & 15) + 16 * (2 * (kb & 1) + h)) * 16);
    }
    // ctx: the lane's projection codebook in global memory
    __device__ __forceinline__ static f16x8 step(const Frag& f, int s, int, const void* ctx) {
        const uint32_t code = (f.c[s >> 1] >> (16 * (s & 1))) & 0xffffu;
        const f16x8 r = vq_row(reinterpret_cast<const uint8_t*>(ctx), code);
        return s < f.nvalid ? r : f16x8{};
    }
};

template <class PF>
constexpr int pf_bn() {
    return 32 * PF::NA * kPrefillWaves;   // weight rows per work item
}

// WV waves per workgroup (32 NA weight rows each), NS token-tile buffers of
// PF::BM tokens in dynamic LDS (NS - 1 tiles in flight ahead of the one in
// use).  (WV and NS are file-level constants, not template parameters: a
// static __shared__ array sized by a template parameter lost its host-side
// launch stub with this compiler; the token tiles now sit in dynamic LDS.)
// ID: offsets / perm_src are the identity map of a one-expert layer.  ROT
// (gate/up of a rotated layer): the token tile rows are the fp16 rotated rows
// of the assignments (x16 = [rows, H] in permuted order) and the raw fp32
// products go to A.gu instead of h.
template <class PF, int PHASE, bool ID, bool ROT = false>
__global__ __launch_bounds__(64 * kPrefillWaves, MOEQ_PF_OCC) void k_prefill(PrefillArgs A) {
    static_assert(!ROT || (PHASE == 0 && !ID), "rotated: gate/up of a routed layer");
    constexpr int WV = kPrefillWaves;
    constexpr int NS = kPrefillStages;
    constexpr int NA = PF::NA;
    constexpr int BN = pf_bn<PF>();    // weight rows per work item
    constexpr int BM = PF::BM;         // tokens per work item
    constexpr int NBM = BM / 32;       // 32-token B tiles per work item
    constexpr int JX = BM / 4 / WV;    // 1 KB staging loads per wave per token tile
    // dynamic LDS: NS token-tile buffers of BM x 128 fp16, then the codebooks
    // the workgroup keeps in LDS (small-codebook VQ)
    extern __shared__ _Float16 pf_lds[];
    _Float16* const xs = pf_lds;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int K = PHASE == 0 ? A.H : A.I;
    const int nrg = (PHASE == 0 ? 2 * A.I : A.H) / 16;       // record row groups
    const int nnt = (nrg + BN / 16 - 1) / (BN / 16);          // weight tiles of BN rows
    int ntile = 0;
    const WorkItem it =
        locate_item<BM, ID>(A.offsets, A.rec, A.E, A.fmt, A.rows, nnt, blockIdx.x, lane, ntile);
    if (it.e < 0) return;
    const int nkb = (K + kNvTileK - 1) / kNvTileK;
    const int64_t gstride = PF::group_bytes(K);               // bytes per row group
    const int g0 = ntile * (BN / 16) + wave * 2 * NA;         // first row group of the wave
    const int mcount = min(BM, it.me - it.m0);
    const int nbt = (mcount + 31) / 32;                      // 32-token B tiles in use
    const uint8_t* base = A.pool + (int64_t)it.ridx * A.stride;

    // X staging with direct-to-LDS loads: wave-instruction j of wave w fills
    // rows 4 (JX w + j) .. +3 (1 KB); lane L writes row + (L >> 4), physical
    // 16-byte chunk L & 15, which holds logical chunk (L & 15) ^ (row & 15)
    // (an XOR swizzle that keeps the B-operand reads free of bank conflicts).
    // Rows past the expert's end re-read its last row: they only feed output
    // columns that are never stored.  Inputs past K re-read input 0 of the
    // row: the matching weights are zero codes with zero scales.
    const _Float16* xsrc = PHASE == 0 ? A.x16 : A.h16;
    int trow[JX];
#pragma unroll
    for (int j = 0; j < JX; ++j) {
        const int row = min(4 * (JX * wave + j) + (lane >> 4), mcount - 1);
        const int prow = it.r0 + it.m0 + row;
        trow[j] = PHASE == 0 && !ID && !ROT ? A.perm_src[prow] / A.k : prow;
    }
    auto issue_x = [&](int kb, int buf) {
#pragma unroll
        for (int j = 0; j < JX; ++j) {
            const int row = 4 * (JX * wave + j) + (lane >> 4);
            int kk = kb * kNvTileK + 8 * ((lane & 15) ^ (row & 15));
            if (kk >= K) kk = 0;
            __builtin_amdgcn_global_load_lds(xsrc + (int64_t)trow[j] * K + kk,
                                             xs + buf * (BM * kNvTileK) +
                                                 4 * (JX * wave + j) * kNvTileK,
                                             16, 0, 0);
        }
    };

    // weights: A tile a of this wave = record groups g0 + 2a, g0 + 2a + 1
    bool valid[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) valid[a] = g0 + 2 * a + ((lane & 31) < 16 ? 0 : 1) < nrg;
    auto load_w = [&](int kb, typename PF::Frag (&wa)[NA]) {
#pragma unroll
        for (int a = 0; a < NA; ++a)
            PF::load(wa[a], base + (int64_t)(g0 + 2 * a) * gstride, gstride, kb, K, lane,
                     valid[a], A.res, A.res_scale);
    };
    // the lane's codebooks: small ones copied into LDS by the workgroup (gate
    // then up, or down), large ones read from L2; rows 16..31 of an A tile
    // are up rows in the gate/up pass
    const bool up_row = PHASE == 0 && (lane & 31) >= 16;
    const void* ctx = nullptr;
    if constexpr (PF::cb_lds(0) > 0) {
        _Float16* const pf_cb = pf_lds + NS * BM * kNvTileK;
        constexpr int NCH = PF::cb_lds(PHASE) / 16;        // 16-byte rows
        constexpr int PER = NCH / (PHASE == 0 ? 2 : 1);
        for (int i = tid; i < NCH; i += 64 * WV) {
            const uint8_t* src = A.cb8[PHASE == 0 ? i / PER : 2] + (int64_t)(i % PER) * 16;
            *reinterpret_cast<u32x4*>(pf_cb + (int64_t)i * 8) =
                *reinterpret_cast<const u32x4*>(src);
        }
        ctx = pf_cb + (up_row ? PER * 8 : 0);
    } else if constexpr (PF::kScales) {
        ctx = A.cb[PHASE == 0 ? (up_row ? 1 : 0) : 2] + (int64_t)it.ridx * A.cb_stride;
    }

    f32x16 acc[NA][NBM];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int q = 0; q < NBM; ++q) acc[a][q] = f32x16{};

    const int h = lane >> 5;
    // The main loop, specialised for the number of live 32-token B tiles so
    // that no branch sits between the decode and the MFMAs; register buffers
    // and LDS buffers alternate with a compile-time parity.
    auto run = [&](auto nb_c) {
        constexpr int NB = decltype(nb_c)::value;
        typename PF::Frag w[2][NA];
        load_w(0, w[0]);
#pragma unroll
        for (int b = 0; b < NS - 1; ++b)
            if (b < nkb) issue_x(b, b);
        // wait for W(0) and X(0); X(1 .. NS-2) may stay in flight
        if (NS == 3 && nkb > 1)
            __builtin_amdgcn_s_waitcnt(kVmcnt0 | JX);
        else
            __builtin_amdgcn_s_waitcnt(kVmcnt0);
        __syncthreads();
        // B reads: row (lane & 31) of each 32-token tile, logical chunk 8h + s
        const _Float16* xrow0 = xs + (lane & 31) * kNvTileK;
        auto step = [&](int kb, auto p_c) {
            constexpr int P = decltype(p_c)::value;
            const bool more = kb + 1 < nkb;
            // W(kb + 1) first, then X(kb + NS - 1): the wait below then leaves
            // only the newest token tile in flight
            if (more) load_w(kb + 1, w[P ^ 1]);
            const bool ahead = kb + NS - 1 < nkb;
            if (ahead) issue_x(kb + NS - 1, (kb + NS - 1) % NS);
            const _Float16* xb = xrow0 + (kb % NS) * (BM * kNvTileK);
            auto rd = [&](int s, int q) {
                const int cofs = 8 * ((8 * h + s) ^ (lane & 15));
                return *reinterpret_cast<const f16x8*>(xb + 32 * q * kNvTileK + cofs);
            };
#pragma unroll
            for (int s = 0; s < 8; ++s) {
#pragma unroll
                for (int j = 0; j < PF::NSUB; ++j) {
                    f16x8 av[NA];
#pragma unroll
                    for (int a = 0; a < NA; ++a) av[a] = PF::step(w[P][a], s, j, ctx);
#pragma unroll
                    for (int q = 0; q < NB; ++q) {
                        const f16x8 b = rd(s, q);
#pragma unroll
                        for (int a = 0; a < NA; ++a) acc[a][q] = mfma32(av[a], b, acc[a][q]);
                    }
                }
            }
            // W(kb + 1) and X(kb + 1) must have landed; with three buffers
            // X(kb + 2) may still be in flight
            if (NS == 3 && ahead)
                __builtin_amdgcn_s_waitcnt(kVmcnt0 | JX);
            else
                __builtin_amdgcn_s_waitcnt(kVmcnt0);
            __syncthreads();
        };
        for (int kb = 0; kb < nkb; kb += 2) {
            step(kb, std::integral_constant<int, 0>{});
            if (kb + 1 < nkb) step(kb + 1, std::integral_constant<int, 1>{});
        }
    };
    if constexpr (NBM == 2) {
        if (nbt == 1) run(std::integral_constant<int, 1>{});
        else run(std::integral_constant<int, 2>{});
    } else {
        switch (nbt) {
            case 1: run(std::integral_constant<int, 1>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            default: run(std::integral_constant<int, 4>{}); break;
        }
    }

    // epilogue: lane holds D[row 8(i/4) + 4h + i%4][token 32q + (lane & 31)]
#pragma unroll
    for (int q = 0; q < NBM; ++q) {
        const int tok = 32 * q + (lane & 31);
        if (q >= nbt || tok >= mcount) continue;
        const int64_t prow = it.r0 + it.m0 + tok;            // permuted row
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            const int ga = g0 + 2 * a;
            if constexpr (PF::kScales) {
                // per-output-row fp16 scales after the code tiles: acc element
                // e of this lane belongs to row (e / 4) * 8 + 4h + e % 4 of the
                // 32-row tile (record group ga + (e >= 8), its row (e/4 % 2) * 8
                // + 4h + e % 4)
                const _Float16* sp =
                    reinterpret_cast<const _Float16*>(base + (int64_t)nrg * gstride);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int r = ((e >> 2) & 1) * 8 + 4 * h + (e & 3);   // row in its group
                    const int g = ga + (e >> 3);
                    const int o = PHASE == 0 ? (g & 1) * A.I + 16 * (g >> 1) + r : 16 * g + r;
                    if (g < nrg) acc[a][q][e] *= (float)sp[o];
                }
            }
            if (PHASE == 0 && ROT) {
                if (ga >= nrg) continue;
                const int ch = 16 * (ga >> 1) + 4 * h;
                // gate rows ch..+3, ch+8..+11: acc i, i + 4; up: i + 8, i + 12
                float* gp = A.gu + prow * (2 * A.I) + ch;
                *reinterpret_cast<f32x4*>(gp) =
                    f32x4{acc[a][q][0], acc[a][q][1], acc[a][q][2], acc[a][q][3]};
                *reinterpret_cast<f32x4*>(gp + 8) =
                    f32x4{acc[a][q][4], acc[a][q][5], acc[a][q][6], acc[a][q][7]};
                *reinterpret_cast<f32x4*>(gp + A.I) =
                    f32x4{acc[a][q][8], acc[a][q][9], acc[a][q][10], acc[a][q][11]};
                *reinterpret_cast<f32x4*>(gp + A.I + 8) =
                    f32x4{acc[a][q][12], acc[a][q][13], acc[a][q][14], acc[a][q][15]};
            } else if (PHASE == 0) {
                if (ga >= nrg) continue;
                const int ch = 16 * (ga >> 1) + 4 * h;       // channel of rows 4h..4h+3
                f16x4 h0, h1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    h0[i] = (_Float16)(acc[a][q][i] * acc[a][q][i + 8] /
                                       (1.0f + expf(-acc[a][q][i])));
                    h1[i] = (_Float16)(acc[a][q][i + 4] * acc[a][q][i + 12] /
                                       (1.0f + expf(-acc[a][q][i + 4])));
                }
                _Float16* hp = A.h16 + prow * A.I + ch;
                *reinterpret_cast<f16x4*>(hp) = h0;
                *reinterpret_cast<f16x4*>(hp + 8) = h1;
            } else {
#pragma unroll
                for (int r8 = 0; r8 < 4; ++r8) {
                    const int r = 8 * r8 + 4 * h;            // row within the 32-row tile
                    if (ga + (r >> 4) >= nrg) continue;
                    f32x4 y = {acc[a][q][4 * r8], acc[a][q][4 * r8 + 1], acc[a][q][4 * r8 + 2],
                               acc[a][q][4 * r8 + 3]};
                    *reinterpret_cast<f32x4*>(A.y_perm + prow * A.H + 16 * ga + r) = y;
                }
            }
        }
    }
}

}  // namespace

namespace {

template <class PF, bool ID>
int launch_pf(const PrefillArgs& a, int64_t tk, int64_t active, int phase, hipStream_t s) {
    constexpr bool kId = ID;
    constexpr int BN = pf_bn<PF>();
    static_assert(PF::BM % 32 == 0 && PF::BM <= kBMMax, "token tile");
    // sum over experts of ceil(M_e / BM) <= T*k / BM + (number of active experts)
    const int64_t items = tk / PF::BM + active;
    if (items == 0) return MOE_OK;
    const int nrg = (phase == 0 ? 2 * a.I : a.H) / 16;
    const int64_t nnt = (nrg + BN / 16 - 1) / (BN / 16);
#if MOEQ_PF_ORDER == 0
    // 8 slices of ceil(items * nnt / 8) workgroups cover every item; slots past
    // the actual item count exit at once
    const int64_t nblocks = 8 * ((items * nnt + 7) / 8);
#else
    // each XCD takes every 8th item, nnt workgroups per item; slots past the
    // actual item count exit at once
    const int64_t nblocks = 8 * ((items + 7) / 8) * nnt;
#endif
    dim3 grid((unsigned)nblocks);
    // token-tile buffers, then the codebooks kept in LDS (at most 64 KB)
    const size_t lds = (size_t)kPrefillStages * PF::BM * kNvTileK * 2 + (size_t)PF::cb_lds(phase);
    if (phase == 0 && a.gu) {
        if constexpr (!kId)
            k_prefill<PF, 0, false, true><<<grid, 64 * kPrefillWaves, lds, s>>>(a);
    } else if (phase == 0) {
        k_prefill<PF, 0, ID><<<grid, 64 * kPrefillWaves, lds, s>>>(a);
    } else {
        k_prefill<PF, 1, ID><<<grid, 64 * kPrefillWaves, lds, s>>>(a);
    }
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

}  // namespace

int launch_ffn_prefill(const LayerView& L, int fmt, int n_fmt, const uint16_t* x16,
                       const int32_t* perm_src, const int32_t* offsets, int64_t T, int32_t k,
                       uint16_t* h16, float* y_perm, int phase, void* stream, float* gu) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    PrefillArgs a;
    a.pool = phase == 0 ? L.pool13[fmt] : L.pool2[fmt];
    a.stride = phase == 0 ? L.stride13[fmt] : L.stride2[fmt];
    for (int p = 0; p < 3; ++p) {
        a.cb[p] = L.cb[p];
        a.cb8[p] = L.cb8[p];
    }
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
    a.rows = (int)T;
    a.gu = phase == 0 ? gu : nullptr;
    a.res = phase == 0 ? L.res13 : L.res2;
    a.res_scale = L.res_scale;
    const int64_t tk = T * k;
    const int64_t act = tk < n_fmt ? tk : n_fmt;
    const bool id = offsets == nullptr;   // NVFP4 and BF16 only (prefill_fmt)
    switch (fmt) {
        case MOE_FMT_BF16:
            return id ? launch_pf<PfBf16, true>(a, tk, act, phase, s)
                      : launch_pf<PfBf16, false>(a, tk, act, phase, s);
        case MOE_FMT_VQ:
            return launch_pf<PfVq, false>(a, tk, act, phase, s);
        case MOE_FMT_VQ8:
        case MOE_FMT_VQ8_M1:
        case MOE_FMT_VQ8_M2:
        case MOE_FMT_VQ8_M3: {
            const int m = vq8_rate(fmt, L.vq8_m);
            if (m == 1) return launch_pf<PfVq8<1>, false>(a, tk, act, phase, s);
            if (m == 3) return launch_pf<PfVq8<3>, false>(a, tk, act, phase, s);
            return launch_pf<PfVq8<2>, false>(a, tk, act, phase, s);
        }
        case MOE_FMT_NVFP4R:
            return id ? launch_pf<PfNv2, true>(a, tk, act, phase, s)
                      : launch_pf<PfNv2, false>(a, tk, act, phase, s);
        default:
            return id ? launch_pf<PfNv, true>(a, tk, act, phase, s)
                      : launch_pf<PfNv, false>(a, tk, act, phase, s);
    }
}

}  // namespace moeq
