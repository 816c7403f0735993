// Internal declarations shared by the library's translation units.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "moeq.h"

namespace moeq {

// Per-thread detail of the last rejected call (read by moe_last_error).
void set_error(const std::string& msg);
int fail(int status, const std::string& msg);

// Record geometry ------------------------------------------------------------
//
// NVFP4 tile: 16 rows x 128 inputs = 1024 code bytes + 128 scale bytes.
//   code bytes: lane L (0..63) owns bytes [16L, 16L+16): row (L & 15),
//     inputs kb*128 + (L >> 4)*32 + [0, 32), canonical nibble order.
//   scale bytes: lane L owns bytes 1024 + [2L, 2L+2): the two E4M3 scales of
//     those 32 inputs.
// VQ tile: 16 rows x 256 inputs = 1024 code bytes.
//   lane L owns bytes [16L, 16L+16) = 8 uint16 codes: row (L & 15), groups
//     covering inputs kb*256 + (L >> 4)*64 + 8s + [0, 8), s = 0..7.
// VQ8 tile (m = 1, 2 or 3 uint8 codes per group): 16 rows x 256 inputs =
//   512 m code bytes; lane L owns bytes [8mL, 8mL + 8m): row (L & 15), the
//   groups of inputs kb*256 + (L >> 4)*64 + 8s + [0, 8), s = 0..7, each group's
//   m codes consecutive (code j of group s at byte m*s + j).
// BF16 tile: 16 rows x 128 inputs = 4096 bytes in 4 slices of 1024: slice j,
//   lane L owns bytes [1024j + 16L, +16) = 8 bf16 weights of row (L & 15),
//   inputs kb*128 + (L >> 4)*32 + 8j + [0, 8) (so one 16-byte load per lane
//   reads a contiguous 1 KB slice).
// A record is a sequence of row groups of 16 rows, each a sequence of tiles
// along the input dimension (padded with zero codes/scales).  Gate/up
// records interleave row groups: group 2j = gate rows 16j.., 2j+1 = up rows.
// VQ and VQ8 records end with the fp16 per-row scales (gate, up / down),
// padded to 256 bytes.
constexpr int kNvTileK = 128;
constexpr int kNvTileBytes = 1152;
constexpr int kNvScaleOff = 1024;
constexpr int kVqTileK = 256;
constexpr int kVqTileBytes = 1024;
constexpr int kVq8TileK = 256;
constexpr int kVq8TileBytesPerCode = 512;   // times m
constexpr int kBf16TileK = 128;
constexpr int kBf16TileBytes = 4096;

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

inline int64_t nv_tiles_k(int32_t kin) { return round_up(kin, kNvTileK) / kNvTileK; }
inline int64_t vq_tiles_k(int32_t kin) { return round_up(kin, kVqTileK) / kVqTileK; }

inline int64_t nv_matrix_bytes(int32_t n, int32_t kin) {
    return (int64_t)(n / 16) * nv_tiles_k(kin) * kNvTileBytes;
}
inline int64_t vq_codes_bytes(int32_t n, int32_t kin) {
    return (int64_t)(n / 16) * vq_tiles_k(kin) * kVqTileBytes;
}
inline int64_t vq8_codes_bytes(int32_t n, int32_t kin, int32_t m) {
    return (int64_t)(n / 16) * vq_tiles_k(kin) * kVq8TileBytesPerCode * m;
}
// NVFP4 record bytes (which = 0: gate/up, 1: down); also the offset of the
// residual plane inside a MOE_FMT_NVFP4R record.
inline int64_t nv_record_bytes(int which, int32_t H, int32_t I) {
    return which == 0 ? round_up(nv_matrix_bytes(2 * I, H), 256)
                      : round_up(nv_matrix_bytes(H, I), 256);
}
inline int64_t bf16_tiles_k(int32_t kin) { return round_up(kin, kBf16TileK) / kBf16TileK; }
inline int64_t bf16_matrix_bytes(int32_t n, int32_t kin) {
    return (int64_t)(n / 16) * bf16_tiles_k(kin) * kBf16TileBytes;
}

// Launchers (device code lives in the .hip files) ----------------------------
constexpr int kNumFmt = MOE_FMT_MAX + 1;   // format tags 1 .. MOE_FMT_MAX
// Small-codebook VQ at the layer's rate (MOE_FMT_VQ8) or an explicit one.
inline bool is_vq8(int fmt) {
    return fmt == MOE_FMT_VQ8 || (fmt >= MOE_FMT_VQ8_M1 && fmt <= MOE_FMT_VQ8_M3);
}
// Codes per 8-weight group of a small-codebook VQ format.
inline int vq8_rate(int fmt, int layer_vq8_m) {
    return fmt == MOE_FMT_VQ8 ? layer_vq8_m : fmt - MOE_FMT_VQ8_M1 + 1;
}
struct LayerView {
    int32_t E, H, I;
    int32_t vq8_m;
    const int32_t* rec;
    const uint8_t* pool13[kNumFmt];   // indexed by format tag
    const uint8_t* pool2[kNumFmt];
    int64_t stride13[kNumFmt];
    int64_t stride2[kNumFmt];
    const uint8_t* cb[3];       // VQ codebooks gate, up, down
    int64_t cb_stride;
    const uint8_t* cb8[3];      // VQ8 codebooks gate, up, down: [m][256][8] fp16
    int64_t res13, res2;        // MOE_FMT_NVFP4R: residual plane offset in a record
    float res_scale;            // ... and its decode factor 2^-nvfp4r_shift
    const uint8_t* rot;         // rotation sign bits per expert (NULL: not rotated)
    int64_t rot_stride;         // bytes per expert: (2H + 3I) / 8
    int32_t rot_in2;            // Hadamard block of the down input: 128 or 512
};

int launch_route_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                      int32_t* ids, float* w, void* stream);
int launch_permute(const int32_t* ids, int64_t T, int32_t k, int32_t E,
                   int32_t* counts, int32_t* offsets, int32_t* perm_src,
                   int32_t* inv_perm, void* ws, void* stream);
size_t permute_ws_bytes(int64_t T, int32_t k, int32_t E);
bool route_permute_fused_ok(int64_t T, int32_t k);
int launch_route_permute(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids,
                         float* w, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                         int32_t* inv_perm, void* stream);
int launch_combine(const float* y_perm, const int32_t* inv_perm, const float* w,
                   const float* y_shared, int64_t T, int32_t k, int32_t H, float* out,
                   void* stream);
// A rotated layer: the down outputs y' (not yet rotated back) rotated back
// per slot with its expert's down-output signs and combined as launch_combine
// does, the same bits as launch_rot_out followed by launch_combine
// (inv_perm NULL: slot (t, j) is row t*k + j).
int launch_combine_rot(const LayerView& L, const float* y_perm, const int32_t* inv_perm,
                       const int32_t* ids, const float* w, const float* y_shared, int64_t T,
                       int32_t k, float* out, void* stream);
int launch_x_to_f16(const uint16_t* x, int64_t n, uint16_t* x16, void* stream);
// gu != NULL (gate/up of a rotated layer): x is the fp16 rotated rows
// [T*k, H] in permuted order, and the raw fp32 products g | u go to
// gu [T*k, 2I] instead of h.
int launch_ffn_decode(const LayerView& L, int fmt, int n_fmt, const uint16_t* x_bf16,
                      const int32_t* perm_src, const int32_t* offsets, int64_t T,
                      int32_t k, uint16_t* h16, float* y_perm, int phase,
                      void* stream, float* gu = nullptr);
// A mixed layer of NVFP4 and one VQ form (decode batches): both formats'
// gate/up (phase 0) or down (phase 1) work in one launch, when both pick the
// same input split (ffn_decode_pair_ok); the same bits as the two launches.
bool ffn_decode_pair_ok(const LayerView& L, int fmt1, int n1, int fmt2, int n2, int64_t T,
                        int32_t k);
int launch_ffn_decode_pair(const LayerView& L, int fmt1, int n1, int fmt2, int n2,
                           const uint16_t* x_bf16, const int32_t* perm_src,
                           const int32_t* offsets, int64_t T, int32_t k, uint16_t* h16,
                           float* y_perm, int phase, void* stream);
// The one expert of a shared-expert layer through the identity map (rows
// 0 .. T-1 are tokens 0 .. T-1): phase 0 writes fp32 partial g | u to part
// (shared_part_bytes) and then h, phase 1 writes y [T, H].
#ifndef MOEQ_SH_TARGET
#define MOEQ_SH_TARGET 512
#endif
constexpr int kSharedMaxSplit = 16;                  // workgroups splitting the gate/up inputs
constexpr int kSharedTargetBlocks = MOEQ_SH_TARGET;  // gate/up workgroups aimed for
// Bytes of the fp32 partial sums the decode path of a one-expert layer of
// format fmt writes for T tokens: nsplit x T x 2I x 4 with the split that
// launch_shared_decode takes; 0 where the grouped GEMM runs instead.
size_t shared_part_bytes(int fmt, int64_t T, int32_t H, int32_t I);
int launch_shared_decode(const LayerView& L, int fmt, const uint16_t* x_bf16, int64_t T,
                         uint16_t* h16, float* part, float* y, int phase, void* stream);
// Experts at T >= kPrefillMinTokens use the grouped-GEMM kernels, every
// format for routed layers; the identity map of a one-expert layer
// (perm_src == offsets == NULL) only for NVFP4 (one or two planes) and BF16.
constexpr int64_t kPrefillMinTokens = 128;
inline bool prefill_fmt(int fmt, bool identity) {
    return !identity || fmt == MOE_FMT_NVFP4 || fmt == MOE_FMT_BF16 || fmt == MOE_FMT_NVFP4R;
}
int launch_ffn_prefill(const LayerView& L, int fmt, int n_fmt, const uint16_t* x16,
                       const int32_t* perm_src, const int32_t* offsets, int64_t T, int32_t k,
                       uint16_t* h16, float* y_perm, int phase, void* stream,
                       float* gu = nullptr);
// Rotated layers: x' = rotated rows of x per assignment (fp16 [T*k, H]);
// h' from the raw gate/up products gu (fp16 [rows, I]); y rotated back in
// place (fp32 [rows, H]).
int launch_rot_in(const LayerView& L, const uint16_t* x_bf16, const int32_t* perm_src,
                  const int32_t* offsets, int64_t T, int32_t k, uint16_t* xrot, void* stream);
// row_ids != NULL: rows in assignment order, row r of expert row_ids[r]
// (offsets unused).
int launch_rot_mid(const LayerView& L, const float* gu, const int32_t* offsets, int64_t rows,
                   uint16_t* h16, void* stream, const int32_t* row_ids = nullptr);
int launch_rot_out(const LayerView& L, float* y, const int32_t* offsets, int64_t rows,
                   void* stream);
// The small-batch fused layer (single-format layers, E <= 256, k <= 8,
// T*k <= kSmallFusedAssign): gate/up with the routing inside (topk_ids /
// topk_w written, h16 [T*k, I] in token order), then down + gated combine
// (+ y_shared) into out [T, H].  A rotated layer (H <= kSmallRotMaxH) takes
// four launches and after h16 (rounded up to 256 bytes) the raw products
// [T*k, 2I] fp32 and then y' [T*k, H] fp32 (small_rot_ws_bytes in all).
#ifndef MOEQ_SMALL_ASSIGN
#define MOEQ_SMALL_ASSIGN 16
#endif
constexpr int64_t kSmallFusedAssign = MOEQ_SMALL_ASSIGN;
constexpr int32_t kSmallRotMaxH = 12288;   // the rotated row in LDS: 2H bytes
inline size_t small_rot_ws_bytes(int64_t T, int32_t k, int32_t H, int32_t I) {
    const int64_t tk = T * k;
    return (size_t)(round_up(tk * I, 128) * 2 + round_up(tk * 2 * I, 64) * 4 + tk * H * 4);
}
int launch_layer_small(const LayerView& L, int fmt, const uint16_t* x_bf16, const float* logits,
                       int64_t T, int32_t k, int32_t* topk_ids, float* topk_w, uint16_t* h16,
                       const float* y_shared, float* out, void* stream);
// The same with a BF16 shared expert SL (E == 1, same H): out = routed sum +
// the shared FFN; sh_h16 [T, SL.I] fp16 and sh_part (shared_part_bytes) are
// its workspace.
int launch_layer_small_shared(const LayerView& L, int fmt, const LayerView& SL,
                              const uint16_t* x_bf16, const float* logits, int64_t T, int32_t k,
                              int32_t* topk_ids, float* topk_w, uint16_t* h16, uint16_t* sh_h16,
                              float* sh_part, float* out, void* stream);
int launch_dequant(const LayerView& L, int fmt, int32_t rec_index, int32_t proj,
                   float* out, void* stream);
int launch_probe_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, void* stream);

}  // namespace moeq
