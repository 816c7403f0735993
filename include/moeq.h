/*
 * moeq.h -- C ABI of the routed-expert MoE forward over low-bit expert
 * weights, for AMD Instinct MI355X (gfx950).
 *
 * The forward, for T tokens with hidden size H, E experts of intermediate
 * size I and k experts per token:
 *
 *   moe_route_topk    logits [T, E]            -> topk_ids [T, k], topk_w [T, k]
 *   moe_permute       topk_ids                 -> counts, offsets, perm_src, inv_perm
 *   moe_expert_ffn_q  x [T, H], perm_src, ...  -> y_perm [T*k, H]
 *   moe_combine       y_perm, inv_perm, topk_w -> out [T, H]
 *
 * (moe_layer_forward runs the four in one call, fused for decode batches),
 * and, for layers with a shared expert that every token passes through,
 *
 *   moe_shared_ffn      x [T, H]                   -> y_shared [T, H]
 *   moe_combine_shared  y_perm, inv_perm, topk_w,
 *                       y_shared                   -> out [T, H]
 *
 * (moe_layer_forward_shared runs the routed layer and its shared expert in
 * one call).
 *
 * Passages these calls follow (titles and sections of the source pages):
 *   - 256 routed experts per MoE layer, 8 active per token:
 *     "GLM-5-NVFP4-MTP", Model Description.
 *   - only the expert MLP (gate, up, down projections) is low-bit:
 *     "GLM-5-NVFP4-MTP", What's quantized.
 *   - NVFP4 = 4-bit E2M1 codes with an FP8 (E4M3) scale per 16 elements:
 *     "GLM-5-NVFP4-MTP", Model Description.
 *   - AQLM-style vector quantization, per-group codes into a shared codebook:
 *     "GLM-5.2 mixed-bit VQ (AQLM) ~1.90 bpw", What it is.
 *   - a per-expert tier map that the runtime must honour, failing closed
 *     rather than decoding with the wrong format:
 *     "GLM-5.3-EXL3-TR3-3.42bpw", What is quantized / Serving;
 *     "GLM-5.3-Flash-TR3-8bpw (K8)", Why K8 uses the native eager path.
 *   - records addressed by expert id at a fixed stride:
 *     "GLM-5.3 Vision NestQuant 1.75-4 bit", Contents.
 *   - a fixed expert-combine order (the order changes the bits):
 *     "GLM-5.3-Flash-TR3-8bpw (K8)", Fidelity / Excess over control.
 *   - stored matrices rotated by random signs and a Hadamard-128 transform
 *     on both sides, the activations rotated online, with the wide variant
 *     of the down projection's input side (one Hadamard-512 per 512
 *     intermediate channels): "GLM-5.3 Vision NestQuant 1.75-4 bit", Method.
 *   - a nested two-level format, a base plus a residual plane that lifts an
 *     expert to the higher tier at serving time with the base bytes
 *     unchanged: "GLM-5.3 Vision NestQuant 1.75-4 bit", introduction.
 *   - BF16 shared experts beside the low-bit routed ones:
 *     "GLM-5.3-EXL3-TR3-3.42bpw", What is quantized; "GLM-5-NVFP4-MTP",
 *     What's quantized (shared experts are among the non-expert weights
 *     kept in BF16).
 *
 * Conventions
 *   - Pointers marked [device] are device memory on the current HIP device;
 *     [host] pointers are host memory.  The caller allocates and owns every
 *     buffer.  The library never allocates, frees or synchronises, keeps no
 *     state between calls and is safe to call from several threads.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device calls are
 *     stream-ordered and asynchronous: they return after the launch.
 *   - Arguments are checked on the host before any launch.  A rejected call
 *     launches nothing and returns a negative status; moe_last_error() then
 *     describes it (per thread).  There is no fallback path: an unsupported
 *     format or shape is an error (MOE_EUNSUPPORTED), never a silent decode
 *     with another format.
 *   - T == 0 is valid for every device call; moe_permute then writes
 *     counts = 0 and offsets = 0, the other calls launch nothing.
 *   - Device-side preconditions that cannot be checked without reading device
 *     memory (logits not NaN; topk_ids in [0, E) and the k ids of a token
 *     distinct, as moe_route_topk writes them; perm_src/offsets produced by
 *     moe_permute for the same topk_ids; the per-expert record table agreeing
 *     with the host tier map) are the caller's; violating them gives
 *     unspecified results but no out-of-bounds access beyond the buffers'
 *     stated sizes for ids in range.  (With a token naming one expert twice,
 *     that expert can hold more than T rows; the decode-size FFN kernels,
 *     T < 128, compute the first T of them only.)
 *   - Operand range: the expert FFNs multiply on the matrix cores' fp16
 *     operands, so each activation x and each SwiGLU output h must lie in
 *     fp16's finite range, |v| <= 65504 (every bf16 value up to 65280 is
 *     exact there; below 2^-14 a value is rounded to fp16's subnormal grid,
 *     error < 2^-25).  A token with a value beyond the range gets a
 *     non-finite output row; the other tokens' rows are unaffected, since no
 *     product mixes two tokens.
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
#define MOE_OK            0
#define MOE_EINVAL       -1   /* bad argument: null pointer, size, shape */
#define MOE_EUNSUPPORTED -2   /* format / shape this library does not decode */
#define MOE_EWORKSPACE   -3   /* workspace smaller than *_workspace_bytes() */
#define MOE_EHIP         -4   /* a HIP launch failed */

/* ---------------------------------------------------------------- formats */
#define MOE_FMT_NVFP4 1       /* E2M1 codes + E4M3 scale per 16 inputs */
#define MOE_FMT_VQ    2       /* 8-wide groups, uint16 codes, fp16 codebook,
                                 fp16 scale per output channel */
#define MOE_FMT_VQ8   3       /* 8-wide groups, M = 1, 2 or 3 uint8 codes into M
                                 256-entry fp16 codebooks whose rows are
                                 summed, fp16 scale per output channel
                                 (M bits per weight) */
#define MOE_FMT_BF16  4       /* bf16 weights as stored, no scales */
#define MOE_FMT_NVFP4R 5      /* nested two-level NVFP4: an NVFP4 base plane
                                 plus an NVFP4 residual plane on top of it
                                 (weights = base + residual) */
#define MOE_FMT_VQ8_M1 6      /* MOE_FMT_VQ8 at an explicit rate: 1, 2 or 3 */
#define MOE_FMT_VQ8_M2 7      /* uint8 codes per group (bits per weight), */
#define MOE_FMT_VQ8_M3 8      /* whatever the layer's vq8_m; one pool each */
#define MOE_FMT_MAX   8       /* largest format tag */

#define MOE_PROJ_GATE 0
#define MOE_PROJ_UP   1
#define MOE_PROJ_DOWN 2

/* Limits of this library. */
#define MOE_MAX_E     1024    /* experts per layer */
#define MOE_MAX_K     16      /* experts per token */
#define MOE_VQ_NCODE  65536   /* codebook entries (uint16 codes) */
#define MOE_VQ8_NCODE 256     /* entries of each small codebook (uint8 codes) */
#define MOE_VQ8_MAX_M 3       /* small codebooks per group */
#define MOE_ROT_BLOCK 128     /* Hadamard block of rotated layers */
#define MOE_ROT_BLOCK_WIDE 512 /* the down-input block of the wide variant */

/*
 * A packed expert layer.  Host struct; the pointers inside are [device]
 * unless noted.
 *
 * Every expert has a format tag.  Experts of one format are stored as
 * fixed-size records in that format's pool: the record of expert e is at
 * pool + index(e) * stride, where index(e) is e's rank among the experts of
 * its format (so a single-format layer has index(e) = e).  Record sizes are
 * given by moe_record_bytes() and their bytes by the moe_pack_* calls.
 *
 *   fmt_host   [host]   uint8 [E]: a format tag (MOE_FMT_*) per expert.
 *   rec_dev    [device] int32 [E]: (fmt << 24) | index(e), as written by
 *                       moe_record_table() from the same fmt_host.
 *   nvfp4_w13 / nvfp4_w2   pool bases of NVFP4 gate/up and down records;
 *   vq_w13 / vq_w2         pool bases of VQ gate/up and down records;
 *   *_stride               bytes between consecutive records of a pool
 *                          (>= moe_record_bytes(), multiple of 256).
 *   vq_codebook[p]  fp16 [65536, 8] codebook of projection p (gate, up,
 *                   down).  vq_codebook_stride = bytes between the codebooks
 *                   of consecutive VQ records (index(e)); 0 means one
 *                   codebook per projection shared by every expert.
 *   vq8_m           codes per group of the MOE_FMT_VQ8 experts (1, 2 or 3);
 *                   any value if the layer has none.
 *   vq8_w13 / vq8_w2   pool bases of the MOE_FMT_VQ8 records;
 *   vq8_codebook[p] fp16 [n][256][8]: the small codebooks of projection p,
 *                   shared by every small-codebook VQ expert of the layer; an
 *                   expert at rate m (MOE_FMT_VQ8: vq8_m; MOE_FMT_VQ8_Mm: m)
 *                   reads codebooks 0 .. m-1, so n must be at least the
 *                   largest rate in the layer.
 *   vq8r_w13[m-1] / vq8r_w2[m-1]  pool bases of the MOE_FMT_VQ8_Mm records
 *                   (moe_record_bytes_vq8(.., m) each), m = 1, 2, 3: a
 *                   layer's small-codebook VQ experts at mixed rates, the
 *                   rate chosen per expert ("GLM-5.2 mixed-bit VQ (AQLM)
 *                   ~1.90 bpw", What it is: one layer's modules at 1, 2 and
 *                   3 bits, chosen per module).
 *   bf16_w13 / bf16_w2 pool bases of the MOE_FMT_BF16 records.
 *   nvfp4r_w13 / nvfp4r_w2  pool bases of the MOE_FMT_NVFP4R records: each
 *                   record is an NVFP4 record (the base plane) followed by
 *                   the NVFP4 record of the residual plane, each of
 *                   moe_record_bytes(MOE_FMT_NVFP4, ...) bytes.  A resident
 *                   layer may point nvfp4_w13 / nvfp4_w2 at the same pools
 *                   with the same strides: an expert tagged MOE_FMT_NVFP4
 *                   then runs on its base plane alone, and retagging it
 *                   MOE_FMT_NVFP4R adds the residual plane on top, with the
 *                   base bytes unchanged ("GLM-5.3 Vision NestQuant 1.75-4
 *                   bit", introduction: a nested two-level format whose
 *                   residual plane lifts an expert to the higher tier at
 *                   serving time).
 *   nvfp4r_shift    0 .. 14: the residual plane holds the residual times
 *                   2^nvfp4r_shift (a per-layer power of two that brings its
 *                   small block maxima into the E4M3 scales' normal range)
 *                   and is decoded times 2^-nvfp4r_shift; every decoded value
 *                   stays exact in fp16.  Any value if the layer has no
 *                   MOE_FMT_NVFP4R experts.
 *   rot_signs       NULL: the stored matrices are the weights.  Otherwise
 *                   every expert's matrices are stored rotated,
 *                   W_rot = R_out W R_in^T with R = blockdiag(H_128/sqrt(128))
 *                   diag(s) ("GLM-5.3 Vision NestQuant 1.75-4 bit", Method:
 *                   random signs + Hadamard-128 on both sides of each matrix),
 *                   and the FFN rotates activations online.  [device] uint8,
 *                   moe_rot_sign_bytes(H, I) per expert at e * that stride,
 *                   from moe_pack_rot_signs: the sign bits of the gate/up
 *                   input (shared by gate and up), the gate output, the up
 *                   output, the down input and the down output.  Needs H and
 *                   I multiples of 128.
 *   rot_in2_block   the Hadamard block of the down projection's input side
 *                   of a rotated layer: 0 or MOE_ROT_BLOCK (128, like every
 *                   other side), or MOE_ROT_BLOCK_WIDE (512: R_in2 =
 *                   blockdiag(H_512/sqrt(512)) diag(s), the page's variant
 *                   for the down projections of some layers -- random signs
 *                   and one Hadamard-512 per tensor-parallel shard of the
 *                   intermediate dimension, with a flat input-channel scale,
 *                   "GLM-5.3 Vision NestQuant 1.75-4 bit", Method; needs I a
 *                   multiple of 512).  Any other value: MOE_EUNSUPPORTED.
 *                   Ignored when rot_signs is NULL.
 *   record_mode     MOE_REC_COMPACT: index(e) = e's rank among the experts of
 *                   its format (rec from moe_record_table);
 *                   MOE_REC_RESIDENT: every pool that is used holds a record for
 *                   every expert at slot e, index(e) = e (rec from
 *                   moe_record_table_resident).  A resident layer switches an
 *                   expert's tier between calls by rewriting fmt_host[e] and
 *                   rec_dev[e] only ("GLM-5.3 Vision NestQuant 1.75-4 bit",
 *                   introduction and Serving: experts move between bit tiers
 *                   at serve time; "GLM-5.3-EXL3-TR3-3.42bpw", What is
 *                   quantized: the per-expert tier map).  Launch sizes follow
 *                   the number of experts per format, so a HIP graph captured
 *                   before a switch stays valid only if those counts are
 *                   unchanged (a swap of tiers).
 *
 * Unused pools (no expert of that format) may be NULL.
 */
typedef struct moe_qlayer {
    int32_t E, H, I;
    int32_t vq8_m;
    const uint8_t* fmt_host;
    const int32_t* rec_dev;
    const void* nvfp4_w13;  int64_t nvfp4_w13_stride;
    const void* nvfp4_w2;   int64_t nvfp4_w2_stride;
    const void* vq_w13;     int64_t vq_w13_stride;
    const void* vq_w2;      int64_t vq_w2_stride;
    const void* vq_codebook[3];
    int64_t vq_codebook_stride;
    const void* vq8_w13;    int64_t vq8_w13_stride;
    const void* vq8_w2;     int64_t vq8_w2_stride;
    const void* vq8_codebook[3];
    const void* bf16_w13;   int64_t bf16_w13_stride;
    const void* bf16_w2;    int64_t bf16_w2_stride;
    int32_t record_mode;
    int32_t rot_in2_block;
    const uint8_t* rot_signs;
    const void* nvfp4r_w13; int64_t nvfp4r_w13_stride;
    const void* nvfp4r_w2;  int64_t nvfp4r_w2_stride;
    int32_t nvfp4r_shift;
    int32_t reserved2;
    const void* vq8r_w13[3]; int64_t vq8r_w13_stride[3];
    const void* vq8r_w2[3];  int64_t vq8r_w2_stride[3];
} moe_qlayer;

#define MOE_REC_COMPACT   0
#define MOE_REC_RESIDENT  1

/* ------------------------------------------------------------- messages */

/* Static text for a status code. */
const char* moe_strerror(int status);
/* Detail of the last rejected call on this thread ("" if none). */
const char* moe_last_error(void);

/* -------------------------------------------------------------- routing */

/*
 * moe_route_topk -- per token, the k experts with the largest router logits
 * and their softmax weights renormalised over the chosen k.
 *   ("GLM-5-NVFP4-MTP", Model Description: 8 of 256 experts per token.)
 *
 *   logits    [device] fp32 [T, E], row-major.
 *   topk_ids  [device] int32 [T, k] out: ids[t, j] = expert of rank j.
 *             Ranking: larger logit first; equal logits -> lower expert id
 *             first; -0.0 and +0.0 are equal.
 *   topk_w    [device] fp32 [T, k] out: w[t, j] = exp(l_j - l_0) /
 *             sum_{i<k} exp(l_i - l_0) (fp32 arithmetic).
 *   Limits: 1 <= E <= MOE_MAX_E, 1 <= k <= min(E, MOE_MAX_K), T >= 0.
 *   Precondition: no NaN logits, and each token's largest logit is finite
 *   (other logits may be -inf; they then get weight 0).
 */
int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                   int32_t* topk_ids, float* topk_w, void* stream);

/* -------------------------------------------------------------- permute */

/* Workspace bytes moe_permute needs for these sizes (may be 0). */
size_t moe_permute_workspace_bytes(int64_t T, int32_t k, int32_t E);

/*
 * moe_permute -- group the T*k assignments by expert (a stable counting sort).
 *   (The pages' serving stacks run the routed experts through grouped MoE
 *   runners, which gather each expert's tokens into one contiguous group
 *   before its expert GEMMs: "GLM-5.3-Flash-TR3-8bpw (K8)", Serving --
 *   live-qualified turnkey profile (a Triton MoE runner behind an all-to-all);
 *   "GLM-5-NVFP4-MTP", How to Run (a CUTLASS MoE runner backend).)
 *   Assignment a = t*k + j goes to expert e_a = topk_ids[a].  moe_permute
 *   itself takes any ids in [0, E); the FFN calls that use its output need a
 *   token's k ids distinct (see Conventions).
 *   counts   [device] int32 [E] out: number of assignments per expert.
 *   offsets  [device] int32 [E+1] out: exclusive prefix sum of counts,
 *            offsets[E] = T*k.
 *   perm_src [device] int32 [T*k] out: for each expert in ascending id, its
 *            assignments in ascending a.  Row i of y_perm belongs to token
 *            perm_src[i] / k.
 *   inv_perm [device] int32 [T*k] out: inv_perm[perm_src[i]] = i.
 *   ws       [device] workspace of >= moe_permute_workspace_bytes() bytes
 *            (NULL allowed when that is 0).
 *   Limits: as moe_route_topk; T*k < 2^31.
 *   The result is unique, so it is bit-identical run to run.
 */
int moe_permute(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E,
                int32_t* counts, int32_t* offsets, int32_t* perm_src,
                int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_permute -- moe_route_topk followed by moe_permute, with the
 * same outputs bit for bit.  For T*k <= 64 (a decode step) both run in one
 * launch of one workgroup (the ids never leave the chip between the two
 * steps); larger batches run the two steps' own kernels.  Same arguments,
 * limits and errors as the two calls; ws/ws_bytes as for moe_permute
 * (moe_permute_workspace_bytes gives the size; it is 0, and ws may be NULL,
 * for T*k <= 4096).
 */
int moe_route_permute(const float* logits, int64_t T, int32_t E, int32_t k,
                      int32_t* topk_ids, float* topk_w, int32_t* counts,
                      int32_t* offsets, int32_t* perm_src, int32_t* inv_perm,
                      void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ expert FFN */

/* Workspace bytes moe_expert_ffn_q needs (the SwiGLU activations h, the fp16
 * copy of x, and for a rotated layer the rotated x rows and the gate/up
 * products). */
size_t moe_ffn_workspace_bytes(const moe_qlayer* layer, int64_t T, int32_t k);

/*
 * moe_expert_ffn_q -- the expert MLP for every assignment, with the weights
 * decoded in registers from each expert's own format.
 *   ("GLM-5-NVFP4-MTP", What's quantized: gate, up and down projections.)
 *
 *   For row i of the permuted order, with e the expert whose offsets range
 *   holds i and t = perm_src[i] / k:
 *     g = W_gate[e] x_t,  u = W_up[e] x_t      (I outputs each, K = H)
 *     h = silu(g) * u = g * u / (1 + exp(-g))
 *     y_perm[i] = W_down[e] h                  (H outputs, K = I)
 *
 *   x        [device] bf16 [T, H] as uint16 bits, token order.
 *   perm_src [device] int32 [T*k], offsets [device] int32 [E+1]: from
 *            moe_permute, for ids with a token's k experts distinct (so no
 *            expert holds more than T rows).
 *   y_perm   [device] fp32 [T*k, H] out.
 *   ws       [device] >= moe_ffn_workspace_bytes() bytes, 256-byte aligned.
 *
 *   Arithmetic: the matrix cores multiply fp16 operands and accumulate in
 *   fp32.  Decoded NVFP4 and VQ weights are exact in fp16 (an E2M1 value
 *   times an E4M3 scale; fp16 codebook entries, the per-channel scale applied
 *   in fp32 after the dot product); bf16 weights and x are converted to fp16
 *   (exact for 2^-17 <= |v| <= 65504 with 8 significant bits; smaller
 *   magnitudes round to fp16's subnormal grid, spacing 2^-24); h enters the
 *   down product as fp16.
 *   Rotated layers (rot_signs != NULL): x_t is rotated per assignment with
 *   its expert's input signs (x' = H_128 (s x) / 16, fp16), the stored
 *   matrices multiply x', the gate and up products are rotated back
 *   (g = s H_128 g' / 8) before SwiGLU, h is rotated for the down product
 *   (h' = H_128 (s h) / 16; with rot_in2_block 512, h' = H_512 (s h) / 32)
 *   and its output rotated back (y = s H_128 y' / 8); the powers of two make
 *   the rotations' 1/sqrt(128) and 1/sqrt(512) factors exact (16 * 8 = 128,
 *   32 * 8 = 256 = sqrt(128 * 512)).
 *   Requirements: H and I multiples of 16 (of 128 for a rotated layer);
 *   every format tag in layer->fmt_host must be one of MOE_FMT_*, else
 *   MOE_EUNSUPPORTED; every pool that a tag refers to must be non-NULL.
 */
int moe_expert_ffn_q(const moe_qlayer* layer, const uint16_t* x_bf16,
                     const int32_t* perm_src, const int32_t* offsets,
                     int64_t T, int32_t k, float* y_perm,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * The two halves of moe_expert_ffn_q, for callers that keep h themselves
 * (or time the halves apart).  moe_expert_ffn_q(...) is exactly
 * moe_expert_gateup_q into a workspace h followed by moe_expert_down_q.
 *
 * moe_expert_gateup_q -- h[i] = silu(W_gate[e] x_t) * (W_up[e] x_t) for every
 *   permuted row i (e, t as above), written as fp16 to
 *   h_f16 [device] [T*k, I] (for a rotated layer: h' = H_128 (s h) / 16, or
 *   H_512 (s h) / 32 with rot_in2_block 512, the down product's input).  ws [device] >= moe_gateup_workspace_bytes(),
 *   256-byte aligned (holds the fp16 copy of x, or the rotated rows).
 * moe_expert_down_q -- y_perm[i] = W_down[e] h[i] (fp32 [T*k, H]) from
 *   h_f16 [device] [T*k, I] and offsets [device] [E+1].
 * Same requirements and errors as moe_expert_ffn_q.
 */
size_t moe_gateup_workspace_bytes(const moe_qlayer* layer, int64_t T, int32_t k);
int moe_expert_gateup_q(const moe_qlayer* layer, const uint16_t* x_bf16,
                        const int32_t* perm_src, const int32_t* offsets,
                        int64_t T, int32_t k, uint16_t* h_f16,
                        void* ws, size_t ws_bytes, void* stream);
int moe_expert_down_q(const moe_qlayer* layer, const uint16_t* h_f16,
                      const int32_t* offsets, int64_t T, int32_t k,
                      float* y_perm, void* stream);

/* -------------------------------------------------------- shared expert */

/* Workspace bytes moe_shared_ffn needs (h, and x as fp16 for T >= 128). */
size_t moe_shared_ffn_workspace_bytes(const moe_qlayer* shared, int64_t T);

/*
 * moe_shared_ffn -- the shared expert, an expert that every token passes
 * through with weight 1:  y_shared[t] = W_down (silu(W_gate x_t) * W_up x_t).
 *   ("GLM-5.3-EXL3-TR3-3.42bpw", What is quantized: the layers keep BF16
 *   shared experts beside the routed ones.)
 *
 *   shared   a one-expert layer (E == 1) in any format, normally
 *            MOE_FMT_BF16; its I is the shared expert's intermediate size.
 *   x        [device] bf16 [T, H] bits, token order.
 *   y_shared [device] fp32 [T, H] out.
 *   ws       [device] >= moe_shared_ffn_workspace_bytes(), 256-byte aligned.
 *   The same kernels, arithmetic and errors as moe_expert_ffn_q with
 *   perm_src = (0, 1, .., T-1), offsets = (0, T) and k = 1, which this call
 *   implies without reading them from memory.
 */
int moe_shared_ffn(const moe_qlayer* shared, const uint16_t* x_bf16, int64_t T,
                   float* y_shared, void* ws, size_t ws_bytes, void* stream);

/* -------------------------------------------------------------- combine */

/*
 * moe_combine -- out[t] = sum_{j=0}^{k-1} topk_w[t, j] * y_perm[inv_perm[t*k+j]],
 * summed in ascending j in fp32, one writer per output element (no atomics),
 * so the result is bit-identical run to run.
 *   ("GLM-5.3-Flash-TR3-8bpw (K8)", Fidelity: the combine order changes the
 *   bits, so it is fixed.)
 *   y_perm [device] fp32 [T*k, H]; inv_perm [device] int32 [T*k];
 *   topk_w [device] fp32 [T, k]; out [device] fp32 [T, H] out.
 */
int moe_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w,
                int64_t T, int32_t k, int32_t H, float* out, void* stream);

/*
 * moe_combine_shared -- moe_combine with the shared expert's output added
 * after the routed sum:
 *   out[t] = (sum_{j=0}^{k-1} topk_w[t, j] * y_perm[inv_perm[t*k+j]]) + y_shared[t]
 * (the routed sum in ascending j in fp32, then one fp32 add; one writer per
 * element).  y_shared [device] fp32 [T, H] (from moe_shared_ffn); the other
 * arguments as moe_combine.
 */
int moe_combine_shared(const float* y_perm, const int32_t* inv_perm, const float* topk_w,
                       const float* y_shared, int64_t T, int32_t k, int32_t H, float* out,
                       void* stream);

/* -------------------------------------------------------- whole layer */

/*
 * moe_layer_forward -- the whole routed layer in one call: moe_route_topk,
 * moe_permute, moe_expert_ffn_q and moe_combine (moe_combine_shared when
 * y_shared is not NULL), with every intermediate in the workspace.
 * (The routed-expert forward: "GLM-5-NVFP4-MTP", Model Description and
 * What's quantized.)
 *
 *   layer      as for moe_expert_ffn_q.
 *   x_bf16     [device] bf16 [T, H]; logits [device] fp32 [T, E].
 *   y_shared   [device] fp32 [T, H] or NULL: a shared expert's output
 *              (moe_shared_ffn), added after the routed sum.
 *   topk_ids, topk_w  [device] [T, k] out, as moe_route_topk writes them.
 *   out        [device] fp32 [T, H] out.
 *   workspace  [device] >= moe_layer_forward_workspace_bytes(layer, T, k)
 *              bytes, 256-byte aligned; contents on return unspecified.
 *
 * Small batches of single-format layers (T*k <= 16, k <= 8, E <= 256:
 * decode) take a fused path of two launches and no permutation: the gate/up
 * kernel ranks the token's experts from the logits itself, the down kernel
 * forms the gated sum in ascending j.  A rotated layer (H <= 12288) takes
 * four: the gate/up kernel also rotates the token's row for its expert, then
 * the middle rotation, the down pass per slot, and the combine rotating each
 * slot's output back.  Its results are the bits of the step-by-step calls on
 * the same inputs (each expert's rows, partial sums, rotations and the
 * combine are taken in the same order).  Other batches run the step-by-step
 * calls (a rotated layer's combine rotating the down outputs back, with the
 * same bits as moe_expert_down_q's rotation followed by moe_combine).
 * Errors as for those calls (checked before any launch).
 */
size_t moe_layer_forward_workspace_bytes(const moe_qlayer* layer, int64_t T, int32_t k);
int moe_layer_forward(const moe_qlayer* layer, const uint16_t* x_bf16, const float* logits,
                      int64_t T, int32_t k, const float* y_shared, int32_t* topk_ids,
                      float* topk_w, float* out, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * moe_layer_forward_static -- moe_layer_forward without a workspace argument:
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that must not allocate, harnesses that forbid it).
 * Its workspace is a device array inside the library, MOE_STATIC_WS_BYTES
 * bytes per GPU, which each GPU the library runs on holds until the process
 * ends.  The caller still passes the inputs and outputs, as for
 * moe_layer_forward (same arguments without workspace / workspace_bytes, same
 * kernels, the same results bit for bit).
 *   - The call allocates nothing.  Its first call on a device looks up that
 *     device's array address (hipGetSymbolAddress) and keeps it: make that
 *     first call outside graph capture.
 *   - The array of the current device is used; `stream` must belong to it.
 *   - MOE_EWORKSPACE (nothing launched) if the batch needs more than
 *     MOE_STATIC_WS_BYTES, i.e. moe_layer_forward_workspace_bytes(layer, T, k)
 *     > MOE_STATIC_WS_BYTES (at H 6144, I 2048, E 256, k 8: batches of up to
 *     T = 138 tokens fit).
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (two streams, two threads) race and give unspecified
 *     results; calls ordered on one stream are safe.  The array keeps the
 *     last call's contents; nothing in it needs to start at zero (each call
 *     writes every byte it reads before reading it).
 */
#define MOE_STATIC_WS_BYTES (32u << 20)
int moe_layer_forward_static(const moe_qlayer* layer, const uint16_t* x_bf16, const float* logits,
                             int64_t T, int32_t k, const float* y_shared, int32_t* topk_ids,
                             float* topk_w, float* out, void* stream);

/*
 * moe_layer_forward_shared -- moe_shared_ffn followed by moe_layer_forward
 * with its output as y_shared, in one call: out = (the routed layer's gated
 * sum) + the shared expert's FFN of every token.
 * (Shared experts beside the routed ones: "GLM-5.3-EXL3-TR3-3.42bpw", What
 * is quantized.)
 *
 *   layer, x_bf16, logits, k, topk_ids, topk_w, out  as for moe_layer_forward.
 *   shared     a one-expert layer (E == 1, unrotated) with the routed layer's
 *              H, as for moe_shared_ffn.
 *   workspace  [device] >= moe_layer_forward_shared_workspace_bytes(layer,
 *              shared, T, k) bytes, 256-byte aligned; contents on return
 *              unspecified.
 *
 * When moe_layer_forward would take its fused path and the shared expert is
 * BF16, the layer runs in three launches: the routed and the shared gate/up
 * passes in one, the routed down + combine beside the shared SwiGLU in the
 * next, then the shared down pass, which adds each of its outputs to the
 * routed sum (the combine's last addition).  The results are the bits of
 * moe_shared_ffn + moe_layer_forward on the same inputs.  Otherwise it runs
 * those two calls.  Errors as for them (checked before any launch), and
 * MOE_EINVAL if the shared layer's H differs from the routed layer's.
 */
size_t moe_layer_forward_shared_workspace_bytes(const moe_qlayer* layer,
                                                const moe_qlayer* shared, int64_t T, int32_t k);
int moe_layer_forward_shared(const moe_qlayer* layer, const moe_qlayer* shared,
                             const uint16_t* x_bf16, const float* logits, int64_t T, int32_t k,
                             int32_t* topk_ids, float* topk_w, float* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------------------- host-side packers */

/*
 * moe_quantize_nvfp4 -- [host] encode fp32 weights w [n, kin] (row-major,
 * kin % 16 == 0) to canonical NVFP4 bytes:
 *   codes  [n, kin/2]  element 2i in the low nibble of byte i;
 *   scales [n, kin/16] E4M3 (OCP E4M3FN) byte per 16 contiguous inputs.
 * Per block: S = E4M3(amax/6), nearest, ties to even, saturating at 448;
 * S == 0 -> all codes 0; else each element -> nearest E2M1 magnitude of
 * |w|/S, ties to even mantissa, saturating at 6, sign bit only on nonzero
 * magnitudes.  ("GLM-5-NVFP4-MTP", Model Description.)
 * Returns MOE_EINVAL on a null pointer, bad size or a non-finite weight
 * (then the outputs are unspecified).
 */
int moe_quantize_nvfp4(const float* w, int32_t n, int32_t kin,
                       uint8_t* codes, uint8_t* scales);

/*
 * moe_quantize_nvfp4_residual -- [host] the two planes of MOE_FMT_NVFP4R:
 * base = moe_quantize_nvfp4(w); residual = moe_quantize_nvfp4(r) with
 * r = fp32((w - base value) * 2^shift) (exact in fp64, rounded once to
 * fp32), 0 <= shift <= 14.  Same byte layout and errors as
 * moe_quantize_nvfp4.
 * ("GLM-5.3 Vision NestQuant 1.75-4 bit", introduction and Method: a base
 * plus a residual plane coding what the base leaves.)
 */
int moe_quantize_nvfp4_residual(const float* w, int32_t n, int32_t kin, int32_t shift,
                                uint8_t* base_codes, uint8_t* base_scales,
                                uint8_t* res_codes, uint8_t* res_scales);

/*
 * Bytes of one expert record in the device tile layout.
 *   fmt = MOE_FMT_NVFP4 / MOE_FMT_VQ / MOE_FMT_BF16 / MOE_FMT_NVFP4R (twice
 *   the NVFP4 record: base plane, then residual plane) / MOE_FMT_VQ8_Mm
 *   (= moe_record_bytes_vq8(which, H, I, m)) (MOE_FMT_VQ8: use
 *   moe_record_bytes_vq8 with the layer's vq8_m); which = 0 for the gate/up record
 *   (both projections, rows interleaved by 16), 1 for the down record.
 * Returns 0 for an unsupported format or shape.
 */
size_t moe_record_bytes(int fmt, int which, int32_t H, int32_t I);

/* Bytes of one MOE_FMT_VQ8 record with m codes per group (0 on bad sizes). */
size_t moe_record_bytes_vq8(int which, int32_t H, int32_t I, int32_t m);

/*
 * moe_pack_nvfp4_expert -- [host] lay the canonical NVFP4 bytes of one
 * expert out as its two device records (gate/up and down).
 *   ("GLM-5-NVFP4-MTP", Model Description: 4-bit E2M1 codes with an E4M3
 *   scale per 16 elements; "GLM-5.3 Vision NestQuant 1.75-4 bit", Contents:
 *   one record per expert, addressed by expert id at a fixed stride.)
 *   gate/up codes [I, H/2], scales [I, H/16]; down codes [H, I/2],
 *   scales [H, I/16] ([host], canonical layout as moe_quantize_nvfp4 writes
 *   it); w13_rec / w2_rec [host] out, moe_record_bytes() each (the caller
 *   uploads them).  MOE_EINVAL on a null pointer or a scale byte that is the
 *   E4M3 NaN (0x7F or 0xFF: E4M3FN has no infinities); MOE_EUNSUPPORTED if
 *   H or I is not a positive multiple of 16.  Nothing else is checked: every
 *   other code and scale byte is a finite value.
 */
int moe_pack_nvfp4_expert(const uint8_t* gate_codes, const uint8_t* gate_scales,
                          const uint8_t* up_codes, const uint8_t* up_scales,
                          const uint8_t* down_codes, const uint8_t* down_scales,
                          int32_t H, int32_t I, uint8_t* w13_rec, uint8_t* w2_rec);

/*
 * moe_pack_nvfp4r_expert -- [host] lay one MOE_FMT_NVFP4R expert out as its
 * two records: the base plane's NVFP4 record (from base_parts) followed by
 * the residual plane's (from res_parts).  base_parts / res_parts: the six
 * arrays moe_pack_nvfp4_expert takes, in its order (gate codes, gate scales,
 * up codes, up scales, down codes, down scales).  w13_rec / w2_rec [host]
 * out, moe_record_bytes(MOE_FMT_NVFP4R, ...) each.  Errors as
 * moe_pack_nvfp4_expert (an E4M3 NaN scale byte in either plane: MOE_EINVAL).
 */
int moe_pack_nvfp4r_expert(const uint8_t* const base_parts[6], const uint8_t* const res_parts[6],
                           int32_t H, int32_t I, uint8_t* w13_rec, uint8_t* w2_rec);

/*
 * moe_pack_vq_expert -- [host] lay one VQ expert out as its two records.
 *   codes uint16 [n, kin/8] (group g covers inputs 8g..8g+7), scales fp16
 *   bits [n], for gate/up (n = I, kin = H) and down (n = H, kin = I).
 *   ("GLM-5.2 mixed-bit VQ (AQLM) ~1.90 bpw", What it is.)
 *   MOE_EINVAL on a null pointer or a scale that is not finite (fp16 inf or
 *   NaN); MOE_EUNSUPPORTED if H or I is not a positive multiple of 16.
 */
int moe_pack_vq_expert(const uint16_t* gate_codes, const uint16_t* gate_scales,
                       const uint16_t* up_codes, const uint16_t* up_scales,
                       const uint16_t* down_codes, const uint16_t* down_scales,
                       int32_t H, int32_t I, uint8_t* w13_rec, uint8_t* w2_rec);

/*
 * moe_pack_vq8_expert -- [host] lay one MOE_FMT_VQ8 expert out as its two
 * records.  codes uint8 [n, kin/8, m] (code j of group g indexes codebook
 * j; group g covers inputs 8g..8g+7), scales fp16 bits [n], for gate/up
 * (n = I, kin = H) and down (n = H, kin = I); m = 1, 2 or 3.
 *   ("GLM-5.2 mixed-bit VQ (AQLM) ~1.90 bpw", What it is: modules of 1, 2
 *   and 3 bits per weight, each indexing codebooks shared by the experts.)
 *   MOE_EINVAL on a null pointer or a scale that is not finite;
 *   MOE_EUNSUPPORTED for H or I not a positive multiple of 16 or m outside
 *   1..3.
 */
int moe_pack_vq8_expert(const uint8_t* gate_codes, const uint16_t* gate_scales,
                        const uint8_t* up_codes, const uint16_t* up_scales,
                        const uint8_t* down_codes, const uint16_t* down_scales,
                        int32_t H, int32_t I, int32_t m, uint8_t* w13_rec, uint8_t* w2_rec);

/*
 * moe_pack_bf16_expert -- [host] lay one MOE_FMT_BF16 expert out as its two
 * records.  gate, up [I, H] and down [H, I]: bf16 bits, row-major.
 * MOE_EINVAL if a weight is not finite or |w| > 65504 (the kernels use the
 * weights as fp16).
 */
int moe_pack_bf16_expert(const uint16_t* gate, const uint16_t* up, const uint16_t* down,
                         int32_t H, int32_t I, uint8_t* w13_rec, uint8_t* w2_rec);

/*
 * moe_record_table -- [host] fill rec [E] = (fmt << 24) | index(e) from the
 * tier map, and n_by_fmt [MOE_FMT_MAX + 1] (may be NULL) with the number of
 * experts of each tag (entry 0 is 0).  MOE_EUNSUPPORTED on an unknown tag.
 */
int moe_record_table(const uint8_t* fmt_host, int32_t E, int32_t* rec, int32_t* n_by_fmt);

/* Bytes of one expert's rotation signs: (2H + 3I) / 8 (0 on bad sizes). */
size_t moe_rot_sign_bytes(int32_t H, int32_t I);

/*
 * moe_pack_rot_signs -- [host] one expert's rotation signs (int8 +1 / -1) as
 * the bits rot_signs holds: s_in13 [H] (gate/up input), s_out_gate [I],
 * s_out_up [I], s_in2 [I] (down input), s_out2 [H] (down output), in that
 * order, bit i of byte b = channel 8b + i of the section is -1.
 * out [host] moe_rot_sign_bytes(H, I).  MOE_EINVAL on a value other than +-1.
 */
int moe_pack_rot_signs(const int8_t* s_in13, const int8_t* s_out_gate, const int8_t* s_out_up,
                       const int8_t* s_in2, const int8_t* s_out2, int32_t H, int32_t I,
                       uint8_t* out);

/*
 * moe_rotate_matrix -- [host] W_rot = R_out W R_in^T for fp32 W [n_out, n_in]
 * (n_out, n_in multiples of 128; s_out [n_out], s_in [n_in] int8 +-1),
 * computed in fp64 and rounded once to fp32 into out [n_out, n_in] (may
 * alias w).  The offline step of a rotated format: rotate, then encode.
 */
int moe_rotate_matrix(const float* w, int32_t n_out, int32_t n_in, const int8_t* s_out,
                      const int8_t* s_in, float* out);

/*
 * moe_rotate_matrix_blocks -- [host] the same with a Hadamard block per side:
 * R_out = blockdiag(H_bo/sqrt(bo)) diag(s_out), R_in likewise with bi; bo and
 * bi each MOE_ROT_BLOCK or MOE_ROT_BLOCK_WIDE, n_out a multiple of bo and n_in
 * of bi ("GLM-5.3 Vision NestQuant 1.75-4 bit", Method: the down matrix of a
 * wide-variant layer takes bo = 128, bi = 512).  MOE_EINVAL otherwise.
 */
int moe_rotate_matrix_blocks(const float* w, int32_t n_out, int32_t n_in, const int8_t* s_out,
                             const int8_t* s_in, int32_t block_out, int32_t block_in,
                             float* out);

/*
 * moe_record_table_resident -- [host] rec [E] = (fmt << 24) | e for a layer
 * in MOE_REC_RESIDENT mode (every used pool holds every expert at slot e).
 * MOE_EUNSUPPORTED on an unknown tag.
 */
int moe_record_table_resident(const uint8_t* fmt_host, int32_t E, int32_t* rec);

/* ------------------------------------------------------------ test hook */

/*
 * moe_dequant_q -- decode projection `proj` (MOE_PROJ_*) of expert `expert`
 * to fp32 out [n, kin] ([device]; gate/up: [I, H], down: [H, I]) with the
 * same device decode routines the FFN kernels use.
 *   (The weight values the formats define: an E2M1 code times its E4M3 block
 *   scale, "GLM-5-NVFP4-MTP", Model Description; a codebook row times the
 *   row's scale, "GLM-5.2 mixed-bit VQ (AQLM) ~1.90 bpw", What it is.)
 *   A test hook: it lets the stored bytes be compared with the oracle's
 *   decode without running an FFN.  Errors as moe_expert_ffn_q's layer checks,
 *   MOE_EINVAL for an expert outside [0, E), a bad proj or a NULL out.  NVFP4 and VQ values are
 * exact; a MOE_FMT_VQ8 value with m >= 2 is fp32(fp32(C_0 + .. + C_{m-1}) * S) (fp32
 * sums; the FFN kernels multiply each codebook row exactly instead); a
 * MOE_FMT_BF16 value is the stored weight as the kernels' fp16 operand; a
 * MOE_FMT_NVFP4R value is fp32(base + residual * 2^-nvfp4r_shift) (the FFN
 * kernels multiply each plane exactly instead).  For a rotated layer this is the stored (rotated)
 * matrix.
 */
int moe_dequant_q(const moe_qlayer* layer, int32_t expert, int32_t proj,
                  float* out, void* stream);

/* ------------------------------------------------------ measurement aid */

/* Workgroups moe_probe_read launches (the size of its sink). */
#define MOE_PROBE_BLOCKS 2048

/*
 * moe_probe_read -- read `bytes` of [device] buf once with 16-byte
 * non-temporal loads (the weight-streaming kernels' kind of load) and write
 * the XOR of what each workgroup read to sink [device] uint32
 * [MOE_PROBE_BLOCKS]: timing it gives the HBM read rate those kernels can
 * reach.  bytes must be a multiple of 16 and buf 16-byte aligned.
 */
int moe_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOEQ_H */
