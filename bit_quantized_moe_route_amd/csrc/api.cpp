// C ABI: argument checks, workspace layout and dispatch to the HIP launchers.
#include <cmath>
#include <cstdint>
#include <string>

#include "internal.h"

namespace moeq {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int status, const std::string& msg) {
    g_last_error = msg;
    return status;
}

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int check_route_sizes(const char* fn, int64_t T, int32_t E, int32_t k) {
    if (T < 0) return fail(MOE_EINVAL, std::string(fn) + ": T < 0");
    if (E < 1 || E > MOE_MAX_E)
        return fail(MOE_EINVAL, std::string(fn) + ": E must be in [1, " + std::to_string(MOE_MAX_E) + "]");
    if (k < 1 || k > E || k > MOE_MAX_K)
        return fail(MOE_EINVAL, std::string(fn) + ": k must be in [1, min(E, " +
                                    std::to_string(MOE_MAX_K) + ")]");
    if (T * (int64_t)k >= (int64_t)1 << 31) return fail(MOE_EINVAL, std::string(fn) + ": T*k too large");
    return MOE_OK;
}

struct LayerInfo {
    LayerView view;
    int32_t count[kNumFmt];
};

// Validate a layer descriptor; fill the device view and per-format counts.
int check_layer(const char* fn, const moe_qlayer* L, LayerInfo& out) {
    const std::string f(fn);
    if (!L) return fail(MOE_EINVAL, f + ": layer is NULL");
    if (L->E < 1 || L->E > MOE_MAX_E) return fail(MOE_EINVAL, f + ": bad E");
    if (L->H <= 0 || L->I <= 0) return fail(MOE_EINVAL, f + ": bad H or I");
    if (!L->fmt_host || !L->rec_dev) return fail(MOE_EINVAL, f + ": fmt_host / rec_dev is NULL");
    if (L->record_mode != MOE_REC_COMPACT && L->record_mode != MOE_REC_RESIDENT)
        return fail(MOE_EINVAL, f + ": unknown record_mode");
    for (int t = 0; t < kNumFmt; ++t) out.count[t] = 0;
    for (int e = 0; e < L->E; ++e) {
        const int t = L->fmt_host[e];
        if (t < MOE_FMT_NVFP4 || t > MOE_FMT_MAX)
            return fail(MOE_EUNSUPPORTED, f + ": expert " + std::to_string(e) +
                                              " has format tag " + std::to_string(t) +
                                              ", which this library does not decode");
        out.count[t]++;
    }
    if (L->H % 16 || L->I % 16)
        return fail(MOE_EUNSUPPORTED, f + ": H and I must be multiples of 16");
    LayerView& v = out.view;
    v.E = L->E;
    v.H = L->H;
    v.I = L->I;
    v.rec = L->rec_dev;
    v.pool13[0] = v.pool2[0] = nullptr;
    v.stride13[0] = v.stride2[0] = 0;
    v.pool13[MOE_FMT_NVFP4] = static_cast<const uint8_t*>(L->nvfp4_w13);
    v.pool2[MOE_FMT_NVFP4] = static_cast<const uint8_t*>(L->nvfp4_w2);
    v.stride13[MOE_FMT_NVFP4] = L->nvfp4_w13_stride;
    v.stride2[MOE_FMT_NVFP4] = L->nvfp4_w2_stride;
    v.pool13[MOE_FMT_VQ] = static_cast<const uint8_t*>(L->vq_w13);
    v.pool2[MOE_FMT_VQ] = static_cast<const uint8_t*>(L->vq_w2);
    v.stride13[MOE_FMT_VQ] = L->vq_w13_stride;
    v.stride2[MOE_FMT_VQ] = L->vq_w2_stride;
    v.pool13[MOE_FMT_VQ8] = static_cast<const uint8_t*>(L->vq8_w13);
    v.pool2[MOE_FMT_VQ8] = static_cast<const uint8_t*>(L->vq8_w2);
    v.stride13[MOE_FMT_VQ8] = L->vq8_w13_stride;
    v.stride2[MOE_FMT_VQ8] = L->vq8_w2_stride;
    v.pool13[MOE_FMT_BF16] = static_cast<const uint8_t*>(L->bf16_w13);
    v.pool2[MOE_FMT_BF16] = static_cast<const uint8_t*>(L->bf16_w2);
    v.stride13[MOE_FMT_BF16] = L->bf16_w13_stride;
    v.stride2[MOE_FMT_BF16] = L->bf16_w2_stride;
    for (int m = 1; m <= MOE_VQ8_MAX_M; ++m) {
        const int f = MOE_FMT_VQ8_M1 + m - 1;
        v.pool13[f] = static_cast<const uint8_t*>(L->vq8r_w13[m - 1]);
        v.pool2[f] = static_cast<const uint8_t*>(L->vq8r_w2[m - 1]);
        v.stride13[f] = L->vq8r_w13_stride[m - 1];
        v.stride2[f] = L->vq8r_w2_stride[m - 1];
    }
    v.pool13[MOE_FMT_NVFP4R] = static_cast<const uint8_t*>(L->nvfp4r_w13);
    v.pool2[MOE_FMT_NVFP4R] = static_cast<const uint8_t*>(L->nvfp4r_w2);
    v.stride13[MOE_FMT_NVFP4R] = L->nvfp4r_w13_stride;
    v.stride2[MOE_FMT_NVFP4R] = L->nvfp4r_w2_stride;
    v.res13 = nv_record_bytes(0, L->H, L->I);
    v.res2 = nv_record_bytes(1, L->H, L->I);
    v.res_scale = 1.0f;
    for (int p = 0; p < 3; ++p) v.cb[p] = static_cast<const uint8_t*>(L->vq_codebook[p]);
    v.cb_stride = L->vq_codebook_stride;
    for (int p = 0; p < 3; ++p) v.cb8[p] = static_cast<const uint8_t*>(L->vq8_codebook[p]);
    v.vq8_m = L->vq8_m;
    v.rot = L->rot_signs;
    v.rot_stride = (int64_t)(2 * (int64_t)L->H + 3 * (int64_t)L->I) / 8;
    if (v.rot && (L->H % MOE_ROT_BLOCK || L->I % MOE_ROT_BLOCK))
        return fail(MOE_EUNSUPPORTED, f + ": a rotated layer needs H and I multiples of 128");
    v.rot_in2 = MOE_ROT_BLOCK;
    if (v.rot && L->rot_in2_block != 0 && L->rot_in2_block != MOE_ROT_BLOCK) {
        if (L->rot_in2_block != MOE_ROT_BLOCK_WIDE)
            return fail(MOE_EUNSUPPORTED, f + ": rot_in2_block must be 0, 128 or 512");
        if (L->I % MOE_ROT_BLOCK_WIDE)
            return fail(MOE_EUNSUPPORTED,
                        f + ": the 512-block down-input rotation needs I a multiple of 512");
        v.rot_in2 = MOE_ROT_BLOCK_WIDE;
    }
    if (out.count[MOE_FMT_NVFP4R]) {
        if (L->nvfp4r_shift < 0 || L->nvfp4r_shift > 14)
            return fail(MOE_EUNSUPPORTED, f + ": nvfp4r_shift must be in [0, 14]");
        v.res_scale = std::ldexp(1.0f, -L->nvfp4r_shift);
    }
    if (out.count[MOE_FMT_VQ8] && (L->vq8_m < 1 || L->vq8_m > MOE_VQ8_MAX_M))
        return fail(MOE_EUNSUPPORTED, f + ": vq8_m must be 1, 2 or 3");
    for (int fmt = MOE_FMT_NVFP4; fmt < kNumFmt; ++fmt) {
        if (!out.count[fmt]) continue;
        const char* name = fmt == MOE_FMT_NVFP4     ? "NVFP4"
                           : fmt == MOE_FMT_VQ      ? "VQ"
                           : fmt == MOE_FMT_VQ8     ? "VQ8"
                           : fmt == MOE_FMT_BF16    ? "BF16"
                           : fmt == MOE_FMT_NVFP4R  ? "NVFP4R"
                           : fmt == MOE_FMT_VQ8_M1  ? "VQ8 (1 bit)"
                           : fmt == MOE_FMT_VQ8_M2  ? "VQ8 (2 bits)"
                                                    : "VQ8 (3 bits)";
        if (!v.pool13[fmt] || !v.pool2[fmt])
            return fail(MOE_EINVAL, f + ": " + name + " experts present but their pool is NULL");
        const int rate = is_vq8(fmt) ? vq8_rate(fmt, L->vq8_m) : 0;
        const int64_t b13 = is_vq8(fmt) ? (int64_t)moe_record_bytes_vq8(0, L->H, L->I, rate)
                                        : (int64_t)moe_record_bytes(fmt, 0, L->H, L->I);
        const int64_t b2 = is_vq8(fmt) ? (int64_t)moe_record_bytes_vq8(1, L->H, L->I, rate)
                                       : (int64_t)moe_record_bytes(fmt, 1, L->H, L->I);
        if (v.stride13[fmt] < b13 || v.stride2[fmt] < b2 || v.stride13[fmt] % 256 ||
            v.stride2[fmt] % 256)
            return fail(MOE_EINVAL, f + ": " + name +
                                        " record stride smaller than moe_record_bytes() or not a "
                                        "multiple of 256");
    }
    if (out.count[MOE_FMT_VQ]) {
        for (int p = 0; p < 3; ++p)
            if (!v.cb[p]) return fail(MOE_EINVAL, f + ": VQ experts present but a codebook is NULL");
        if (v.cb_stride < 0 || (v.cb_stride && v.cb_stride < (int64_t)MOE_VQ_NCODE * 16))
            return fail(MOE_EINVAL, f + ": bad vq_codebook_stride");
    }
    int n_vq8 = 0;
    for (int fmt = MOE_FMT_NVFP4; fmt < kNumFmt; ++fmt) n_vq8 += is_vq8(fmt) ? out.count[fmt] : 0;
    if (n_vq8)
        for (int p = 0; p < 3; ++p)
            if (!v.cb8[p]) return fail(MOE_EINVAL, f + ": VQ8 experts present but a codebook is NULL");
    return MOE_OK;
}

// moe_expert_gateup_q: the fp16 copy of x, or for a rotated layer the rotated
// rows x' [T*k, H] and the raw gate/up products [T*k, 2I] fp32.
size_t gateup_ws(const moe_qlayer* L, int64_t T, int32_t k) {
    if (L->rot_signs)
        return align_up((size_t)T * k * L->H * 2) + align_up((size_t)T * k * 2 * L->I * 4);
    return align_up((size_t)T * L->H * 2);
}

// moe_expert_ffn_q: gate/up's workspace, then h [T*k, I] fp16.
size_t ffn_ws(const moe_qlayer* L, int64_t T, int32_t k) {
    return gateup_ws(L, T, k) + align_up((size_t)T * k * L->I * 2);
}

// moe_shared_ffn: x16 | h16 | the gate/up partial sums of the decode path
// (sized for the split that path takes; none where the grouped GEMM runs).
// The format is the one expert's tag (an unreadable or unknown tag sizes for
// the largest split; the call itself then fails its layer checks).
size_t shared_ws(const moe_qlayer* L, int64_t T) {
    const int fmt = L->fmt_host ? L->fmt_host[0] : 0;
    return align_up((size_t)T * L->H * 2) + align_up((size_t)T * L->I * 2) +
           align_up(shared_part_bytes(fmt, T, L->H, L->I));
}

// moe_layer_forward: the small-batch fused path needs only h [T*k, I] fp16
// (a rotated layer also the raw products and y', small_rot_ws_bytes); the
// step-by-step path counts | offsets | perm_src | inv_perm | the permute
// workspace | the expert-FFN workspace | y_perm [T*k, H] fp32, which is more.
bool layer_small_ok(const LayerInfo& li, int64_t T, int32_t k) {
    int nfmt = 0;
    for (int f = MOE_FMT_NVFP4; f < kNumFmt; ++f) nfmt += li.count[f] > 0;
    return nfmt == 1 && li.view.E <= 256 && k <= 8 && T * k <= kSmallFusedAssign &&
           (!li.view.rot || li.view.H <= kSmallRotMaxH);
}

struct LayerWs {
    size_t counts, offsets, perm_src, inv_perm, pws, ffn, y_perm, total;
};

LayerWs layer_ws(const moe_qlayer* L, int64_t T, int32_t k) {
    LayerWs w;
    const size_t tk = (size_t)T * k;
    w.counts = 0;
    w.offsets = w.counts + align_up((size_t)L->E * 4);
    w.perm_src = w.offsets + align_up((size_t)(L->E + 1) * 4);
    w.inv_perm = w.perm_src + align_up(tk * 4);
    w.pws = w.inv_perm + align_up(tk * 4);
    w.ffn = w.pws + align_up(permute_ws_bytes(T, k, L->E));
    w.y_perm = w.ffn + ffn_ws(L, T, k);
    w.total = w.y_perm + align_up(tk * L->H * 4);
    return w;
}

// The two formats of a layer holding exactly NVFP4 and one VQ form, for the
// one-launch decode path (false for other layers).
bool decode_pair(const LayerInfo& li, int64_t T, int32_t k, int& f1, int& f2) {
    int nf = 0;
    f1 = f2 = 0;
    for (int f = MOE_FMT_NVFP4; f < kNumFmt; ++f) {
        if (!li.count[f]) continue;
        ++nf;
        if (f == MOE_FMT_NVFP4) f1 = f;
        else f2 = f;
    }
    return nf == 2 && f1 && f2 &&
           ffn_decode_pair_ok(li.view, f1, li.count[f1], f2, li.count[f2], T, k);
}

// Gate/up + SwiGLU of every format present.  perm_src == offsets == NULL is
// the identity map of a one-expert layer (k = 1; part: the decode path's
// partial sums).  x16 [T, H] is workspace for the fp16 copy of x that the
// grouped-GEMM kernels stage through LDS.
int run_gateup(const LayerInfo& li, const uint16_t* x_bf16, const int32_t* perm_src,
               const int32_t* offsets, int64_t T, int32_t k, uint16_t* h_f16, uint16_t* x16,
               float* part, void* stream) {
    const bool prefill = T >= kPrefillMinTokens;
    if (li.view.rot) {
        // rotated layer: x' rows per assignment (in the place of x16), the raw
        // products in gu (after them), then h' from both
        float* gu = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(x16) +
                                             align_up((size_t)T * k * li.view.H * 2));
        int st = launch_rot_in(li.view, x_bf16, perm_src, offsets, T, k, x16, stream);
        if (st) return st;
        for (int fmt = MOE_FMT_NVFP4; fmt < kNumFmt; ++fmt) {
            if (!li.count[fmt]) continue;
            st = prefill && prefill_fmt(fmt, false)
                     ? launch_ffn_prefill(li.view, fmt, li.count[fmt], x16, perm_src, offsets, T,
                                          k, h_f16, nullptr, 0, stream, gu)
                     : launch_ffn_decode(li.view, fmt, li.count[fmt], x16, perm_src, offsets, T,
                                         k, h_f16, nullptr, 0, stream, gu);
            if (st) return st;
        }
        return launch_rot_mid(li.view, gu, offsets, T * k, h_f16, stream);
    }
    bool need_x16 = false;
    for (int fmt = MOE_FMT_NVFP4; fmt < kNumFmt; ++fmt)
        need_x16 |= prefill && li.count[fmt] && prefill_fmt(fmt, offsets == nullptr);
    if (need_x16) {
        const int st = launch_x_to_f16(x_bf16, T * li.view.H, x16, stream);
        if (st) return st;
    }
    int f1, f2;
    if (!prefill && offsets && decode_pair(li, T, k, f1, f2))
        return launch_ffn_decode_pair(li.view, f1, li.count[f1], f2, li.count[f2], x_bf16, perm_src,
                                      offsets, T, k, h_f16, nullptr, 0, stream);
    for (int fmt = MOE_FMT_NVFP4; fmt < kNumFmt; ++fmt) {
        if (!li.count[fmt]) continue;
        const int st =
            prefill && prefill_fmt(fmt, offsets == nullptr)
                ? launch_ffn_prefill(li.view, fmt, li.count[fmt], x16, perm_src, offsets, T, k,
                                     h_f16, nullptr, 0, stream)
            : offsets ? launch_ffn_decode(li.view, fmt, li.count[fmt], x_bf16, perm_src, offsets,
                                          T, k, h_f16, nullptr, 0, stream)
                      : launch_shared_decode(li.view, fmt, x_bf16, T, h_f16, part, nullptr, 0,
                                             stream);
        if (st) return st;
    }
    return MOE_OK;
}

// Down projection of every format present (offsets == NULL: identity map).
// rot_back = false leaves a rotated layer's outputs in the rotated domain
// (launch_combine_rot rotates them back).
int run_down(const LayerInfo& li, const uint16_t* h_f16, const int32_t* offsets, int64_t T,
             int32_t k, float* y_perm, void* stream, bool rot_back = true) {
    const bool prefill = T >= kPrefillMinTokens;
    int f1, f2;
    if (!prefill && offsets && !li.view.rot && decode_pair(li, T, k, f1, f2))
        return launch_ffn_decode_pair(li.view, f1, li.count[f1], f2, li.count[f2], nullptr,
                                      nullptr, offsets, T, k, const_cast<uint16_t*>(h_f16),
                                      y_perm, 1, stream);
    for (int fmt = MOE_FMT_NVFP4; fmt < kNumFmt; ++fmt) {
        if (!li.count[fmt]) continue;
        uint16_t* h = const_cast<uint16_t*>(h_f16);
        const int st =
            prefill && prefill_fmt(fmt, offsets == nullptr)
                ? launch_ffn_prefill(li.view, fmt, li.count[fmt], nullptr, nullptr, offsets, T, k,
                                     h, y_perm, 1, stream)
            : offsets ? launch_ffn_decode(li.view, fmt, li.count[fmt], nullptr, nullptr, offsets,
                                          T, k, h, y_perm, 1, stream)
                      : launch_shared_decode(li.view, fmt, nullptr, T, h, nullptr, y_perm, 1,
                                             stream);
        if (st) return st;
    }
    if (li.view.rot && rot_back) return launch_rot_out(li.view, y_perm, offsets, T * k, stream);
    return MOE_OK;
}

}  // namespace

}  // namespace moeq

using namespace moeq;

extern "C" {

const char* moe_strerror(int status) {
    switch (status) {
        case MOE_OK: return "success";
        case MOE_EINVAL: return "invalid argument";
        case MOE_EUNSUPPORTED: return "unsupported format or shape (failed closed)";
        case MOE_EWORKSPACE: return "workspace too small";
        case MOE_EHIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_ids,
                   float* topk_w, void* stream) {
    g_last_error.clear();
    int st = check_route_sizes("moe_route_topk", T, E, k);
    if (st) return st;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_w) return fail(MOE_EINVAL, "moe_route_topk: null pointer");
    return launch_route_topk(logits, T, E, k, topk_ids, topk_w, stream);
}

size_t moe_permute_workspace_bytes(int64_t T, int32_t k, int32_t E) {
    if (T < 0 || k < 1 || E < 1) return 0;
    return permute_ws_bytes(T, k, E);
}

int moe_permute(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t* counts,
                int32_t* offsets, int32_t* perm_src, int32_t* inv_perm, void* ws,
                size_t ws_bytes, void* stream) {
    g_last_error.clear();
    int st = check_route_sizes("moe_permute", T, E, k);
    if (st) return st;
    if (!counts || !offsets) return fail(MOE_EINVAL, "moe_permute: null pointer");
    const size_t need = permute_ws_bytes(T, k, E);
    if (need && (!ws || ws_bytes < need))
        return fail(MOE_EWORKSPACE, "moe_permute: workspace needs " + std::to_string(need) + " bytes");
    if (T > 0 && (!topk_ids || !perm_src || !inv_perm))
        return fail(MOE_EINVAL, "moe_permute: null pointer");
    // T == 0 still writes counts = 0 and offsets = 0 (one tiny launch)
    return launch_permute(topk_ids, T, k, E, counts, offsets, perm_src, inv_perm, ws, stream);
}

int moe_route_permute(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_ids,
                      float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                      int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    int st = check_route_sizes("moe_route_permute", T, E, k);
    if (st) return st;
    if (!counts || !offsets) return fail(MOE_EINVAL, "moe_route_permute: null pointer");
    if (T > 0 && (!logits || !topk_ids || !topk_w || !perm_src || !inv_perm))
        return fail(MOE_EINVAL, "moe_route_permute: null pointer");
    const size_t need = permute_ws_bytes(T, k, E);
    if (need && (!ws || ws_bytes < need))
        return fail(MOE_EWORKSPACE,
                    "moe_route_permute: workspace needs " + std::to_string(need) + " bytes");
    if (route_permute_fused_ok(T, k))
        return launch_route_permute(logits, T, E, k, topk_ids, topk_w, counts, offsets, perm_src,
                                    inv_perm, stream);
    st = launch_route_topk(logits, T, E, k, topk_ids, topk_w, stream);
    if (st) return st;
    return launch_permute(topk_ids, T, k, E, counts, offsets, perm_src, inv_perm, ws, stream);
}

size_t moe_ffn_workspace_bytes(const moe_qlayer* layer, int64_t T, int32_t k) {
    if (!layer || T < 0 || k < 1 || layer->H <= 0 || layer->I <= 0) return 0;
    return ffn_ws(layer, T, k);
}

size_t moe_gateup_workspace_bytes(const moe_qlayer* layer, int64_t T, int32_t k) {
    if (!layer || T < 0 || k < 1 || layer->H <= 0 || layer->I <= 0) return 0;
    return gateup_ws(layer, T, k);
}

int moe_expert_gateup_q(const moe_qlayer* layer, const uint16_t* x_bf16, const int32_t* perm_src,
                        const int32_t* offsets, int64_t T, int32_t k, uint16_t* h_f16, void* ws,
                        size_t ws_bytes, void* stream) {
    g_last_error.clear();
    LayerInfo li;
    int st = check_layer("moe_expert_gateup_q", layer, li);
    if (st) return st;
    st = check_route_sizes("moe_expert_gateup_q", T, layer->E, k);
    if (st) return st;
    if (T == 0) return MOE_OK;
    if (!x_bf16 || !perm_src || !offsets || !h_f16)
        return fail(MOE_EINVAL, "moe_expert_gateup_q: null pointer");
    const size_t need = gateup_ws(layer, T, k);
    if (!ws || ws_bytes < need)
        return fail(MOE_EWORKSPACE,
                    "moe_expert_gateup_q: workspace needs " + std::to_string(need) + " bytes");
    if (reinterpret_cast<uintptr_t>(ws) % kAlign)
        return fail(MOE_EINVAL, "moe_expert_gateup_q: workspace must be 256-byte aligned");
    // the grouped-GEMM kernels stage fp16 tokens through LDS: convert x once;
    // the decode kernels convert each fragment they read
    return run_gateup(li, x_bf16, perm_src, offsets, T, k, h_f16, static_cast<uint16_t*>(ws),
                      nullptr, stream);
}

int moe_expert_down_q(const moe_qlayer* layer, const uint16_t* h_f16, const int32_t* offsets,
                      int64_t T, int32_t k, float* y_perm, void* stream) {
    g_last_error.clear();
    LayerInfo li;
    int st = check_layer("moe_expert_down_q", layer, li);
    if (st) return st;
    st = check_route_sizes("moe_expert_down_q", T, layer->E, k);
    if (st) return st;
    if (T == 0) return MOE_OK;
    if (!h_f16 || !offsets || !y_perm) return fail(MOE_EINVAL, "moe_expert_down_q: null pointer");
    return run_down(li, h_f16, offsets, T, k, y_perm, stream);
}

int moe_expert_ffn_q(const moe_qlayer* layer, const uint16_t* x_bf16, const int32_t* perm_src,
                     const int32_t* offsets, int64_t T, int32_t k, float* y_perm, void* ws,
                     size_t ws_bytes, void* stream) {
    g_last_error.clear();
    LayerInfo li;
    int st = check_layer("moe_expert_ffn_q", layer, li);
    if (st) return st;
    st = check_route_sizes("moe_expert_ffn_q", T, layer->E, k);
    if (st) return st;
    if (T == 0) return MOE_OK;
    if (!x_bf16 || !perm_src || !offsets || !y_perm)
        return fail(MOE_EINVAL, "moe_expert_ffn_q: null pointer");
    const size_t need = ffn_ws(layer, T, k);
    if (!ws || ws_bytes < need)
        return fail(MOE_EWORKSPACE,
                    "moe_expert_ffn_q: workspace needs " + std::to_string(need) + " bytes");
    if (reinterpret_cast<uintptr_t>(ws) % kAlign)
        return fail(MOE_EINVAL, "moe_expert_ffn_q: workspace must be 256-byte aligned");
    uint8_t* w = static_cast<uint8_t*>(ws);
    const size_t xbytes = gateup_ws(layer, T, k);
    uint16_t* h16 = reinterpret_cast<uint16_t*>(w + xbytes);
    st = moe_expert_gateup_q(layer, x_bf16, perm_src, offsets, T, k, h16, ws, xbytes, stream);
    if (st) return st;
    return moe_expert_down_q(layer, h16, offsets, T, k, y_perm, stream);
}

size_t moe_shared_ffn_workspace_bytes(const moe_qlayer* shared, int64_t T) {
    if (!shared || T < 0 || shared->H <= 0 || shared->I <= 0) return 0;
    return shared_ws(shared, T);
}

int moe_shared_ffn(const moe_qlayer* shared, const uint16_t* x_bf16, int64_t T,
                   float* y_shared, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    LayerInfo li;
    int st = check_layer("moe_shared_ffn", shared, li);
    if (st) return st;
    if (shared->E != 1) return fail(MOE_EINVAL, "moe_shared_ffn: the shared layer must have E == 1");
    if (shared->rot_signs)
        return fail(MOE_EUNSUPPORTED, "moe_shared_ffn: a rotated shared layer is not supported");
    st = check_route_sizes("moe_shared_ffn", T, 1, 1);
    if (st) return st;
    if (T == 0) return MOE_OK;
    if (!x_bf16 || !y_shared) return fail(MOE_EINVAL, "moe_shared_ffn: null pointer");
    const size_t need = shared_ws(shared, T);
    if (!ws || ws_bytes < need)
        return fail(MOE_EWORKSPACE,
                    "moe_shared_ffn: workspace needs " + std::to_string(need) + " bytes");
    if (reinterpret_cast<uintptr_t>(ws) % kAlign)
        return fail(MOE_EINVAL, "moe_shared_ffn: workspace must be 256-byte aligned");
    uint8_t* w = static_cast<uint8_t*>(ws);
    uint16_t* x16 = reinterpret_cast<uint16_t*>(w);
    uint16_t* h16 = reinterpret_cast<uint16_t*>(w + align_up((size_t)T * shared->H * 2));
    float* part = reinterpret_cast<float*>(w + align_up((size_t)T * shared->H * 2) +
                                           align_up((size_t)T * shared->I * 2));
    st = run_gateup(li, x_bf16, nullptr, nullptr, T, 1, h16, x16, part, stream);
    if (st) return st;
    return run_down(li, h16, nullptr, T, 1, y_shared, stream);
}

int moe_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w, int64_t T,
                int32_t k, int32_t H, float* out, void* stream) {
    g_last_error.clear();
    if (T < 0 || k < 1 || k > MOE_MAX_K || H <= 0 || H % 4)
        return fail(MOE_EINVAL, "moe_combine: need T >= 0, 1 <= k <= 16, H > 0, H % 4 == 0");
    if (T == 0) return MOE_OK;
    if (!y_perm || !inv_perm || !topk_w || !out) return fail(MOE_EINVAL, "moe_combine: null pointer");
    return launch_combine(y_perm, inv_perm, topk_w, nullptr, T, k, H, out, stream);
}

int moe_combine_shared(const float* y_perm, const int32_t* inv_perm, const float* topk_w,
                       const float* y_shared, int64_t T, int32_t k, int32_t H, float* out,
                       void* stream) {
    g_last_error.clear();
    if (T < 0 || k < 1 || k > MOE_MAX_K || H <= 0 || H % 4)
        return fail(MOE_EINVAL,
                    "moe_combine_shared: need T >= 0, 1 <= k <= 16, H > 0, H % 4 == 0");
    if (T == 0) return MOE_OK;
    if (!y_perm || !inv_perm || !topk_w || !y_shared || !out)
        return fail(MOE_EINVAL, "moe_combine_shared: null pointer");
    return launch_combine(y_perm, inv_perm, topk_w, y_shared, T, k, H, out, stream);
}

size_t moe_layer_forward_workspace_bytes(const moe_qlayer* layer, int64_t T, int32_t k) {
    if (!layer || T < 0 || k < 1 || layer->E < 1 || layer->H <= 0 || layer->I <= 0) return 0;
    return layer_ws(layer, T, k).total;
}

int moe_layer_forward(const moe_qlayer* layer, const uint16_t* x_bf16, const float* logits,
                      int64_t T, int32_t k, const float* y_shared, int32_t* topk_ids,
                      float* topk_w, float* out, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    LayerInfo li;
    int st = check_layer("moe_layer_forward", layer, li);
    if (st) return st;
    st = check_route_sizes("moe_layer_forward", T, layer->E, k);
    if (st) return st;
    if (layer->H % 4) return fail(MOE_EINVAL, "moe_layer_forward: H % 4 != 0");
    if (T == 0) return MOE_OK;
    if (!x_bf16 || !logits || !topk_ids || !topk_w || !out)
        return fail(MOE_EINVAL, "moe_layer_forward: null pointer");
    const LayerWs lw = layer_ws(layer, T, k);
    if (!ws || ws_bytes < lw.total)
        return fail(MOE_EWORKSPACE,
                    "moe_layer_forward: workspace needs " + std::to_string(lw.total) + " bytes");
    if (reinterpret_cast<uintptr_t>(ws) % kAlign)
        return fail(MOE_EINVAL, "moe_layer_forward: workspace must be 256-byte aligned");
    uint8_t* w = static_cast<uint8_t*>(ws);
    if (layer_small_ok(li, T, k)) {
        int fmt = MOE_FMT_NVFP4;
        while (!li.count[fmt]) ++fmt;
        return launch_layer_small(li.view, fmt, x_bf16, logits, T, k, topk_ids, topk_w,
                                  reinterpret_cast<uint16_t*>(w), y_shared, out, stream);
    }
    int32_t* counts = reinterpret_cast<int32_t*>(w + lw.counts);
    int32_t* offsets = reinterpret_cast<int32_t*>(w + lw.offsets);
    int32_t* perm_src = reinterpret_cast<int32_t*>(w + lw.perm_src);
    int32_t* inv_perm = reinterpret_cast<int32_t*>(w + lw.inv_perm);
    float* y_perm = reinterpret_cast<float*>(w + lw.y_perm);
    st = moe_route_permute(logits, T, layer->E, k, topk_ids, topk_w, counts, offsets, perm_src,
                           inv_perm, w + lw.pws, lw.ffn - lw.pws, stream);
    if (st) return st;
    if (li.view.rot) {
        // rotated: the down outputs stay rotated and the combine rotates each
        // slot back (one pass over y instead of two)
        const size_t xbytes = gateup_ws(layer, T, k);
        uint16_t* h16 = reinterpret_cast<uint16_t*>(w + lw.ffn + xbytes);
        st = run_gateup(li, x_bf16, perm_src, offsets, T, k, h16,
                        reinterpret_cast<uint16_t*>(w + lw.ffn), nullptr, stream);
        if (st) return st;
        st = run_down(li, h16, offsets, T, k, y_perm, stream, false);
        if (st) return st;
        return launch_combine_rot(li.view, y_perm, inv_perm, topk_ids, topk_w, y_shared, T, k,
                                  out, stream);
    }
    st = moe_expert_ffn_q(layer, x_bf16, perm_src, offsets, T, k, y_perm, w + lw.ffn,
                          lw.y_perm - lw.ffn, stream);
    if (st) return st;
    return launch_combine(y_perm, inv_perm, topk_w, y_shared, T, k, layer->H, out, stream);
}

// moe_layer_forward_shared: the routed layer's workspace | the shared
// expert's (moe_shared_ffn) | y_shared [T, H] fp32 (the unfused order).
size_t moe_layer_forward_shared_workspace_bytes(const moe_qlayer* layer,
                                                const moe_qlayer* shared, int64_t T, int32_t k) {
    if (!layer || !shared || T < 0 || k < 1 || layer->E < 1 || layer->H <= 0 ||
        layer->I <= 0 || shared->H <= 0 || shared->I <= 0)
        return 0;
    return align_up(layer_ws(layer, T, k).total) + shared_ws(shared, T) +
           align_up((size_t)T * layer->H * 4);
}

int moe_layer_forward_shared(const moe_qlayer* layer, const moe_qlayer* shared,
                             const uint16_t* x_bf16, const float* logits, int64_t T, int32_t k,
                             int32_t* topk_ids, float* topk_w, float* out, void* ws,
                             size_t ws_bytes, void* stream) {
    g_last_error.clear();
    LayerInfo li, ls;
    int st = check_layer("moe_layer_forward_shared", layer, li);
    if (st) return st;
    st = check_layer("moe_layer_forward_shared (shared layer)", shared, ls);
    if (st) return st;
    if (shared->E != 1)
        return fail(MOE_EINVAL, "moe_layer_forward_shared: the shared layer must have E == 1");
    if (shared->rot_signs)
        return fail(MOE_EUNSUPPORTED,
                    "moe_layer_forward_shared: a rotated shared layer is not supported");
    if (shared->H != layer->H)
        return fail(MOE_EINVAL, "moe_layer_forward_shared: the shared layer's H differs");
    st = check_route_sizes("moe_layer_forward_shared", T, layer->E, k);
    if (st) return st;
    if (layer->H % 4) return fail(MOE_EINVAL, "moe_layer_forward_shared: H % 4 != 0");
    if (T == 0) return MOE_OK;
    if (!x_bf16 || !logits || !topk_ids || !topk_w || !out)
        return fail(MOE_EINVAL, "moe_layer_forward_shared: null pointer");
    const size_t lw = layer_ws(layer, T, k).total;
    const size_t sw = shared_ws(shared, T);
    const size_t need = align_up(lw) + sw + align_up((size_t)T * layer->H * 4);
    if (!ws || ws_bytes < need)
        return fail(MOE_EWORKSPACE, "moe_layer_forward_shared: workspace needs " +
                                        std::to_string(need) + " bytes");
    if (reinterpret_cast<uintptr_t>(ws) % kAlign)
        return fail(MOE_EINVAL, "moe_layer_forward_shared: workspace must be 256-byte aligned");
    uint8_t* w = static_cast<uint8_t*>(ws);
    uint8_t* wsh = w + align_up(lw);
    if (layer_small_ok(li, T, k) && !li.view.rot && ls.count[MOE_FMT_BF16] == 1) {
        int fmt = MOE_FMT_NVFP4;
        while (!li.count[fmt]) ++fmt;
        // the shared workspace as moe_shared_ffn lays it out: x16 | h16 | partials
        uint16_t* sh_h16 = reinterpret_cast<uint16_t*>(wsh + align_up((size_t)T * shared->H * 2));
        float* sh_part = reinterpret_cast<float*>(wsh + align_up((size_t)T * shared->H * 2) +
                                                  align_up((size_t)T * shared->I * 2));
        return launch_layer_small_shared(li.view, fmt, ls.view, x_bf16, logits, T, k, topk_ids,
                                         topk_w, reinterpret_cast<uint16_t*>(w), sh_h16, sh_part,
                                         out, stream);
    }
    float* y_sh = reinterpret_cast<float*>(wsh + sw);
    st = moe_shared_ffn(shared, x_bf16, T, y_sh, wsh, sw, stream);
    if (st) return st;
    return moe_layer_forward(layer, x_bf16, logits, T, k, y_sh, topk_ids, topk_w, out, w, lw,
                             stream);
}

int moe_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    g_last_error.clear();
    if (!buf || !sink) return fail(MOE_EINVAL, "moe_probe_read: null pointer");
    if (bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
        return fail(MOE_EINVAL, "moe_probe_read: bytes and buf must be multiples of 16");
    if (bytes == 0) return MOE_OK;
    return launch_probe_read(buf, bytes, sink, MOE_PROBE_BLOCKS, stream);
}

int moe_dequant_q(const moe_qlayer* layer, int32_t expert, int32_t proj, float* out,
                  void* stream) {
    g_last_error.clear();
    LayerInfo li;
    int st = check_layer("moe_dequant_q", layer, li);
    if (st) return st;
    if (expert < 0 || expert >= layer->E) return fail(MOE_EINVAL, "moe_dequant_q: bad expert");
    if (proj < MOE_PROJ_GATE || proj > MOE_PROJ_DOWN) return fail(MOE_EINVAL, "moe_dequant_q: bad proj");
    if (!out) return fail(MOE_EINVAL, "moe_dequant_q: out is NULL");
    // the record index of this expert within its format's pool (host-side)
    const int fmt = layer->fmt_host[expert];
    int32_t ridx = 0;
    if (layer->record_mode == MOE_REC_RESIDENT)
        ridx = expert;
    else
        for (int e = 0; e < expert; ++e) ridx += layer->fmt_host[e] == fmt;
    return launch_dequant(li.view, fmt, ridx, proj, out, stream);
}

}  // extern "C"
