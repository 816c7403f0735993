"""GPU parity on the edges of the boundary's contract:

* per-expert VQ codebooks (moe_qlayer.vq_codebook_stride != 0: each VQ
  record has its own three codebooks at index(e) * stride) through the
  decode kernels, the grouped GEMM, the fused one-call layer and the dequant
  hook, in a layer where VQ record indices differ from expert ids;
* activations across the whole range the matrix cores' fp16 operands hold:
  outlier channels up to the largest bf16 value below 65504 are exact;
* a token with an activation beyond that range: its own output row is not
  finite, every other token's row is unaffected (the products of one token
  never mix with another's).
"""

import numpy as np
import pytest
import torch

import bit_quantized_moe_route_amd as moeq
import oracle
import synth
from bit_quantized_moe_route_amd.layers import build_layer
from tests.gpu_common import assert_rows_close, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
CB_STRIDE = moeq.VQ_NCODE * 16          # one 65536 x 8 fp16 codebook


def to_np(t):
    return t.detach().cpu().numpy()


# ------------------------------------------------------- per-expert codebooks

def _cbx_layer(wl):
    """wl's layer with every VQ record's own codebooks (record order)."""
    fmt = synth.tier_map(wl)
    vq = [e for e in range(wl.E) if fmt[e] == synth.FMT_VQ]      # ascending = record order
    cbs = [np.concatenate([synth.vq_codebook_expert(wl, e, p) for e in vq]) for p in range(3)]
    return build_layer(
        wl.E, wl.H, wl.I, fmt,
        nvfp4_weights=lambda e, p: synth.nvfp4_source_weights(wl, e, p),
        vq_codes=lambda e, p: (synth.vq_codes(wl, e, p), synth.vq_scales(wl, e, p)),
        codebooks=cbs, codebook_stride=CB_STRIDE, device=DEV, workers=8)


def _cbx_weights(wl, e):
    fmt = synth.tier_map(wl)[e]
    W = []
    for p in range(3):
        if fmt == synth.FMT_VQ:
            W.append(oracle.vq_dequant(synth.vq_codes(wl, e, p), synth.vq_scales(wl, e, p),
                                       synth.vq_codebook_expert(wl, e, p)))
        else:
            W.append(oracle.nvfp4_dequant(*oracle.nvfp4_quantize(
                synth.nvfp4_source_weights(wl, e, p))))
    return W


CBX_MIXED = synth.small_workload("cbx_mixed", E=10, k=2, H=272, I=80, T=9, fmt="mixed",
                                 cfg=180, n_nvfp4=4)
CBX_VQ = synth.small_workload("cbx_vq", E=8, k=2, H=256, I=96, T=4, fmt="vq", cfg=181)


@pytest.mark.parametrize("T", [9, 260])
def test_per_expert_codebooks_forward(T):
    """The decode kernels (T = 9) and the grouped GEMM (T = 260) read each VQ
    expert's own codebooks: every y_perm row and every output row against
    the oracle with those codebooks; the dequant hook bit-exact."""
    wl = CBX_MIXED
    say("per-expert codebooks", T)
    lay = _cbx_layer(wl)
    fmt = synth.tier_map(wl)
    assert lay.c().vq_codebook_stride == CB_STRIDE
    # record index != expert id for the VQ experts of this mixed layer
    assert any(lay.record_index(e) != e for e in range(wl.E) if fmt[e] == synth.FMT_VQ)
    W = {e: _cbx_weights(wl, e) for e in range(wl.E)}
    for e in range(wl.E):
        for p in range(3):
            got = to_np(moeq.dequant_q(lay, e, p)).astype(np.float64)
            assert np.array_equal(got, W[e][p]), (e, p)
    x_bits = synth.activations(wl, T)
    lg = synth.logits(wl, T)
    r = moeq.forward(lay, torch.from_numpy(x_bits.view(np.int16)).to(DEV),
                     torch.from_numpy(lg).to(DEV), wl.k)
    torch.cuda.synchronize()
    out, ids, w, y = oracle.forward(x_bits, lg, wl.k, lambda e: W[e])
    assert np.array_equal(to_np(r["topk_ids"]), ids)
    inv = to_np(r["inv_perm"]).reshape(T, wl.k)
    y_perm = to_np(r["y_perm"])
    for j in range(wl.k):
        assert_rows_close(y_perm[inv[:, j]], y[:, j], f"per-expert codebooks y slot {j}")
    assert_rows_close(to_np(r["out"]), out, "per-expert codebooks out")


def test_per_expert_codebooks_fused_layer():
    """A VQ-only layer with per-expert codebooks through the fused decode
    path of moe_layer_forward (T k = 8 assignments): routing inside gate/up,
    the combine inside down."""
    wl = CBX_VQ
    T = wl.T[0]
    say("per-expert codebooks, fused layer")
    lay = _cbx_layer(wl)
    W = {e: _cbx_weights(wl, e) for e in range(wl.E)}
    x_bits = synth.activations(wl, T)
    lg = synth.logits(wl, T)
    ids, w, out = moeq.layer_forward(lay, torch.from_numpy(x_bits.view(np.int16)).to(DEV),
                                     torch.from_numpy(lg).to(DEV), wl.k)
    torch.cuda.synchronize()
    ref, ref_ids, ref_w, _ = oracle.forward(x_bits, lg, wl.k, lambda e: W[e])
    assert np.array_equal(to_np(ids), ref_ids)
    assert_rows_close(to_np(out), ref, "per-expert codebooks fused out")


def test_layer_descriptor_rejects_a_short_codebook_stride():
    wl = CBX_VQ
    lay = _cbx_layer(wl)
    lay.codebook_stride = CB_STRIDE - 16
    lay._c = None
    x = torch.zeros((2, wl.H), dtype=torch.int16, device=DEV)
    lg = torch.zeros((2, wl.E), dtype=torch.float32, device=DEV)
    with pytest.raises(moeq.MoeError) as ei:
        moeq.layer_forward(lay, x, lg, wl.k)
    assert ei.value.status == moeq.MOE_EINVAL


# ------------------------------------------------------- activation range

OUT_WL = synth.small_workload("outliers", E=8, k=2, H=512, I=256, T=40, cfg=182)
BIG = np.float32(65280.0)       # the largest bf16 value below fp16's 65504
OUT_CH = (3, 130, 300, 511)     # outlier channels
COL_SCALE = np.float32(2.0 ** -10)


def _outlier_source(wl, e, p):
    """The workload's weights with the outlier channels' input columns scaled
    by 2^-10 (gate and up), as a layer whose outlier channels carry small
    weights: the products stay inside fp16 while x spans its whole range."""
    w = synth.nvfp4_source_weights(wl, e, p)
    if p != synth.PROJ_DOWN:
        w = w.copy()
        w[:, list(OUT_CH)] *= COL_SCALE
    return w


def _outlier_layer(wl):
    return build_layer(wl.E, wl.H, wl.I, synth.tier_map(wl),
                       nvfp4_weights=lambda e, p: _outlier_source(wl, e, p), device=DEV,
                       workers=8)


def _outlier_x(wl, T):
    x = synth.activations(wl, T)
    f = oracle.bf16_bits_to_f64(x).astype(np.float32)
    rs = np.random.default_rng(7)
    for t in range(T):
        for c in OUT_CH:
            f[t, c] = rs.choice([-1, 1]) * rs.choice([BIG, np.float32(3000.0), np.float32(2e4)])
    # bf16 bits of values already exact in bf16 (BIG, 3000, 2e4 round to
    # themselves except 2e4 -> 19968, still below 65504)
    return synth.f32_to_bf16_bits(f)


@pytest.mark.parametrize("T", [40, 200])
def test_outlier_activations_within_fp16_range(T):
    """Tokens with channels at +-65280 (the largest bf16 value the fp16
    operands hold), +-2e4 and +-3000: decode (T = 40) and grouped GEMM
    (T = 200) rows within tolerance of the oracle."""
    wl = OUT_WL
    say("outlier activations", T)
    lay = _outlier_layer(wl)
    x_bits = _outlier_x(wl, T)
    xf = oracle.bf16_bits_to_f64(x_bits)
    assert np.max(np.abs(xf)) == float(BIG) and np.max(np.abs(xf)) <= 65504
    W = {e: [oracle.nvfp4_dequant(*oracle.nvfp4_quantize(_outlier_source(wl, e, p)))
             for p in range(3)] for e in range(wl.E)}
    lg = synth.logits(wl, T)
    r = moeq.forward(lay, torch.from_numpy(x_bits.view(np.int16)).to(DEV),
                     torch.from_numpy(lg).to(DEV), wl.k)
    torch.cuda.synchronize()
    out, ids, w, y = oracle.forward(x_bits, lg, wl.k, lambda e: W[e])
    # h stays inside fp16 for this layer (the kernels' h operand)
    for e in range(wl.E):
        g = xf @ W[e][0].T
        u = xf @ W[e][1].T
        assert np.max(np.abs(g * u / (1 + np.exp(-np.clip(g, -700, 700))))) < 65504
    inv = to_np(r["inv_perm"]).reshape(T, wl.k)
    y_perm = to_np(r["y_perm"])
    for j in range(wl.k):
        assert_rows_close(y_perm[inv[:, j]], y[:, j], f"outliers y slot {j}")
    assert_rows_close(to_np(r["out"]), out, "outliers out")


@pytest.mark.parametrize("T", [12, 160])
def test_out_of_range_token_stays_in_its_row(T):
    """One token with a channel at 1e5 (beyond the fp16 operand range, which
    the header states as the limit): that token's output row is not finite,
    and every other token's row still matches the oracle."""
    wl = OUT_WL
    say("out-of-range token", T)
    lay = _outlier_layer(wl)
    x_bits = synth.activations(wl, T)
    bad = T // 3
    f = oracle.bf16_bits_to_f64(x_bits).astype(np.float32)
    f[bad, 17] = np.float32(1e5)
    x_bits = synth.f32_to_bf16_bits(f)
    lg = synth.logits(wl, T)
    r = moeq.forward(lay, torch.from_numpy(x_bits.view(np.int16)).to(DEV),
                     torch.from_numpy(lg).to(DEV), wl.k)
    torch.cuda.synchronize()
    got = to_np(r["out"])
    assert not np.all(np.isfinite(got[bad]))
    keep = np.array([t for t in range(T) if t != bad])
    W = {e: [oracle.nvfp4_dequant(*oracle.nvfp4_quantize(_outlier_source(wl, e, p)))
             for p in range(3)] for e in range(wl.E)}
    out, _, _, _ = oracle.forward(x_bits[keep], lg[keep], wl.k, lambda e: W[e])
    assert_rows_close(got[keep], out, "tokens beside the out-of-range one")
