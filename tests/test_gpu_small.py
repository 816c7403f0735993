"""GPU parity at sizes the oracle finishes in seconds: every step of the path
through the C ABI against the oracle, element by element.  Shapes span
several tiles and ragged tails (inputs not a multiple of the 128/256-input
tile, odd token counts, token counts past 16, 32 and 64)."""

import numpy as np
import pytest
import torch

import bit_quantized_moe_route_amd as moeq
import oracle
import synth
from tests.gpu_common import (W_TOL, assert_rows_close, build_shared_layer, build_small_layer,
                               say)
from tests.oracle_runs import expert_weights, shared_weights

pytestmark = pytest.mark.gpu

DEV = "cuda"

SMALL = {
    "tiny": synth.TINY,
    "nv_ragged": synth.small_workload("nv_ragged", E=16, k=4, H=272, I=80, T=37, cfg=101),
    "vq_small": synth.small_workload("vq_small", E=12, k=3, H=512, I=144, T=21, fmt="vq", cfg=102),
    "vq_ragged": synth.small_workload("vq_ragged", E=8, k=2, H=208, I=48, T=9, fmt="vq", cfg=103),
    "mixed_small": synth.small_workload("mixed_small", E=24, k=6, H=384, I=96, T=70, fmt="mixed",
                                        logits="hot", cfg=104, n_nvfp4=9, n_hot=4, hot_share=0.6),
    "nv_k1": synth.small_workload("nv_k1", E=4, k=1, H=128, I=32, T=5, cfg=105),
    "nv_kE": synth.small_workload("nv_kE", E=6, k=6, H=160, I=64, T=3, cfg=106),
    # token counts that take the grouped-GEMM path: several 128-row tiles
    # per expert, skewed counts, ragged H (odd number of 16-row groups) and I
    "nv_prefill": synth.small_workload("nv_prefill", E=8, k=2, H=512, I=256, T=700, cfg=108),
    "nv_prefill_ragged": synth.small_workload("nv_prefill_ragged", E=16, k=4, H=272, I=80,
                                              T=300, logits="zipf", zipf_s=1.1, cfg=109),
    "mixed_prefill": synth.small_workload("mixed_prefill", E=12, k=3, H=256, I=128, T=260,
                                          fmt="mixed", logits="hot", cfg=110, n_nvfp4=5,
                                          n_hot=3, hot_share=0.6),
    # small-codebook VQ: one and two 8-bit codes per group, ragged shapes, and a
    # layer of all three formats (token counts past 64 and 128 included)
    "vq8_1": synth.small_workload("vq8_1", E=12, k=3, H=512, I=144, T=21, fmt="vq8", cfg=120,
                                  vq8_m=1),
    "vq8_2_ragged": synth.small_workload("vq8_2_ragged", E=8, k=2, H=208, I=48, T=9, fmt="vq8",
                                         cfg=121, vq8_m=2),
    "vq8_3_ragged": synth.small_workload("vq8_3_ragged", E=8, k=2, H=208, I=48, T=21, fmt="vq8",
                                         cfg=124, vq8_m=3),
    "mixed3_m3": synth.small_workload("mixed3_m3", E=24, k=6, H=384, I=96, T=70, fmt="mixed3",
                                      logits="hot", cfg=125, n_nvfp4=8, n_hot=4, hot_share=0.6,
                                      vq8_m=3),
    "mixed3": synth.small_workload("mixed3", E=24, k=6, H=384, I=96, T=70, fmt="mixed3",
                                   logits="hot", cfg=122, n_nvfp4=8, n_hot=4, hot_share=0.6,
                                   vq8_m=2),
    "mixed3_prefill": synth.small_workload("mixed3_prefill", E=12, k=3, H=256, I=128, T=260,
                                           fmt="mixed3", logits="hot", cfg=123, n_nvfp4=4,
                                           n_hot=3, hot_share=0.6, vq8_m=1),
    # BF16 experts (the weights as stored): alone with ragged shapes, beside
    # NVFP4 ones, and in the grouped-GEMM path next to NVFP4 experts
    "bf16_ragged": synth.small_workload("bf16_ragged", E=8, k=2, H=272, I=80, T=37, fmt="bf16",
                                        cfg=140),
    "nv_bf16": synth.small_workload("nv_bf16", E=16, k=4, H=384, I=96, T=70, fmt="nv_bf16",
                                    cfg=141, n_nvfp4=8),
    "nv_bf16_prefill": synth.small_workload("nv_bf16_prefill", E=12, k=3, H=272, I=144, T=260,
                                            fmt="nv_bf16", logits="zipf", zipf_s=1.1, cfg=142,
                                            n_nvfp4=6),
    # rotated layers (signs + Hadamard-128 on both sides of every matrix):
    # decode with ragged T, the grouped-GEMM path, all four formats
    "rot_nv": synth.small_workload("rot_nv", E=16, k=4, H=384, I=256, T=37, cfg=170, rot=True),
    "rot_prefill": synth.small_workload("rot_prefill", E=8, k=2, H=512, I=256, T=300,
                                        logits="zipf", zipf_s=1.1, cfg=171, rot=True),
    "rot_mixed3": synth.small_workload("rot_mixed3", E=24, k=6, H=384, I=128, T=70,
                                       fmt="mixed3", logits="hot", cfg=172, n_nvfp4=8, n_hot=4,
                                       hot_share=0.6, vq8_m=2, rot=True),
    "rot_nv_bf16": synth.small_workload("rot_nv_bf16", E=12, k=3, H=256, I=128, T=9,
                                        fmt="nv_bf16", cfg=173, n_nvfp4=5, rot=True),
    "rot_bf16_prefill": synth.small_workload("rot_bf16_prefill", E=6, k=2, H=256, I=128,
                                             T=200, fmt="nv_bf16", cfg=174, n_nvfp4=3,
                                             rot=True),
    # the decode / grouped-GEMM boundary (T = 127 decode kernels, with hot
    # experts past 16 tokens in several 16-token chunks; T = 128 the grouped
    # GEMM), the same weights
    "edge_t127": synth.small_workload("edge_t127", E=16, k=4, H=256, I=128, T=127,
                                      logits="zipf", zipf_s=1.1, cfg=228),
    "edge_t128": synth.small_workload("edge_t128", E=16, k=4, H=256, I=128, T=128,
                                      logits="zipf", zipf_s=1.1, cfg=228),
    "edge_t127_mixed3": synth.small_workload("edge_t127_mixed3", E=24, k=6, H=256, I=128,
                                             T=127, fmt="mixed3", logits="hot", cfg=229,
                                             n_nvfp4=8, n_hot=4, hot_share=0.6, vq8_m=2),
    # the library's largest layer shape in experts and slots (E = 1024, k = 16):
    # many active experts in the decode kernels' expert lookup and in the
    # grouped GEMM's work list
    "max_e_decode": synth.small_workload("max_e_decode", E=1024, k=16, H=128, I=64, T=20,
                                         cfg=226),
    "max_e_prefill": synth.small_workload("max_e_prefill", E=1024, k=16, H=128, I=64, T=200,
                                          logits="zipf", zipf_s=1.1, cfg=227),
    # the wide down-input rotation (signs + one Hadamard-512 per 512
    # intermediate channels): decode, the grouped GEMM with two 512-blocks
    # (two of a workgroup's four waves idle), rows enough for whole-row
    # workgroups with a wave taking two blocks (I = 2560: five blocks), and a
    # mixed-format layer
    "rot512_nv": synth.small_workload("rot512_nv", E=16, k=4, H=384, I=512, T=37, cfg=211,
                                      rot=True, rot_in2=512),
    "rot512_prefill": synth.small_workload("rot512_prefill", E=8, k=2, H=256, I=1024, T=300,
                                           logits="zipf", zipf_s=1.1, cfg=212, rot=True,
                                           rot_in2=512),
    "rot512_rows": synth.small_workload("rot512_rows", E=4, k=2, H=256, I=2560, T=600, cfg=213,
                                        rot=True, rot_in2=512),
    "rot512_mixed3": synth.small_workload("rot512_mixed3", E=24, k=6, H=384, I=512, T=70,
                                          fmt="mixed3", logits="hot", cfg=214, n_nvfp4=8,
                                          n_hot=4, hot_share=0.6, vq8_m=2, rot=True,
                                          rot_in2=512),
    # VQ codes in the grouped GEMM: small codebooks in LDS (1-3 codes per
    # group) and 16-bit codes from L2, inputs not a multiple of the 256-input
    # tile (zero codes past K still select a row: masked), a rotated layer
    "vq8_2_prefill": synth.small_workload("vq8_2_prefill", E=8, k=2, H=208, I=80, T=300,
                                          fmt="vq8", logits="zipf", zipf_s=1.1, cfg=126,
                                          vq8_m=2),
    "vq8_3_prefill": synth.small_workload("vq8_3_prefill", E=6, k=2, H=272, I=48, T=200,
                                          fmt="vq8", cfg=127, vq8_m=3),
    "vq8_1_prefill": synth.small_workload("vq8_1_prefill", E=6, k=3, H=400, I=144, T=150,
                                          fmt="vq8", cfg=128, vq8_m=1),
    "vq_prefill": synth.small_workload("vq_prefill", E=8, k=2, H=336, I=64, T=260, fmt="vq",
                                       cfg=129),
    "rot_vq8_prefill": synth.small_workload("rot_vq8_prefill", E=8, k=2, H=256, I=128, T=200,
                                            fmt="vq8", cfg=176, vq8_m=2, rot=True),
    # rotated 16-bit VQ in the grouped GEMM (128-token items: the middle
    # rotation's epilogue takes four 32-token tiles), two 128-channel blocks
    "rot_vq_prefill": synth.small_workload("rot_vq_prefill", E=8, k=2, H=256, I=256, T=200,
                                           fmt="vq", logits="zipf", zipf_s=1.1, cfg=223,
                                           rot=True),
    # small-codebook VQ experts at mixed rates (1, 2 and 3 bits per weight in
    # one layer, three shared codebooks per projection): decode with ragged
    # shapes, the grouped GEMM under Zipf routing
    "vqmix_ragged": synth.small_workload("vqmix_ragged", E=12, k=3, H=208, I=48, T=21,
                                         fmt="vqmix", cfg=130, vq8_m=3),
    "vqmix_prefill": synth.small_workload("vqmix_prefill", E=12, k=3, H=272, I=80, T=260,
                                          fmt="vqmix", logits="zipf", zipf_s=1.1, cfg=131,
                                          vq8_m=3),
}

_layers = {}


def layer_for(name):
    if name not in _layers:
        _layers[name] = build_small_layer(SMALL[name], DEV)
    return _layers[name]


def to_np(t):
    return t.detach().cpu().numpy()


# ------------------------------------------------------------------ dequant

@pytest.mark.parametrize("name", ["tiny", "nv_ragged", "vq_small", "vq_ragged", "mixed_small"])
def test_dequant_bit_exact(name):
    wl = SMALL[name]
    say("dequant", name)
    layer = layer_for(name)
    for e in range(wl.E):
        W = expert_weights(wl, e)
        for p in range(3):
            got = to_np(moeq.dequant_q(layer, e, p)).astype(np.float64)
            assert np.array_equal(got, W[p]), (name, e, p)


@pytest.mark.parametrize("name", ["vq8_1", "vq8_2_ragged", "mixed3", "vq8_3_ragged",
                                  "vqmix_ragged"])
def test_dequant_vq8(name):
    """Small-codebook VQ decode: exact with one code per group; with two or
    three, the hook's fp32(fp32(C_0 + ..) * S) is within 2 roundings of the
    exact value.  Mixed-rate layers: every expert at its own rate, reading
    the first m of the layer's codebooks."""
    wl = SMALL[name]
    say("dequant vq8", name)
    layer = layer_for(name)
    tm = synth.tier_map(wl)
    vq8_tags = (synth.FMT_VQ8, synth.FMT_VQ8_M1, synth.FMT_VQ8_M2, synth.FMT_VQ8_M3)
    if wl.fmt == "vqmix":
        assert set(np.unique(tm).tolist()) == {synth.FMT_VQ8_M1, synth.FMT_VQ8_M2,
                                               synth.FMT_VQ8_M3}
    for e in np.flatnonzero(np.isin(tm, vq8_tags)):
        W = expert_weights(wl, int(e))
        for p in range(3):
            got = to_np(moeq.dequant_q(layer, int(e), p)).astype(np.float64)
            if synth.vq8_rate(wl, int(e)) == 1:
                assert np.array_equal(got, W[p]), (name, e, p)
            else:
                assert np.all(np.abs(got - W[p]) <= 2.0 ** -22 * np.abs(W[p])), (name, e, p)


@pytest.mark.parametrize("name", ["bf16_ragged", "nv_bf16"])
def test_dequant_bf16(name):
    """BF16 decode: the kernels' fp16 operand, i.e. the stored weight rounded
    to fp16 (nearest even), which is the weight itself for |w| >= 2^-17."""
    wl = SMALL[name]
    say("dequant bf16", name)
    layer = layer_for(name)
    tm = synth.tier_map(wl)
    for e in np.flatnonzero(tm == synth.FMT_BF16):
        W = expert_weights(wl, int(e))
        for p in range(3):
            got = to_np(moeq.dequant_q(layer, int(e), p)).astype(np.float64)
            assert np.array_equal(got, W[p].astype(np.float16).astype(np.float64)), (name, e, p)
            big = np.abs(W[p]) >= 2.0 ** -17
            assert np.array_equal(got[big], W[p][big])


# ------------------------------------------------------------------ route

def _route_check(lg, k):
    ids, w = moeq.route_topk(torch.from_numpy(lg).to(DEV), k)
    oids, ow = oracle.route_topk(lg, k)
    assert np.array_equal(to_np(ids), oids)
    assert np.max(np.abs(to_np(w).astype(np.float64) - ow)) <= W_TOL
    return to_np(ids)


@pytest.mark.parametrize("T,E,k,kind", [(4, 8, 2, "normal"), (1, 256, 8, "uniform"),
                                        (33, 256, 8, "uniform"), (300, 64, 5, "normal"),
                                        (7, 1024, 16, "normal"), (5, 600, 3, "uniform"),
                                        (9, 3, 3, "normal"), (4096, 256, 8, "zipf")])
def test_route_topk(T, E, k, kind):
    say("route", T, E, k, kind)
    if kind == "zipf":
        lg = synth.logits(synth.PREFILL, T)
    else:
        g = np.random.default_rng(T * 1000 + E)
        lg = (g.standard_normal((T, E)) if kind == "normal" else g.random((T, E))).astype(np.float32)
    _route_check(lg, k)


def test_route_ties():
    say("route ties")
    lg = np.zeros((3, 256), np.float32)
    lg[1, ::2] = 1.0                 # 128 tied maxima: ids 0, 2, 4, ...
    lg[2] = np.where(np.arange(256) % 3 == 0, -0.0, 0.0).astype(np.float32)
    lg[2, 200] = -1.0
    ids = _route_check(lg, 8)
    assert list(ids[0]) == list(range(8))
    assert list(ids[1]) == list(range(0, 16, 2))
    # coarse logits: many exact ties across the k-th place
    g = np.random.default_rng(3)
    lg = (np.round(g.standard_normal((64, 256)) * 2) / 2).astype(np.float32)
    _route_check(lg, 8)
    # -inf logits are allowed as long as each token's top logit is finite
    lg = np.full((2, 40), -np.inf, np.float32)
    lg[0, 39] = 1.0
    lg[1, 5] = -3.0
    lg[1, 17] = -3.0
    ids = _route_check(lg, 4)
    assert list(ids[0]) == [39, 0, 1, 2] and list(ids[1]) == [5, 17, 0, 1]


# ------------------------------------------------------------------ permute

# T*k <= 4096 runs in one workgroup; larger batches in up to 64 slices of
# >= 2048 assignments (513*8: two full slices and a ragged one; 20000*8: 53
# slices of 3072)
@pytest.mark.parametrize("T,E,k", [(4, 8, 2), (1, 256, 8), (32, 256, 8), (200, 16, 4),
                                   (4096, 256, 8), (1500, 1024, 16), (3, 1, 1), (0, 8, 2),
                                   (512, 64, 8), (513, 64, 8), (20000, 256, 8)])
def test_permute(T, E, k):
    say("permute", T, E, k)
    g = np.random.default_rng(T + E)
    if T in (4096, 20000):
        ids, _ = oracle.route_topk(synth.logits(synth.PREFILL, T), k)
    else:
        ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, k), np.int32)
    got = moeq.permute(torch.from_numpy(ids).to(DEV), E)
    want = oracle.permute(ids, E)
    for a, b, nm in zip(got, want, ["counts", "offsets", "perm_src", "inv_perm"]):
        assert np.array_equal(to_np(a), b), nm


# ------------------------------------------------------------------ combine

@pytest.mark.parametrize("T,k,H", [(4, 2, 256), (37, 8, 6144), (5, 16, 64)])
def test_combine(T, k, H):
    say("combine", T, k, H)
    g = np.random.default_rng(T)
    E = max(2 * k, 8)
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)])
    _, w = oracle.route_topk(g.standard_normal((T, E)).astype(np.float32), k)
    _, _, perm_src, inv_perm = oracle.permute(ids, E)
    y_perm = g.standard_normal((T * k, H)).astype(np.float32)
    out = moeq.combine(torch.from_numpy(y_perm).to(DEV), torch.from_numpy(inv_perm).to(DEV),
                       torch.from_numpy(w.astype(np.float32)).to(DEV))
    y = y_perm.astype(np.float64)[inv_perm].reshape(T, k, H)
    ref = oracle.combine(y, w.astype(np.float32).astype(np.float64))
    assert_rows_close(to_np(out), ref, "combine", tol=1e-5)


@pytest.mark.parametrize("T,k,H", [(4, 2, 256), (37, 8, 6144), (5, 16, 64)])
def test_combine_shared(T, k, H):
    """combine + the shared expert's output: against the oracle, and bit for
    bit the fp32 sum of the routed combine and y_shared."""
    say("combine_shared", T, k, H)
    g = np.random.default_rng(T + 50)
    E = max(2 * k, 8)
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)])
    _, w = oracle.route_topk(g.standard_normal((T, E)).astype(np.float32), k)
    _, _, perm_src, inv_perm = oracle.permute(ids, E)
    y_perm = g.standard_normal((T * k, H)).astype(np.float32)
    y_sh = g.standard_normal((T, H)).astype(np.float32)
    args = [torch.from_numpy(a).to(DEV) for a in (y_perm, inv_perm, w.astype(np.float32))]
    ysh = torch.from_numpy(y_sh).to(DEV)
    out = moeq.combine_shared(*args, ysh)
    y = y_perm.astype(np.float64)[inv_perm].reshape(T, k, H)
    ref = oracle.combine_shared(y, w.astype(np.float32).astype(np.float64), y_sh)
    assert_rows_close(to_np(out), ref, "combine_shared", tol=1e-5)
    assert torch.equal(out, moeq.combine(*args) + ysh)


# ------------------------------------------------------------------ end to end

def _oracle_forward(wl, x_bits, lg):
    Wc = {}

    def weights(e):
        if e not in Wc:
            Wc[e] = expert_weights(wl, e)
        return Wc[e]
    return oracle.forward(x_bits, lg, wl.k, weights)


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_parity(name):
    wl = SMALL[name]
    T = wl.T[0]
    say("forward", name, T)
    layer = layer_for(name)
    x_bits = synth.activations(wl, T)
    lg = synth.logits(wl, T)
    x = torch.from_numpy(x_bits.view(np.int16)).to(DEV)
    r = moeq.forward(layer, x, torch.from_numpy(lg).to(DEV), wl.k)
    out, ids, w, y = _oracle_forward(wl, x_bits, lg)
    assert np.array_equal(to_np(r["topk_ids"]), ids)
    counts, offsets, perm_src, inv_perm = oracle.permute(ids, wl.E)
    assert np.array_equal(to_np(r["perm_src"]), perm_src)
    assert np.array_equal(to_np(r["offsets"]), offsets)
    y_ref = y.reshape(T * wl.k, wl.H)[perm_src]
    assert_rows_close(to_np(r["y_perm"]), y_ref, name + " y_perm")
    assert_rows_close(to_np(r["out"]), out, name + " out")


def test_forward_deterministic():
    wl = SMALL["mixed_small"]
    T = wl.T[0]
    say("determinism", wl.name)
    layer = layer_for("mixed_small")
    x = torch.from_numpy(synth.activations(wl, T).view(np.int16)).to(DEV)
    lg = torch.from_numpy(synth.logits(wl, T)).to(DEV)
    a = moeq.forward(layer, x, lg, wl.k)
    b = moeq.forward(layer, x, lg, wl.k)
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_zero_scale_expert_gives_exact_zero():
    """An NVFP4 expert whose scales are all zero outputs exactly 0."""
    say("zero-scale expert")
    wl = synth.small_workload("zero", E=4, k=2, H=256, I=64, T=6, cfg=107)
    from bit_quantized_moe_route_amd.layers import build_layer
    layer = build_layer(wl.E, wl.H, wl.I, synth.tier_map(wl),
                        nvfp4_weights=lambda e, p: (np.zeros(synth.proj_shape(wl, p), np.float32)
                                                    if e == 1 else
                                                    synth.nvfp4_source_weights(wl, e, p)),
                        device=DEV)
    lg = np.zeros((wl.T[0], wl.E), np.float32)
    lg[:, 1] = 5.0                                   # every token picks expert 1 first
    x = torch.from_numpy(synth.activations(wl, wl.T[0]).view(np.int16)).to(DEV)
    r = moeq.forward(layer, x, torch.from_numpy(lg).to(DEV), wl.k)
    offs = to_np(r["offsets"])
    y = to_np(r["y_perm"])
    assert offs[2] - offs[1] == wl.T[0]
    assert np.all(y[offs[1]:offs[2]] == 0)


def test_t_zero_is_noop():
    say("T = 0")
    layer = layer_for("tiny")
    x = torch.empty((0, 256), dtype=torch.int16, device=DEV)
    lg = torch.empty((0, 8), dtype=torch.float32, device=DEV)
    r = moeq.forward(layer, x, lg, 2)
    assert r["out"].shape == (0, 256)
    assert torch.all(r["counts"] == 0) and torch.all(r["offsets"] == 0)


# ------------------------------------------------------------------ tier switch

def _forward_check(wl, layer, tiers, rep, label):
    T = wl.T[0]
    x_bits = synth.activations(wl, T, rep=rep)
    lg = synth.logits(wl, T, rep=rep)
    r = moeq.forward(layer, torch.from_numpy(x_bits.view(np.int16)).to(DEV),
                     torch.from_numpy(lg).to(DEV), wl.k)
    Wc = {}

    def weights(e):
        if e not in Wc:
            Wc[e] = expert_weights(wl, e, int(tiers[e]))
        return Wc[e]
    out, ids, w, y = oracle.forward(x_bits, lg, wl.k, weights)
    assert np.array_equal(to_np(r["topk_ids"]), ids)
    counts, offsets, perm_src, inv_perm = oracle.permute(ids, wl.E)
    y_ref = y.reshape(T * wl.k, wl.H)[perm_src]
    assert_rows_close(to_np(r["y_perm"]), y_ref, label + " y_perm")
    assert_rows_close(to_np(r["out"]), out, label + " out")


def test_tier_switch_between_calls():
    """A resident layer (every expert packed in NVFP4, VQ and VQ8) moves experts
    between tiers between calls; each call matches the oracle under the tier
    map in force, including the hot experts moved to the 4-bit tier and
    all-one-format maps."""
    wl = synth.small_workload("tiers", E=24, k=6, H=256, I=96, T=40, fmt="mixed", logits="hot",
                              cfg=130, n_nvfp4=9, n_hot=4, hot_share=0.6, vq8_m=2)
    say("tier switch")
    fmts = {synth.FMT_NVFP4, synth.FMT_VQ, synth.FMT_VQ8}
    layer = build_small_layer(wl, DEV, resident_formats=fmts)
    maps = [synth.tier_map(wl), synth.tier_map_hot(wl),
            np.full(wl.E, synth.FMT_VQ8, np.uint8), np.full(wl.E, synth.FMT_NVFP4, np.uint8),
            np.random.default_rng(5).choice([1, 2, 3], size=wl.E).astype(np.uint8)]
    for i, tm in enumerate(maps):
        if i:
            layer.set_tiers(tm)
        _forward_check(wl, layer, tm, i, f"tiers {i}")
        e = int(np.flatnonzero(tm == tm[0])[0])
        W = expert_weights(wl, e, int(tm[e]))
        got = to_np(moeq.dequant_q(layer, e, 0)).astype(np.float64)
        if tm[e] == synth.FMT_VQ8:
            assert np.all(np.abs(got - W[0]) <= 2.0 ** -22 * np.abs(W[0]))
        else:
            assert np.array_equal(got, W[0])


# ------------------------------------------------------------------ shared expert

SHARED = {
    # one token; 37 tokens (three 16-token chunks, ragged H and I); the
    # grouped-GEMM path with a ragged last 128-token tile; a larger one; a
    # mixed NVFP4 / VQ routed layer
    "sh_t1": synth.small_workload("sh_t1", E=8, k=2, H=256, I=128, T=1, cfg=150, shared=True),
    "sh_ragged": synth.small_workload("sh_ragged", E=16, k=4, H=272, I=80, T=37, cfg=151,
                                      shared=True),
    "sh_prefill": synth.small_workload("sh_prefill", E=8, k=2, H=272, I=80, T=300, cfg=152,
                                       logits="zipf", zipf_s=1.1, shared=True),
    "sh_prefill_big": synth.small_workload("sh_prefill_big", E=8, k=2, H=512, I=256, T=700,
                                           cfg=153, shared=True),
    "sh_mixed": synth.small_workload("sh_mixed", E=24, k=6, H=384, I=96, T=70, fmt="mixed",
                                     logits="hot", cfg=154, n_nvfp4=9, n_hot=4, hot_share=0.6,
                                     shared=True),
}


@pytest.mark.parametrize("name", list(SHARED))
def test_shared_expert_forward(name):
    """Routed experts + the BF16 shared expert: the shared FFN on every token
    and the combined output against the oracle."""
    wl = SHARED[name]
    T = wl.T[0]
    say("shared forward", name, T)
    layer = build_small_layer(wl, DEV)
    shared = build_shared_layer(wl, DEV)
    x_bits = synth.activations(wl, T)
    lg = synth.logits(wl, T)
    x = torch.from_numpy(x_bits.view(np.int16)).to(DEV)
    r = moeq.forward(layer, x, torch.from_numpy(lg).to(DEV), wl.k, shared=shared)
    Ws = shared_weights(wl)
    assert_rows_close(to_np(r["y_shared"]), oracle.expert_ffn(x_bits, *Ws), name + " y_shared")
    Wc = {}

    def weights(e):
        if e not in Wc:
            Wc[e] = expert_weights(wl, e)
        return Wc[e]
    out, ids, w, y = oracle.forward(x_bits, lg, wl.k, weights, shared_weights=Ws)
    assert np.array_equal(to_np(r["topk_ids"]), ids)
    assert_rows_close(to_np(r["out"]), out, name + " out")
    # the shared layer's dequant hook: the stored bf16 weights as fp16
    for p in range(3):
        got = to_np(moeq.dequant_q(shared, 0, p)).astype(np.float64)
        assert np.array_equal(got, Ws[p].astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("T", [37, 300])
def test_shared_ffn_matches_routed_call(T):
    """moe_shared_ffn computes moe_expert_ffn_q with the identity map (the
    decode path splits the gate/up inputs over more workgroups, so the fp32
    sums are grouped differently; the grouped-GEMM path is the same kernel)."""
    wl = SHARED["sh_ragged"]
    say("shared = identity-routed", T)
    shared = build_shared_layer(wl, DEV)
    x = torch.from_numpy(synth.activations(wl, T).view(np.int16)).to(DEV)
    perm = torch.arange(T, dtype=torch.int32, device=DEV)
    offs = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    a = moeq.shared_ffn(shared, x)
    b = moeq.expert_ffn_q(shared, x, perm, offs, 1)
    if T >= 128:
        assert torch.equal(a, b)
    else:
        assert_rows_close(to_np(a), to_np(b).astype(np.float64), "shared vs routed", tol=1e-3)


@pytest.mark.parametrize("fmt,T", [(synth.FMT_NVFP4, 20), (synth.FMT_VQ8, 9), (synth.FMT_VQ, 33),
                                   (synth.FMT_NVFP4, 150), (synth.FMT_NVFP4R, 20),
                                   (synth.FMT_NVFP4R, 150)])
def test_shared_expert_other_formats(fmt, T):
    """A shared-expert layer in a low-bit format goes through the same calls."""
    from bit_quantized_moe_route_amd.layers import build_layer
    wl = synth.small_workload("sh_fmt", E=1, k=1, H=272, I=96, T=T, cfg=160, vq8_m=2)
    say("shared in format", fmt, T)
    lay = build_layer(
        1, wl.H, wl.I, np.array([fmt], np.uint8),
        nvfp4_weights=lambda e, p: synth.nvfp4_source_weights(wl, e, p),
        vq_codes=lambda e, p: (synth.vq_codes(wl, e, p), synth.vq_scales(wl, e, p)),
        codebooks=[synth.vq_codebook(wl, p) for p in range(3)] if fmt == synth.FMT_VQ else None,
        vq8_codes=lambda e, p: (synth.vq8_codes(wl, e, p), synth.vq_scales(wl, e, p)),
        codebooks8=[synth.vq8_codebooks(wl, p) for p in range(3)] if fmt == synth.FMT_VQ8 else None,
        vq8_m=2, device=DEV, workers=1, nvfp4r_shift=synth.NVFP4R_SHIFT)
    x_bits = synth.activations(wl, T)
    y = moeq.shared_ffn(lay, torch.from_numpy(x_bits.view(np.int16)).to(DEV))
    ref = oracle.expert_ffn(x_bits, *expert_weights(wl, 0, fmt))
    assert_rows_close(to_np(y), ref, f"shared fmt {fmt}")


# ------------------------------------------------------------------ rotation

def test_rotated_dequant_is_the_stored_matrix():
    """A rotated layer's dequant hook returns the stored (rotated) matrices."""
    from tests.oracle_runs import stored_weights
    wl = SMALL["rot_nv"]
    say("rotated dequant")
    layer = layer_for("rot_nv")
    for e in (0, 7, 15):
        W = stored_weights(wl, e)
        for p in range(3):
            assert np.array_equal(to_np(moeq.dequant_q(layer, e, p)).astype(np.float64), W[p])


@pytest.mark.parametrize("in2_block,I,T", [(128, 128, 12), (512, 512, 12), (512, 1024, 160)])
def test_rotation_changes_nothing_for_unrotated_weights(in2_block, I, T):
    """Storing R_out W R_in^T (the library's offline rotation, in fp32) and
    running the rotated layer gives the plain layer's output within the
    tolerance: the online rotations undo the stored ones (also with the wide
    512-block on the down projection's input side, decode and grouped GEMM)."""
    from bit_quantized_moe_route_amd.layers import build_layer
    wl = synth.small_workload("rot_id", E=8, k=2, H=256, I=I, T=T, fmt="bf16", cfg=175)
    say("rotation round trip", in2_block, I, T)
    signs = {e: tuple(synth.rot_signs(wl, e, side) for side in range(5)) for e in range(wl.E)}
    sides = {0: (1, 0), 1: (2, 0), 2: (4, 3)}            # proj -> (out side, in side)

    def rotated(e, p):
        w = oracle.bf16_bits_to_f64(synth.bf16_weights(wl, e, p)).astype(np.float32)
        so, si = sides[p]
        return synth.f32_to_bf16_bits(moeq.rotate_matrix(
            w, signs[e][so], signs[e][si], block_in=in2_block if p == 2 else 128))

    plain = build_small_layer(wl, DEV)
    rot = build_layer(wl.E, wl.H, wl.I, synth.tier_map(wl), bf16_weights=rotated, device=DEV,
                      workers=4, rot_signs=lambda e: signs[e], rot_in2_block=in2_block)
    x = torch.from_numpy(synth.activations(wl, T).view(np.int16)).to(DEV)
    lg = torch.from_numpy(synth.logits(wl, T)).to(DEV)
    a = moeq.forward(plain, x, lg, wl.k)["out"]
    b = moeq.forward(rot, x, lg, wl.k)["out"]
    # bf16 rounding of the rotated weights: a few 2^-9 relative per weight
    assert_rows_close(to_np(b), to_np(a).astype(np.float64), "rotated vs plain", tol=2e-2)


# ------------------------------------------------------------------ measurement aid

@pytest.mark.parametrize("nbytes", [1 << 20, (1 << 20) + 48, 16])
def test_probe_read_reads_every_word_once(nbytes):
    """moe_probe_read's per-workgroup XORs combine to the XOR of every 32-bit
    word of the buffer (a word read twice or never would break it)."""
    say("probe read", nbytes)
    g = np.random.default_rng(nbytes)
    words = g.integers(0, 2**31, size=nbytes // 4, dtype=np.int64).astype(np.int32)
    sink = moeq.probe_read(torch.from_numpy(words).to(DEV))
    got = np.bitwise_xor.reduce(to_np(sink).astype(np.uint32))
    assert got == np.bitwise_xor.reduce(words.astype(np.uint32))
