"""GPU parity of the one-call layer forward (moe_layer_forward).

Decode batches (T*k <= 16, k <= 8) of single-format layers run the fused path
(routing inside the gate/up kernel, the gated combine inside the down kernel,
no permutation; a rotated layer rotates x into LDS inside the gate/up kernel
and its down outputs back inside the combine).  Its outputs are checked against the oracle
(routing bit-exact, rows within the FFN tolerance) and against the
step-by-step calls on the same inputs, which they must equal bit for bit:
both take each expert's products, partial sums and the combine in the same
order.  Batches outside the fused path (more assignments, mixed formats) go
through the step-by-step calls and must equal them too."""

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

# (workload, T): T*k <= 16 unless noted
CASES = {
    # the tiny layer of 8 experts, top-2, 4 tokens (8 assignments)
    "tiny": (synth.TINY, 4),
    # one token per batch, k = 1: three of the four slots of a wave are idle
    "nv_k1": (synth.small_workload("lf_nv_k1", E=4, k=1, H=128, I=32, T=5, cfg=180), 5),
    # k = 6: two slot groups, the second with two live slots; ragged H
    # (17 row groups) and I (one partial tile)
    "nv_k6": (synth.small_workload("lf_nv_k6", E=16, k=6, H=272, I=80, T=2, cfg=181), 2),
    # k = 5: the second slot group of the down + combine has one live slot
    "nv_k5": (synth.small_workload("lf_nv_k5", E=12, k=5, H=256, I=96, T=3, cfg=210), 3),
    # k = 8 over 32 experts, one token and two tokens
    "nv_k8_t1": (synth.small_workload("lf_nv_k8", E=32, k=8, H=384, I=256, T=1, cfg=182), 1),
    "nv_k8_t2": (synth.small_workload("lf_nv_k8", E=32, k=8, H=384, I=256, T=2, cfg=182), 2),
    # the other formats, inputs not a multiple of the 256-input tile
    "vq": (synth.small_workload("lf_vq", E=8, k=2, H=208, I=48, T=8, fmt="vq", cfg=183), 8),
    "vq8_1": (synth.small_workload("lf_vq8_1", E=12, k=3, H=512, I=144, T=5, fmt="vq8", cfg=184,
                                   vq8_m=1), 5),
    "vq8_2": (synth.small_workload("lf_vq8_2", E=8, k=8, H=208, I=80, T=2, fmt="vq8", cfg=185,
                                   vq8_m=2), 2),
    "vq8_3": (synth.small_workload("lf_vq8_3", E=8, k=2, H=208, I=48, T=3, fmt="vq8", cfg=186,
                                   vq8_m=3), 3),
    "bf16": (synth.small_workload("lf_bf16", E=8, k=4, H=272, I=80, T=4, fmt="bf16", cfg=187), 4),
    # outside the fused path: 18 assignments; mixed formats; a rotated layer
    "tiny_t9": (synth.TINY, 9),
    "mixed": (synth.small_workload("lf_mixed", E=24, k=6, H=384, I=96, T=2, fmt="mixed",
                                   logits="hot", cfg=188, n_nvfp4=9, n_hot=4, hot_share=0.6), 2),
    # rotated layers: small batches fused (the rotated x row in LDS, the
    # rotations between the passes, the down outputs rotated back inside the
    # combine): rows ending in half a 256-span, two slot groups of 4 (k = 8),
    # small-codebook and 16-bit VQ, BF16, the wide down-input rotation
    "rot": (synth.small_workload("lf_rot", E=16, k=4, H=384, I=256, T=1, cfg=189, rot=True), 1),
    "rot_k8_t2": (synth.small_workload("lf_rot_k8", E=32, k=8, H=256, I=128, T=2, cfg=219,
                                       rot=True), 2),
    "rot_vq8": (synth.small_workload("lf_rot_vq8", E=8, k=2, H=512, I=128, T=3, fmt="vq8",
                                     cfg=220, vq8_m=2, rot=True), 3),
    "rot_vq": (synth.small_workload("lf_rot_vq", E=8, k=2, H=256, I=128, T=4, fmt="vq",
                                    cfg=221, rot=True), 4),
    "rot_bf16": (synth.small_workload("lf_rot_bf16", E=8, k=3, H=384, I=128, T=2, fmt="bf16",
                                      cfg=222, rot=True), 2),
    # the fused rotated path holds the rotated x row in LDS up to H = 12288
    # (with 3-code small codebooks, 64 KB of LDS in all); one block more runs
    # the step-by-step calls
    "rot_h12288": (synth.small_workload("lf_rot_h12288", E=4, k=2, H=12288, I=128, T=1,
                                        fmt="vq8", cfg=224, vq8_m=3, rot=True), 1),
    "rot_h12416": (synth.small_workload("lf_rot_h12416", E=4, k=2, H=12416, I=128, T=1,
                                        cfg=225, rot=True), 1),
    # ... and outside the fused path the combine rotates the down outputs back:
    # many decode tokens with a half 256-span at the end of the rows, the
    # grouped-GEMM path, the wide down-input rotation (also fused: 9
    # assignments), and k = 16
    "rot_t40": (synth.small_workload("lf_rot_t40", E=16, k=4, H=384, I=256, T=40, cfg=215,
                                     rot=True), 40),
    "rot_prefill": (synth.small_workload("lf_rot_pf", E=8, k=2, H=256, I=256, T=160,
                                         logits="zipf", zipf_s=1.1, cfg=216, rot=True), 160),
    "rot512": (synth.small_workload("lf_rot512", E=12, k=3, H=384, I=512, T=3, cfg=217,
                                    rot=True, rot_in2=512), 3),
    "rot_k16": (synth.small_workload("lf_rot_k16", E=32, k=16, H=128, I=128, T=5, cfg=218,
                                     rot=True), 5),
    # the edges of the fused path: exactly 16 assignments (fused) and 17
    # (not), k = 9 > 8 at one token (not), 257 experts (not: more than 256)
    "edge_16": (synth.small_workload("lf_edge16", E=24, k=4, H=256, I=128, T=4, cfg=192), 4),
    "edge_17": (synth.small_workload("lf_edge17", E=24, k=1, H=256, I=128, T=17, cfg=193), 17),
    "edge_k9": (synth.small_workload("lf_edgek9", E=24, k=9, H=256, I=128, T=1, cfg=194), 1),
    "edge_e257": (synth.small_workload("lf_edgee257", E=257, k=8, H=128, I=64, T=2, cfg=195), 2),
}

_layers = {}


def layer_for(wl):
    if wl.name not in _layers:
        _layers[wl.name] = build_small_layer(wl, DEV)
    return _layers[wl.name]


def to_np(t):
    return t.detach().cpu().numpy()


def inputs(wl, T, rep=0):
    x_bits = synth.activations(wl, T, rep=rep)
    lg = synth.logits(wl, T, rep=rep)
    return (x_bits, lg, torch.from_numpy(x_bits.view(np.int16)).to(DEV),
            torch.from_numpy(lg).to(DEV))


def oracle_out(wl, x_bits, lg, shared=None):
    Wc = {}

    def weights(e):
        if e not in Wc:
            Wc[e] = expert_weights(wl, e)
        return Wc[e]
    return oracle.forward(x_bits, lg, wl.k, weights, shared_weights=shared)


@pytest.mark.parametrize("name", list(CASES))
def test_layer_forward_parity(name):
    wl, T = CASES[name]
    say("layer forward", name, T)
    lay = layer_for(wl)
    x_bits, lg, x, lgd = inputs(wl, T)
    ids, w, out = moeq.layer_forward(lay, x, lgd, wl.k)
    ref_out, ref_ids, ref_w, _ = oracle_out(wl, x_bits, lg)
    assert np.array_equal(to_np(ids), ref_ids)
    assert np.max(np.abs(to_np(w).astype(np.float64) - ref_w)) <= W_TOL
    assert_rows_close(to_np(out), ref_out, name + " out")
    # the same bits as the step-by-step calls
    r = moeq.forward(lay, x, lgd, wl.k)
    assert torch.equal(ids, r["topk_ids"])
    assert torch.equal(w, r["topk_w"])
    assert torch.equal(out, r["out"]), name


@pytest.mark.parametrize("name,T", [("sh_t1", 1), ("sh_k4", 4)])
def test_layer_forward_with_shared_expert(name, T):
    """y_shared added after the routed sum, as moe_combine_shared does."""
    wl = {"sh_t1": synth.small_workload("lf_sh_t1", E=8, k=2, H=256, I=128, T=1, cfg=190,
                                        shared=True),
          "sh_k4": synth.small_workload("lf_sh_k4", E=16, k=4, H=272, I=80, T=4, cfg=191,
                                        shared=True)}[name]
    say("layer forward + shared", name, T)
    lay = layer_for(wl)
    sh = build_shared_layer(wl, DEV)
    x_bits, lg, x, lgd = inputs(wl, T)
    y_sh = moeq.shared_ffn(sh, x)
    ids, w, out = moeq.layer_forward(lay, x, lgd, wl.k, y_shared=y_sh)
    ref_out, ref_ids, _, _ = oracle_out(wl, x_bits, lg, shared=shared_weights(wl))
    assert np.array_equal(to_np(ids), ref_ids)
    assert_rows_close(to_np(out), ref_out, name + " out")
    r = moeq.forward(lay, x, lgd, wl.k, shared=sh)
    assert torch.equal(out, r["out"])


def test_layer_forward_repeatable_and_reuses_workspace():
    """Two batches in a row through one workspace: each equals a fresh call
    (no state kept between calls), and a repeated call gives the same bits."""
    wl, T = CASES["nv_k8_t2"]
    say("layer forward workspace reuse")
    lay = layer_for(wl)
    ws = moeq.layer_workspace(lay, T, wl.k)
    res = []
    for rep in (0, 1, 0):
        _, _, x, lgd = inputs(wl, T, rep=rep)
        res.append(moeq.layer_forward(lay, x, lgd, wl.k, ws=ws))
    for a, b in zip(res[0], res[2]):
        assert torch.equal(a, b)
    _, _, x, lgd = inputs(wl, T, rep=1)
    fresh = moeq.layer_forward(lay, x, lgd, wl.k)
    for a, b in zip(res[1], fresh):
        assert torch.equal(a, b)


def test_layer_forward_t_zero():
    say("layer forward T = 0")
    lay = layer_for(synth.TINY)
    x = torch.empty((0, 256), dtype=torch.int16, device=DEV)
    lg = torch.empty((0, 8), dtype=torch.float32, device=DEV)
    ids, w, out = moeq.layer_forward(lay, x, lg, 2)
    assert out.shape == (0, 256) and ids.shape == (0, 2)


def test_layer_forward_graph_replays():
    """The fused path captured in a HIP graph: every replay (with eager work
    and synchronisations between replays, new inputs copied into the captured
    buffers) equals the eager call on the same inputs."""
    wl, T = CASES["nv_k8_t1"]
    say("layer forward graph")
    lay = layer_for(wl)
    _, _, x0, lg0 = inputs(wl, T, rep=0)
    x = x0.clone()
    lg = lg0.clone()
    ws = moeq.layer_workspace(lay, T, wl.k)
    ids = torch.empty((T, wl.k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, wl.k), dtype=torch.float32, device=DEV)
    out = torch.empty((T, wl.H), dtype=torch.float32, device=DEV)
    moeq.layer_forward(lay, x, lg, wl.k, out=out, ids=ids, w=w, ws=ws)   # warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moeq.layer_forward(lay, x, lg, wl.k, out=out, ids=ids, w=w, ws=ws)
    for rep in (1, 2, 1, 3):
        _, _, xr, lgr = inputs(wl, T, rep=rep)
        want = moeq.layer_forward(lay, xr, lgr, wl.k)
        torch.cuda.synchronize()
        x.copy_(xr)
        lg.copy_(lgr)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, want[0]) and torch.equal(w, want[1]), rep
        assert torch.equal(out, want[2]), rep


# moe_layer_forward_shared: fused three-launch form for decode batches with a
# BF16 shared expert; every other case runs moe_shared_ffn + moe_layer_forward
SHARED_CASES = {
    # fused: one and two tokens of top-8 (8 slots per wave), top-4 over
    # ragged H / I (4 slots per wave), small-codebook VQ routed experts
    # (codebooks in LDS beside the shared pass), BF16 routed experts at k = 6
    # (two slot groups per down workgroup: 512-thread SwiGLU blocks)
    "sf_nv_t1": (synth.small_workload("lfs_nv", E=32, k=8, H=384, I=256, T=2, cfg=196,
                                      shared=True), 1),
    "sf_nv_t2": (synth.small_workload("lfs_nv", E=32, k=8, H=384, I=256, T=2, cfg=196,
                                      shared=True), 2),
    "sf_nv_k4": (synth.small_workload("lfs_k4", E=16, k=4, H=272, I=80, T=4, cfg=197,
                                      shared=True), 4),
    "sf_vq8": (synth.small_workload("lfs_vq8", E=12, k=3, H=512, I=144, T=5, fmt="vq8",
                                    cfg=198, vq8_m=2, shared=True), 5),
    "sf_bf16_k6": (synth.small_workload("lfs_bf16", E=16, k=6, H=272, I=80, T=2, fmt="bf16",
                                        cfg=199, shared=True), 2),
    # not fused: 18 assignments; a rotated routed layer
    "sf_t9": (synth.small_workload("lfs_t9", E=8, k=2, H=256, I=128, T=9, cfg=179,
                                   shared=True), 9),
    "sf_rot": (synth.small_workload("lfs_rot", E=16, k=4, H=384, I=256, T=1, cfg=178, rot=True,
                                    shared=True), 1),
}


def two_calls(lay, sh, x, lgd, k):
    y_sh = moeq.shared_ffn(sh, x)
    return moeq.layer_forward(lay, x, lgd, k, y_shared=y_sh)


@pytest.mark.parametrize("name", list(SHARED_CASES))
def test_layer_forward_shared_parity(name):
    wl, T = SHARED_CASES[name]
    say("layer forward with shared layer", name, T)
    lay = layer_for(wl)
    sh = build_shared_layer(wl, DEV)
    x_bits, lg, x, lgd = inputs(wl, T)
    ids, w, out = moeq.layer_forward(lay, x, lgd, wl.k, shared=sh)
    ref_out, ref_ids, _, _ = oracle_out(wl, x_bits, lg, shared=shared_weights(wl))
    assert np.array_equal(to_np(ids), ref_ids)
    assert_rows_close(to_np(out), ref_out, name + " out")
    ids2, w2, out2 = two_calls(lay, sh, x, lgd, wl.k)
    assert torch.equal(ids, ids2) and torch.equal(w, w2)
    assert torch.equal(out, out2), name


def test_layer_forward_shared_other_format_falls_back():
    """A shared expert in NVFP4 takes the two calls (same bits)."""
    from bit_quantized_moe_route_amd.layers import build_layer
    wl, T = SHARED_CASES["sf_nv_t1"]
    say("layer forward with an NVFP4 shared layer")
    lay = layer_for(wl)
    sh = build_layer(1, wl.H, wl.I, np.array([moeq.FMT_NVFP4], np.uint8),
                     nvfp4_weights=lambda e, p: (synth.shared_weights_bf16(wl, p).astype(
                         np.uint32) << 16).view(np.float32), device=DEV, workers=1)
    _, _, x, lgd = inputs(wl, T)
    a = moeq.layer_forward(lay, x, lgd, wl.k, shared=sh)
    b = two_calls(lay, sh, x, lgd, wl.k)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_layer_forward_shared_graph_replays():
    """The three-launch form captured in a HIP graph: every replay (new inputs
    copied into the captured buffers, eager work between replays) equals the
    eager call on the same inputs."""
    wl, T = SHARED_CASES["sf_nv_t2"]
    say("layer forward with shared layer, graph")
    lay = layer_for(wl)
    sh = build_shared_layer(wl, DEV)
    _, _, x0, lg0 = inputs(wl, T, rep=0)
    x = x0.clone()
    lg = lg0.clone()
    ws = moeq.layer_workspace(lay, T, wl.k, shared=sh)
    ids = torch.empty((T, wl.k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, wl.k), dtype=torch.float32, device=DEV)
    out = torch.empty((T, wl.H), dtype=torch.float32, device=DEV)
    moeq.layer_forward(lay, x, lg, wl.k, out=out, ids=ids, w=w, ws=ws, shared=sh)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moeq.layer_forward(lay, x, lg, wl.k, out=out, ids=ids, w=w, ws=ws, shared=sh)
    for rep in (1, 2, 1, 3):
        _, _, xr, lgr = inputs(wl, T, rep=rep)
        want = moeq.layer_forward(lay, xr, lgr, wl.k, shared=sh)
        torch.cuda.synchronize()
        x.copy_(xr)
        lg.copy_(lgr)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, want[0]) and torch.equal(w, want[1]), rep
        assert torch.equal(out, want[2]), rep


def test_layer_forward_shared_t_zero():
    wl, _ = SHARED_CASES["sf_nv_t1"]
    say("layer forward with shared layer, T = 0")
    lay = layer_for(wl)
    sh = build_shared_layer(wl, DEV)
    x = torch.empty((0, wl.H), dtype=torch.int16, device=DEV)
    lg = torch.empty((0, wl.E), dtype=torch.float32, device=DEV)
    ids, w, out = moeq.layer_forward(lay, x, lg, wl.k, shared=sh)
    assert out.shape == (0, wl.H) and ids.shape == (0, wl.k)
