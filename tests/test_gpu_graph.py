"""The forward captured in a HIP graph: every replay, with eager work and
synchronisations in between, equals the eager result bit for bit; and the
fused route + permute call equals the two separate calls bit for bit."""

import numpy as np
import pytest
import torch

import bit_quantized_moe_route_amd as moeq
import oracle
import synth
from tests.gpu_common import build_small_layer, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (32, 256, 8), (512, 256, 8), (700, 64, 8),
                                   (5, 1024, 16), (3, 4, 1), (4096, 256, 8), (300, 1024, 16),
                                   (8, 256, 8), (4, 1024, 16), (64, 16, 1), (9, 64, 7),
                                   (0, 8, 2), (65, 16, 1), (64, 256, 8), (65, 256, 8),
                                   (32, 1024, 16), (33, 1024, 16), (21, 600, 3)])
def test_route_permute_equals_separate_calls(T, E, k):
    say("route_permute", T, E, k)
    g = np.random.default_rng(T + E)
    lg = torch.from_numpy(g.random((T, E)).astype(np.float32)).to(DEV)
    if T >= 4:
        lg[3] = 0.5   # a token of tied logits: the tie rule picks ids 0 .. k-1
    fused = moeq.route_permute(lg, k)
    ids, w = moeq.route_topk(lg, k)
    perm = moeq.permute(ids, E)
    for a, b, nm in zip(fused, (ids, w) + tuple(perm),
                        ("ids", "w", "counts", "offsets", "perm_src", "inv_perm")):
        assert torch.equal(a, b), nm
    # and against the oracle
    lg_np = lg.cpu().numpy()
    oids, _ = oracle.route_topk(lg_np, k) if T else (np.zeros((0, k), np.int32), None)
    assert np.array_equal(fused[0].cpu().numpy(), oids)
    for a, b, nm in zip(fused[2:], oracle.permute(oids, E),
                        ("counts", "offsets", "perm_src", "inv_perm")):
        assert np.array_equal(a.cpu().numpy(), b), nm


def test_graph_replays_equal_eager():
    wl = synth.small_workload("graph_mixed", E=24, k=6, H=384, I=96, T=20, fmt="mixed",
                              logits="hot", cfg=111, n_nvfp4=9, n_hot=4, hot_share=0.6)
    say("graph replays", wl.name)
    layer = build_small_layer(wl, DEV)
    T, k = wl.T[0], wl.k
    lg = torch.from_numpy(synth.logits(wl, T)).to(DEV)
    x = torch.from_numpy(synth.activations(wl, T).view(np.int16)).to(DEV)
    bufs = dict(
        rp=(torch.empty((T, k), dtype=torch.int32, device=DEV),
            torch.empty((T, k), dtype=torch.float32, device=DEV),
            torch.empty(wl.E, dtype=torch.int32, device=DEV),
            torch.empty(wl.E + 1, dtype=torch.int32, device=DEV),
            torch.empty(T * k, dtype=torch.int32, device=DEV),
            torch.empty(T * k, dtype=torch.int32, device=DEV)),
        h=torch.empty((T * k, wl.I), dtype=torch.float16, device=DEV),
        y=torch.empty((T * k, wl.H), dtype=torch.float32, device=DEV),
        out=torch.empty((T, wl.H), dtype=torch.float32, device=DEV),
        ws=moeq.gateup_workspace(layer, T, k))

    def step():
        ids, w, counts, offsets, perm_src, inv_perm = moeq.route_permute(lg, k, wl.E, bufs["rp"])
        moeq.expert_gateup_q(layer, x, perm_src, offsets, k, bufs["h"], bufs["ws"])
        moeq.expert_down_q(layer, bufs["h"], offsets, k, bufs["y"])
        moeq.combine(bufs["y"], inv_perm, w, bufs["out"])

    step()
    torch.cuda.synchronize()
    eager = bufs["out"].clone()
    eager_y = bufs["y"].clone()
    ref = moeq.forward(layer, x, lg, k)["out"]
    assert torch.equal(eager, ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = torch.from_numpy(synth.logits(wl, T, rep=5)).to(DEV)
    for i in range(4):
        bufs["out"].zero_()
        bufs["y"].zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs["out"], eager), f"replay {i}"
        assert torch.equal(bufs["y"], eager_y), f"replay {i}"
        # eager work of the program between replays
        moeq.forward(layer, x, other, k)
        torch.cuda.synchronize()


@pytest.mark.parametrize("T", [16, 40])
def test_graph_with_shared_expert_on_side_stream(T):
    """The forward with a BF16 shared expert on the side stream (fork from and
    join into the capture stream), captured in a graph: every replay equals
    the eager single-stream result bit for bit."""
    wl = synth.small_workload("graph_shared", E=16, k=4, H=272, I=80, T=T, cfg=112, shared=True)
    say("graph shared", T)
    from tests.gpu_common import build_shared_layer
    layer = build_small_layer(wl, DEV)
    shared = build_shared_layer(wl, DEV)
    lg = torch.from_numpy(synth.logits(wl, T)).to(DEV)
    x = torch.from_numpy(synth.activations(wl, T).view(np.int16)).to(DEV)
    serial = moeq.forward(layer, x, lg, wl.k, shared=shared, overlap=False)
    torch.cuda.synchronize()
    over = moeq.forward(layer, x, lg, wl.k, shared=shared, overlap=True)
    torch.cuda.synchronize()
    for key in ("out", "y_shared", "y_perm"):
        assert torch.equal(serial[key], over[key]), key
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = moeq.forward(layer, x, lg, wl.k, shared=shared, overlap=True)
    other = torch.from_numpy(synth.logits(wl, T, rep=3)).to(DEV)
    for i in range(4):
        cap["out"].zero_()
        cap["y_shared"].zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cap["out"], serial["out"]), f"replay {i}"
        assert torch.equal(cap["y_shared"], serial["y_shared"]), f"replay {i}"
        moeq.forward(layer, x, other, wl.k, shared=shared, overlap=True)
        torch.cuda.synchronize()


@pytest.mark.parametrize("T,in2_block,I", [(2, 128, 128), (2, 512, 512)])
def test_graph_rotated_fused_layer(T, in2_block, I):
    """A rotated layer's fused small-batch forward (moe_layer_forward: four
    launches) captured in a graph: replays equal the eager call bit for bit,
    with the program's own calls on other inputs between the replays."""
    wl = synth.small_workload("graph_rot_fused", E=16, k=4, H=384, I=I, T=T, cfg=114, rot=True,
                              rot_in2=in2_block)
    say("graph rotated fused", in2_block)
    layer = build_small_layer(wl, DEV)
    lg = torch.from_numpy(synth.logits(wl, T)).to(DEV)
    x = torch.from_numpy(synth.activations(wl, T).view(np.int16)).to(DEV)
    ws = moeq.layer_workspace(layer, T, wl.k)
    ids, w, out = moeq.layer_forward(layer, x, lg, wl.k, ws=ws)
    eager = out.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _, _, cap = moeq.layer_forward(layer, x, lg, wl.k, ids=ids, w=w, ws=ws)
    other = torch.from_numpy(synth.logits(wl, T, rep=2)).to(DEV)
    for i in range(3):
        cap.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cap, eager), f"replay {i}"
        moeq.layer_forward(layer, x, other, wl.k, ws=ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("in2_block,I", [(128, 128), (512, 512)])
def test_graph_rotated_layer(in2_block, I):
    """A rotated layer's forward (three rotation launches around the GEMMs)
    captured in a graph: replays equal the eager result bit for bit (also with
    the wide down-input rotation)."""
    wl = synth.small_workload("graph_rot", E=16, k=4, H=256, I=I, T=24, cfg=113, rot=True,
                              rot_in2=in2_block)
    say("graph rotated", in2_block)
    layer = build_small_layer(wl, DEV)
    T = wl.T[0]
    lg = torch.from_numpy(synth.logits(wl, T)).to(DEV)
    x = torch.from_numpy(synth.activations(wl, T).view(np.int16)).to(DEV)
    eager = moeq.forward(layer, x, lg, wl.k)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = moeq.forward(layer, x, lg, wl.k)
    other = torch.from_numpy(synth.logits(wl, T, rep=2)).to(DEV)
    for i in range(3):
        cap["out"].zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cap["out"], eager["out"]), f"replay {i}"
        moeq.forward(layer, x, other, wl.k)
        torch.cuda.synchronize()
