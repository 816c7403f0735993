"""moe_layer_forward_static, the entry point that allocates nothing (its
workspace is the library's own per-GPU device array), called through the C
ABI and compared with moe_layer_forward on the same inputs: the same bits,
on two calls in a row with the second batch smaller (the array keeps the
first call's contents), at a small ragged layer and at the GLM-5-class
hidden and intermediate sizes near the array's limit; a batch beyond the
limit is refused before any launch; replays of a captured graph."""

import ctypes

import numpy as np
import pytest
import torch

import bit_quantized_moe_route_amd as moeq
import synth
from tests.gpu_common import build_small_layer, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _inputs(wl, T, rep):
    x = torch.from_numpy(synth.activations(wl, T, rep=rep).view(np.int16)).to(DEV)
    lg = torch.from_numpy(synth.logits(wl, T, rep=rep)).to(DEV)
    return x, lg


def _static(layer, x, lg, k, ids, w, out):
    """The C call itself (no binding logic in between)."""
    L = moeq.lib()
    return L.moe_layer_forward_static(ctypes.byref(layer.c()), moeq._dptr(x), moeq._dptr(lg),
                                      x.shape[0], k, None, moeq._dptr(ids), moeq._dptr(w),
                                      moeq._dptr(out), moeq._stream(x.device))


def _check_calls(wl, layer, sizes):
    k = wl.k
    for i, T in enumerate(sizes):
        say("static layer forward", wl.name, "T", T)
        x, lg = _inputs(wl, T, rep=10 + i)
        ref_ids, ref_w, ref_out = moeq.layer_forward(layer, x, lg, k)
        ids = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
        w = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
        out = torch.full((T, wl.H), float("nan"), dtype=torch.float32, device=DEV)
        assert _static(layer, x, lg, k, ids, w, out) == moeq.MOE_OK, moeq.lib().moe_last_error()
        torch.cuda.synchronize()
        assert torch.equal(ids, ref_ids), T
        assert torch.equal(w, ref_w), T
        assert torch.equal(out, ref_out), T


def test_static_matches_layer_forward_small():
    """A ragged 16-expert layer: T = 37 (route, permute, expert FFN and
    combine kernels), then T = 3 (the fused two-launch path), then T = 37
    again."""
    wl = synth.small_workload("noalloc_small", E=16, k=4, H=272, I=80, T=37, cfg=190)
    _check_calls(wl, build_small_layer(wl, DEV), [37, 3, 37])


def test_static_matches_layer_forward_full_width():
    """H 6144, I 2048, k 8 (16 experts): the largest batch the array holds,
    then a smaller one (T = 8), then one token (fused path); a batch beyond
    the limit is refused with MOE_EWORKSPACE and launches nothing."""
    wl = synth.small_workload("noalloc_wide", E=16, k=8, H=6144, I=2048, T=8, cfg=191)
    layer = build_small_layer(wl, DEV)
    L = moeq.lib()
    tmax = 1
    while L.moe_layer_forward_workspace_bytes(ctypes.byref(layer.c()), tmax + 1,
                                              wl.k) <= moeq.STATIC_WS_BYTES:
        tmax += 1
    assert tmax >= 127
    _check_calls(wl, layer, [tmax, 8, 1])
    T = tmax + 1
    x, lg = _inputs(wl, T, rep=3)
    ids = torch.full((T, wl.k), -7, dtype=torch.int32, device=DEV)
    w = torch.zeros((T, wl.k), dtype=torch.float32, device=DEV)
    out = torch.zeros((T, wl.H), dtype=torch.float32, device=DEV)
    assert _static(layer, x, lg, wl.k, ids, w, out) == moeq.MOE_EWORKSPACE
    assert b"static workspace" in L.moe_last_error()
    torch.cuda.synchronize()
    assert int((ids != -7).sum()) == 0 and float(out.abs().sum()) == 0.0


def test_static_in_a_captured_graph():
    """Captured in a HIP graph (after a first eager call on the device): every
    replay, with eager work and synchronisations between replays, gives the
    bits of the eager moe_layer_forward."""
    wl = synth.small_workload("noalloc_graph", E=16, k=4, H=272, I=80, T=9, cfg=192)
    layer = build_small_layer(wl, DEV)
    T = 9
    x, lg = _inputs(wl, T, rep=0)
    ref_ids, ref_w, ref_out = moeq.layer_forward(layer, x, lg, wl.k)
    ids = torch.empty((T, wl.k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, wl.k), dtype=torch.float32, device=DEV)
    out = torch.empty((T, wl.H), dtype=torch.float32, device=DEV)
    assert _static(layer, x, lg, wl.k, ids, w, out) == moeq.MOE_OK
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rc = _static(layer, x, lg, wl.k, ids, w, out)
    assert rc == moeq.MOE_OK
    for rep in range(4):
        out.fill_(float("nan"))
        ids.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, ref_ids) and torch.equal(w, ref_w) and torch.equal(out, ref_out), rep
        # eager work on the same array between replays
        moeq.layer_forward_static(layer, *_inputs(wl, 5, rep=rep + 1), wl.k)
        torch.cuda.synchronize()
