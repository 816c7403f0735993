"""GPU parity of nested two-level NVFP4 experts (MOE_FMT_NVFP4R).

A two-level record is an NVFP4 base plane followed by an NVFP4 residual
plane; in a nested layer the NVFP4 tier runs on the base planes of the same
records, so an expert moves between the tiers by its tag alone.  Checked
against the oracle (each tier's effective weights), and against a plain
NVFP4 layer of the same weights, which the base tier must equal bit for bit.
"""

import numpy as np
import pytest
import torch

import bit_quantized_moe_route_amd as moeq
import oracle
import synth
from tests.gpu_common import assert_rows_close, build_small_layer, say
from tests.oracle_runs import expert_weights

pytestmark = pytest.mark.gpu

DEV = "cuda"

NESTED = {
    # decode: seeded experts lifted; ragged H (17 row groups) and I; the
    # grouped-GEMM path with a ragged last token tile
    "nest_decode": synth.small_workload("nest_decode", E=12, k=3, H=256, I=128, T=21,
                                        fmt="nested", cfg=200, n_nvfp4=5),
    "nest_ragged": synth.small_workload("nest_ragged", E=16, k=4, H=272, I=80, T=37,
                                        fmt="nested", cfg=201, n_nvfp4=7),
    "nest_prefill": synth.small_workload("nest_prefill", E=8, k=2, H=256, I=128, T=260,
                                         fmt="nested", logits="zipf", zipf_s=1.1, cfg=202,
                                         n_nvfp4=3),
    # stored rotated (signs + Hadamard-128 on both sides): decode and prefill
    "nest_rot": synth.small_workload("nest_rot", E=12, k=3, H=256, I=128, T=21, fmt="nested",
                                     cfg=204, n_nvfp4=5, rot=True),
    "nest_rot_prefill": synth.small_workload("nest_rot_prefill", E=8, k=2, H=256, I=128,
                                             T=200, fmt="nested", cfg=205, n_nvfp4=4,
                                             rot=True),
}


def to_np(t):
    return t.detach().cpu().numpy()


def run(layer, wl, T, rep=0):
    x_bits = synth.activations(wl, T, rep=rep)
    lg = synth.logits(wl, T, rep=rep)
    r = moeq.forward(layer, torch.from_numpy(x_bits.view(np.int16)).to(DEV),
                     torch.from_numpy(lg).to(DEV), wl.k)
    torch.cuda.synchronize()
    return x_bits, lg, r


def oracle_check(wl, layer, x_bits, lg, r, label):
    tiers = layer.fmt_host.copy()
    Wc = {}

    def weights(e):
        if e not in Wc:
            Wc[e] = expert_weights(wl, e, int(tiers[e]))
        return Wc[e]
    out, ids, w, y = oracle.forward(x_bits, lg, wl.k, weights)
    assert np.array_equal(to_np(r["topk_ids"]), ids)
    assert_rows_close(to_np(r["out"]), out, label)


@pytest.mark.parametrize("name", list(NESTED))
def test_nested_forward_parity(name):
    wl = NESTED[name]
    T = wl.T[0]
    say("nested forward", name, T)
    layer = build_small_layer(wl, DEV)
    assert layer.alias == {moeq.FMT_NVFP4: moeq.FMT_NVFP4R}
    x_bits, lg, r = run(layer, wl, T)
    oracle_check(wl, layer, x_bits, lg, r, name)


def test_nested_dequant_is_base_plus_residual():
    wl = NESTED["nest_ragged"]
    say("nested dequant")
    layer = build_small_layer(wl, DEV)
    tm = synth.tier_map(wl)
    for e in (int(np.flatnonzero(tm == moeq.FMT_NVFP4R)[0]), int(np.flatnonzero(tm == 1)[0])):
        W = expert_weights(wl, e, int(tm[e]))
        for p in range(3):
            got = to_np(moeq.dequant_q(layer, e, p)).astype(np.float64)
            assert np.all(np.abs(got - W[p]) <= 2.0 ** -24 * np.abs(W[p])), (e, p)


@pytest.mark.parametrize("name", ["nest_decode", "nest_prefill"])
def test_base_tier_equals_plain_nvfp4_layer(name):
    """Every expert on the base tier of a nested layer: the same bits as a
    plain (compact) NVFP4 layer built from the same weights."""
    wl = NESTED[name]
    T = wl.T[0]
    say("nested base tier == NVFP4", name)
    nested = build_small_layer(wl, DEV)
    nested.set_tiers(np.full(wl.E, moeq.FMT_NVFP4, np.uint8))
    plain = build_small_layer(synth.small_workload(wl.name, wl.E, wl.k, wl.H, wl.I, T,
                                                   logits=wl.logits, cfg=wl.cfg,
                                                   zipf_s=wl.zipf_s), DEV)
    assert plain.alias == {} and set(plain.fmt_host.tolist()) == {moeq.FMT_NVFP4}
    _, _, a = run(nested, wl, T)
    _, _, b = run(plain, wl, T)
    assert torch.equal(a["out"], b["out"])


def test_tier_moves_and_residual_upload():
    """Experts move between the tiers by tag alone, and a residual plane
    written on its own (base bytes untouched) lifts an expert: a zero residual
    plane gives the base tier's bits, the real one the two-level weights."""
    wl = NESTED["nest_decode"]
    T = wl.T[0]
    say("nested tier moves")
    layer = build_small_layer(wl, DEV)
    maps = [synth.tier_map(wl), np.full(wl.E, moeq.FMT_NVFP4R, np.uint8),
            np.where(synth.tier_map(wl) == 1, moeq.FMT_NVFP4R, 1).astype(np.uint8)]
    for i, tm in enumerate(maps):
        layer.set_tiers(tm)
        x_bits, lg, r = run(layer, wl, T, rep=i)
        oracle_check(wl, layer, x_bits, lg, r, f"tiers {i}")
    # residual planes written on their own
    layer.set_tiers(np.full(wl.E, moeq.FMT_NVFP4, np.uint8))
    _, _, base = run(layer, wl, T, rep=5)
    n13 = moeq.record_bytes(moeq.FMT_NVFP4, 0, wl.H, wl.I)
    n2 = moeq.record_bytes(moeq.FMT_NVFP4, 1, wl.H, wl.I)
    for e in range(wl.E):
        layer.set_residual(e, np.zeros(n13, np.uint8), np.zeros(n2, np.uint8))
    layer.set_tiers(np.full(wl.E, moeq.FMT_NVFP4R, np.uint8))
    _, _, zero_res = run(layer, wl, T, rep=5)
    assert torch.equal(zero_res["out"], base["out"])
    for e in range(wl.E):
        parts = [moeq.quantize_nvfp4_residual(synth.nvfp4_source_weights(wl, e, p),
                                              synth.NVFP4R_SHIFT)[1] for p in range(3)]
        layer.set_residual(e, *moeq.pack_nvfp4_expert(*parts, wl.H, wl.I))
    x_bits, lg, r = run(layer, wl, T, rep=5)
    oracle_check(wl, layer, x_bits, lg, r, "residual planes uploaded")


def test_two_level_layer_fused_decode_path():
    """A layer of two-level experts only, through the one-call layer at
    decode sizes (the fused path): the step-by-step calls' bits and the
    oracle."""
    wl = synth.small_workload("nest_only", E=16, k=8, H=384, I=256, T=2, fmt="nested",
                              cfg=203, n_nvfp4=16)
    say("two-level fused decode")
    layer = build_small_layer(wl, DEV, resident_formats={moeq.FMT_NVFP4R})
    assert set(layer.fmt_host.tolist()) == {moeq.FMT_NVFP4R}
    for T in (1, 2):
        x_bits = synth.activations(wl, T)
        lg = synth.logits(wl, T)
        x = torch.from_numpy(x_bits.view(np.int16)).to(DEV)
        lgd = torch.from_numpy(lg).to(DEV)
        ids, w, out = moeq.layer_forward(layer, x, lgd, wl.k)
        r = moeq.forward(layer, x, lgd, wl.k)
        assert torch.equal(out, r["out"]) and torch.equal(ids, r["topk_ids"])
        oracle_check(wl, layer, x_bits, lg, r, f"two-level T={T}")
