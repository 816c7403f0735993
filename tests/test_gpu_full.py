"""GPU parity at the full GLM-5-class sizes (256 experts, top-8, H 6144,
I 2048) in the launch configurations the benchmark times: decode T = 1, 8,
32 (NVFP4), prefill T = 4096 with Zipf(1.1) routing (NVFP4), 2-bit VQ T = 8,
the small-codebook VQ layers (1 and 2 bits per weight) at T = 8 and the mixed
NVFP4/VQ layer at T = 8 and 32, and the decode layer held nested (two-level NVFP4
experts) at T = 8.

Routing and permutation are compared in full (bit-exact).  Expert outputs
are compared row by row against the oracle, all rows of each expert checked:
at T = 8 (NVFP4 decode, 2-bit VQ, mixed NVFP4/VQ) every expert the batch
touches, so each output row is compared too; at other sizes sampled experts
(the oracle encodes and decodes one NVFP4 expert's 37.7M weights in fp64 in
~15 s), and for T = 1 every expert of the token with its combined row.  For
the sampled batches the combine is checked through a property that holds at
any size: out[t] equals the fp64 weighted sum of the kernel's own y_perm
rows in ascending j.  The oracle's experts run in a process pool on the
host's cores."""

import numpy as np
import pytest
import torch

import bit_quantized_moe_route_amd as moeq
import oracle
import synth
from tests.gpu_common import W_TOL, assert_rows_close, build_small_layer, say
from tests.oracle_runs import expert_weights, pool_map

pytestmark = pytest.mark.gpu

DEV = "cuda"
_layers = {}


def layer(name):
    if name not in _layers:
        say("building full layer", name)
        _layers[name] = build_small_layer(synth.WORKLOADS[name], DEV)
    return _layers[name]


def to_np(t):
    return t.detach().cpu().numpy()


def run_forward(wl, lay, T, rep=0):
    x_bits = synth.activations(wl, T, rep=rep)
    lg = synth.logits(wl, T, rep=rep)
    r = moeq.forward(lay, torch.from_numpy(x_bits.view(np.int16)).to(DEV),
                     torch.from_numpy(lg).to(DEV), wl.k)
    torch.cuda.synchronize()
    return x_bits, lg, r


def check_routing(wl, lg, r):
    ids, w = oracle.route_topk(lg, wl.k)
    assert np.array_equal(to_np(r["topk_ids"]), ids)
    assert np.max(np.abs(to_np(r["topk_w"]).astype(np.float64) - w)) <= W_TOL
    counts, offsets, perm_src, inv_perm = oracle.permute(ids, wl.E)
    for key, want in (("counts", counts), ("offsets", offsets), ("perm_src", perm_src),
                      ("inv_perm", inv_perm)):
        assert np.array_equal(to_np(r[key]), want), key
    return ids, w, offsets, perm_src


def check_experts(wl, x_bits, r, ids, offsets, perm_src, experts, fmt_host, workers=None):
    """All rows of each given expert: GPU y_perm vs the oracle FFN."""
    y_perm = to_np(r["y_perm"])
    jobs, spans = [], []
    for e in experts:
        a, b = int(offsets[e]), int(offsets[e + 1])
        toks = perm_src[a:b] // wl.k
        jobs.append((wl.name, int(e), x_bits[toks], int(fmt_host[e])))
        spans.append((a, b))
    refs = pool_map(jobs, workers=workers)
    worst = 0.0
    for (a, b), ref, e in zip(spans, refs, experts):
        worst = max(worst, assert_rows_close(y_perm[a:b], ref, f"{wl.name} expert {e}"))
    return worst


def check_combine_property(wl, r):
    y = to_np(r["y_perm"]).astype(np.float64)
    inv = to_np(r["inv_perm"])
    w = to_np(r["topk_w"]).astype(np.float64)
    T = w.shape[0]
    ref = np.zeros((T, y.shape[1]))
    for j in range(wl.k):
        ref += w[:, j, None] * y[inv.reshape(T, wl.k)[:, j]]
    assert_rows_close(to_np(r["out"]), ref, "combine property", tol=1e-5)


def check_layer_forward_bits(wl, lay, x_bits, lg, r):
    """The one-call layer (fused for small batches; for a rotated layer the
    combine rotating the down outputs back) gives the step-by-step calls'
    bits."""
    ids, w, out = moeq.layer_forward(lay, torch.from_numpy(x_bits.view(np.int16)).to(DEV),
                                     torch.from_numpy(lg).to(DEV), wl.k)
    torch.cuda.synchronize()
    assert torch.equal(ids, r["topk_ids"]) and torch.equal(w, r["topk_w"])
    assert torch.equal(out, r["out"])


def check_every_expert(wl, x_bits, lg, r, ids, w, offsets, perm_src, fmt_host):
    """Every expert the batch touches: all its y_perm rows against the
    oracle FFN, then every output row against the oracle's combine of the
    oracle's rows."""
    act = [int(e) for e in np.nonzero(np.diff(offsets) > 0)[0]]
    say(f"{wl.name}: all {len(act)} touched experts against the oracle")
    jobs = []
    for e in act:
        a, b = int(offsets[e]), int(offsets[e + 1])
        jobs.append((wl.name, e, x_bits[perm_src[a:b] // wl.k], int(fmt_host[e])))
    refs = pool_map(jobs, workers=16)
    y_perm = to_np(r["y_perm"])
    T = ids.shape[0]
    y = np.zeros((T, wl.k, wl.H))
    worst = 0.0
    for e, ref in zip(act, refs):
        a, b = int(offsets[e]), int(offsets[e + 1])
        worst = max(worst, assert_rows_close(y_perm[a:b], ref, f"{wl.name} expert {e}"))
        for i, src in enumerate(perm_src[a:b]):
            y[src // wl.k, src % wl.k] = ref[i]
    assert_rows_close(to_np(r["out"]), oracle.combine(y, w), f"{wl.name} out rows")
    return worst


def pick(offsets, fmt_host=None, fmt=None, n=2, seed=0):
    counts = np.diff(offsets)
    act = np.nonzero(counts > 0)[0]
    if fmt is not None:
        act = act[fmt_host[act] == fmt]
    rs = np.random.default_rng(seed)
    # the busiest expert plus random others
    busiest = act[np.argmax(counts[act])]
    others = rs.choice(act[act != busiest], size=min(n - 1, len(act) - 1), replace=False)
    return [int(busiest)] + [int(e) for e in others]


# ------------------------------------------------------------------ decode

@pytest.mark.timeout(900)
def test_decode_T1_full_forward():
    wl = synth.DECODE
    say("decode T=1 full")
    lay = layer("decode")
    x_bits, lg, r = run_forward(wl, lay, 1)
    ids, w, offsets, perm_src = check_routing(wl, lg, r)
    # every expert of the token: each y_perm row and the combined row
    jobs = [(wl.name, int(e), x_bits, 1) for e in ids[0]]
    y = np.zeros((1, wl.k, wl.H))
    y_perm = to_np(r["y_perm"])
    for j, ref in enumerate(pool_map(jobs)):
        y[0, j] = ref[0]
        row = int(to_np(r["inv_perm"])[j])
        assert_rows_close(y_perm[row:row + 1], ref, f"decode T=1 expert {ids[0, j]}")
    out = oracle.combine(y, w)
    assert_rows_close(to_np(r["out"]), out, "decode T=1 out")
    # the one-call layer (fused at this size): the same routing, the oracle's
    # row, and the step-by-step calls' bits
    x = torch.from_numpy(x_bits.view(np.int16)).to(DEV)
    f_ids, f_w, f_out = moeq.layer_forward(lay, x, torch.from_numpy(lg).to(DEV), wl.k)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(f_ids), ids)
    assert_rows_close(to_np(f_out), out, "decode T=1 layer_forward out")
    assert torch.equal(f_w, r["topk_w"]) and torch.equal(f_out, r["out"])


@pytest.mark.timeout(900)
def test_decode_T2_layer_forward_full():
    """Two tokens through the fused one-call layer (16 assignments): routing
    bit-exact, the step-by-step calls' bits, and token 1's row against the
    oracle (all 8 of its experts)."""
    wl = synth.DECODE
    say("decode T=2 layer_forward full")
    lay = layer("decode")
    x_bits, lg, r = run_forward(wl, lay, 2, rep=3)
    ids, w, offsets, perm_src = check_routing(wl, lg, r)
    x = torch.from_numpy(x_bits.view(np.int16)).to(DEV)
    f_ids, f_w, f_out = moeq.layer_forward(lay, x, torch.from_numpy(lg).to(DEV), wl.k)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(f_ids), ids)
    assert torch.equal(f_w, r["topk_w"]) and torch.equal(f_out, r["out"])
    y = np.zeros((1, wl.k, wl.H))
    for j, ref in enumerate(pool_map([(wl.name, int(e), x_bits[1:2], 1) for e in ids[1]])):
        y[0, j] = ref[0]
    assert_rows_close(to_np(f_out)[1:2], oracle.combine(y, w[1:2]), "decode T=2 token 1 out")


@pytest.mark.timeout(900)
def test_decode_T8_every_expert():
    """Decode T = 8: every touched expert's rows and every output row."""
    wl = synth.DECODE
    say("decode full T=8, every expert")
    lay = layer("decode")
    x_bits, lg, r = run_forward(wl, lay, 8)
    ids, w, offsets, perm_src = check_routing(wl, lg, r)
    check_every_expert(wl, x_bits, lg, r, ids, w, offsets, perm_src, synth.tier_map(wl))
    check_layer_forward_bits(wl, lay, x_bits, lg, r)


@pytest.mark.timeout(900)
def test_decode_T32_full_sampled():
    wl = synth.DECODE
    T = 32
    say("decode full", T)
    lay = layer("decode")
    x_bits, lg, r = run_forward(wl, lay, T)
    ids, w, offsets, perm_src = check_routing(wl, lg, r)
    experts = pick(offsets, n=4, seed=T)
    check_experts(wl, x_bits, r, ids, offsets, perm_src, experts, synth.tier_map(wl))
    check_combine_property(wl, r)
    check_layer_forward_bits(wl, lay, x_bits, lg, r)


@pytest.mark.timeout(900)
def test_dequant_full_sampled():
    wl = synth.DECODE
    say("dequant full")
    lay = layer("decode")
    for e in (0, 131, 255):
        W = expert_weights(wl, e)
        for p in range(3):
            assert np.array_equal(to_np(moeq.dequant_q(lay, e, p)).astype(np.float64), W[p]), (e, p)


@pytest.mark.timeout(900)
def test_decode_deterministic_full():
    wl = synth.DECODE
    say("determinism full T=32")
    lay = layer("decode")
    _, _, a = run_forward(wl, lay, 32, rep=3)
    _, _, b = run_forward(wl, lay, 32, rep=3)
    for key in a:
        assert torch.equal(a[key], b[key]), key


# ------------------------------------------------------------------ prefill

@pytest.mark.timeout(900)
def test_prefill_full_sampled():
    wl = synth.PREFILL
    T = 4096
    say("prefill full", T)
    lay = layer("decode")                   # the same NVFP4 layer
    x_bits, lg, r = run_forward(wl, lay, T)
    ids, w, offsets, perm_src = check_routing(wl, lg, r)
    counts = np.diff(offsets)
    assert counts.max() > 128 * 8 and counts.min() >= 0   # several 128-row tiles for hot experts
    experts = pick(offsets, n=2, seed=1)
    # the smallest active expert as well (a partly filled tile)
    act = np.nonzero(counts > 0)[0]
    experts.append(int(act[np.argmin(counts[act])]))
    check_experts(wl, x_bits, r, ids, offsets, perm_src, experts, synth.tier_map(wl))
    check_combine_property(wl, r)
    check_layer_forward_bits(wl, lay, x_bits, lg, r)


# ------------------------------------------------------------------ VQ and mixed

@pytest.mark.timeout(900)
def test_vq_T8_every_expert():
    """2-bit VQ at T = 8: every touched expert's rows and every output row."""
    wl = synth.VQ
    say("vq full T=8, every expert")
    lay = layer("vq")
    x_bits, lg, r = run_forward(wl, lay, 8)
    ids, w, offsets, perm_src = check_routing(wl, lg, r)
    check_every_expert(wl, x_bits, lg, r, ids, w, offsets, perm_src, synth.tier_map(wl))
    experts = pick(offsets, n=2, seed=2)
    for e in experts[:2]:
        W = expert_weights(wl, e)
        for p in range(3):
            assert np.array_equal(to_np(moeq.dequant_q(lay, e, p)).astype(np.float64), W[p]), (e, p)


@pytest.mark.timeout(900)
def test_vqmix_T8_every_expert():
    """Small-codebook VQ experts at mixed rates (131 / 55 / 70 experts at 1 /
    2 / 3 bits per weight) at the full layer size, T = 8: every touched
    expert's rows and every output row; the dequant hook on one expert of
    each rate."""
    wl = synth.VQMIX
    say("vqmix full T=8, every expert")
    lay = layer("vqmix")
    tm = synth.tier_map(wl)
    x_bits, lg, r = run_forward(wl, lay, 8)
    ids, w, offsets, perm_src = check_routing(wl, lg, r)
    check_every_expert(wl, x_bits, lg, r, ids, w, offsets, perm_src, tm)
    for tag in (synth.FMT_VQ8_M1, synth.FMT_VQ8_M2, synth.FMT_VQ8_M3):
        e = int(np.flatnonzero(tm == tag)[0])
        W = expert_weights(wl, e)
        for p in range(3):
            got = to_np(moeq.dequant_q(lay, e, p)).astype(np.float64)
            assert np.all(np.abs(got - W[p]) <= 2.0 ** -22 * np.abs(W[p])), (e, p)


@pytest.mark.parametrize("name", ["vq1", "vq2x8", "vq3x8"])
def test_vq8_full_sampled(name):
    """Small-codebook VQ (1 and 2 bits per weight) at the full layer size, T = 8."""
    wl = synth.WORKLOADS[name]
    say("vq8 full T=8", name)
    lay = layer(name)
    x_bits, lg, r = run_forward(wl, lay, 8)
    ids, w, offsets, perm_src = check_routing(wl, lg, r)
    experts = pick(offsets, n=4, seed=3)
    check_experts(wl, x_bits, r, ids, offsets, perm_src, experts, synth.tier_map(wl))
    check_combine_property(wl, r)
    for e in experts[:2]:
        W = expert_weights(wl, e)
        for p in range(3):
            got = to_np(moeq.dequant_q(lay, e, p)).astype(np.float64)
            if wl.vq8_m == 1:
                assert np.array_equal(got, W[p]), (e, p)
            else:
                assert np.all(np.abs(got - W[p]) <= 2.0 ** -22 * np.abs(W[p])), (e, p)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [8, 32])
def test_mixed_full(T):
    """The mixed NVFP4/VQ layer: at T = 8 every touched expert and every
    output row, at T = 32 sampled experts of each format."""
    wl = synth.MIXED
    say("mixed full", T)
    lay = layer("mixed")
    fmt_host = synth.tier_map(wl)
    x_bits, lg, r = run_forward(wl, lay, T)
    ids, w, offsets, perm_src = check_routing(wl, lg, r)
    if T == 8:
        check_every_expert(wl, x_bits, lg, r, ids, w, offsets, perm_src, fmt_host)
    else:
        experts = (pick(offsets, fmt_host, synth.FMT_NVFP4, n=2, seed=T)
                   + pick(offsets, fmt_host, synth.FMT_VQ, n=2, seed=T + 1))
        check_experts(wl, x_bits, r, ids, offsets, perm_src, experts, fmt_host)
        check_combine_property(wl, r)
    check_layer_forward_bits(wl, lay, x_bits, lg, r)
    # the hot set takes about 60% of the assignments
    hot = synth.hot_experts(wl)
    share = np.isin(ids, hot).mean()
    say(f"mixed T={T}: hot share {share:.3f}, hot NVFP4 experts "
        f"{int((fmt_host[hot] == synth.FMT_NVFP4).sum())}/{len(hot)}")
    assert 0.35 < share < 0.85


@pytest.mark.timeout(900)
def test_nested_full_sampled():
    """The decode layer's experts held nested (two-level records resident,
    the 20 hot experts lifted to the two-level tier) at T = 8: routing, the
    rows of a two-level and a base-tier expert against the oracle, the
    combine property."""
    wl = synth.NESTED
    T = 8
    say("nested full", T)
    lay = layer("nested")
    fmt_host = synth.tier_map(wl)
    assert int((fmt_host == synth.FMT_NVFP4R).sum()) == wl.n_hot
    x_bits, lg, r = run_forward(wl, lay, T)
    ids, w, offsets, perm_src = check_routing(wl, lg, r)
    experts = (pick(offsets, fmt_host, synth.FMT_NVFP4R, n=1, seed=T)
               + pick(offsets, fmt_host, synth.FMT_NVFP4, n=1, seed=T + 1))
    check_experts(wl, x_bits, r, ids, offsets, perm_src, experts, fmt_host)
    check_combine_property(wl, r)
    check_layer_forward_bits(wl, lay, x_bits, lg, r)


# ------------------------------------------------------------------ shared expert

_shared = {}


def shared_layer(wl):
    if wl.name not in _shared:
        from tests.gpu_common import build_shared_layer
        say("building full shared expert", wl.name)
        _shared[wl.name] = build_shared_layer(wl, DEV)
    return _shared[wl.name]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [1, 2])
def test_layer_forward_shared_full(T):
    """The whole decode layer with its BF16 shared expert in one call
    (moe_layer_forward_shared: three launches at these sizes), as the
    benchmark times it: the bits of moe_shared_ffn + moe_layer_forward on the
    same batch, routing against the oracle, and the shared output of token 0
    against the oracle's shared FFN (out minus the fixed-order routed sum)."""
    from tests.oracle_runs import shared_weights
    wl = synth.DECODE_SHARED
    say("layer_forward_shared full", T)
    lay = layer("decode")
    sh = shared_layer(wl)
    x_bits = synth.activations(wl, T, rep=5)
    lg = synth.logits(wl, T, rep=5)
    x = torch.from_numpy(x_bits.view(np.int16)).to(DEV)
    lgd = torch.from_numpy(lg).to(DEV)
    ids, w, out = moeq.layer_forward(lay, x, lgd, wl.k, shared=sh)
    y_sh = moeq.shared_ffn(sh, x)
    ids2, w2, out2 = moeq.layer_forward(lay, x, lgd, wl.k, y_shared=y_sh)
    routed = moeq.layer_forward(lay, x, lgd, wl.k)[2]
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w, w2) and torch.equal(out, out2)
    ref_ids, _ = oracle.route_topk(lg, wl.k)
    assert np.array_equal(to_np(ids), ref_ids)
    # out - routed sum is y_shared rounded once more: compare y_shared itself
    ref = oracle.expert_ffn(x_bits[:1], *shared_weights(wl))
    assert_rows_close(to_np(y_sh)[:1], ref, "shared FFN of token 0")
    assert torch.equal(out, routed + y_sh)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,T", [("decode_shared", 1), ("decode_shared", 32),
                                    ("prefill_shared", 4096)])
def test_shared_expert_full(name, T):
    """The BF16 shared expert (H 6144, I 2048) beside the full NVFP4 layer, in
    the benchmark's configurations: its output rows against the oracle (all
    rows in decode, a sample spanning every 128-token tile in prefill), and the
    combined output through the combine property plus y_shared."""
    from tests.oracle_runs import shared_weights
    wl = synth.WORKLOADS[name]
    say("shared full", name, T)
    lay = layer("decode")                   # the same routed NVFP4 layer
    sh = shared_layer(wl)
    x_bits = synth.activations(wl, T)
    lg = synth.logits(wl, T)
    r = moeq.forward(lay, torch.from_numpy(x_bits.view(np.int16)).to(DEV),
                     torch.from_numpy(lg).to(DEV), wl.k, shared=sh)
    torch.cuda.synchronize()
    check_routing(wl, lg, r)
    # decode: every row; prefill: one row of every 128-token tile, and the last
    rows = (np.arange(T) if T <= 64 else
            np.array([128 * i + (37 * i) % 128 for i in range(T // 128)] + [T - 1]))
    Ws = shared_weights(wl)
    ref = oracle.expert_ffn(x_bits[rows], *Ws)
    assert_rows_close(to_np(r["y_shared"])[rows], ref, f"{name} y_shared")
    # out = the routed combine (fixed order) + y_shared
    y = to_np(r["y_perm"]).astype(np.float64)
    inv = to_np(r["inv_perm"]).reshape(T, wl.k)
    w = to_np(r["topk_w"]).astype(np.float64)
    want = to_np(r["y_shared"]).astype(np.float64)
    for j in range(wl.k):
        want = want + w[:, j, None] * y[inv[:, j]]
    assert_rows_close(to_np(r["out"]), want, f"{name} out", tol=1e-5)


# ------------------------------------------------------------------ rotated storage

@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,T", [("decode_rot", 1), ("decode_rot", 32), ("decode_rot512", 1),
                                    ("decode_rot512", 32)])
def test_rotated_full_sampled(name, T):
    """The decode layer stored rotated (signs + Hadamard-128 on both sides of
    every matrix, the NVFP4 codes those of the rotated matrices; or the wide
    512-block on the down projection's input side): sampled experts' rows
    against the oracle's R_out^T Q(W_rot) R_in, the combine through its
    property.  Both workloads store the same matrices and signs, so the wide
    one reuses the layer with its down-input block switched."""
    import copy
    wl = synth.WORKLOADS[name]
    say("rotated full", name, T)
    lay = layer("decode_rot")
    if wl.rot_in2 != lay.rot_in2_block:
        lay = copy.copy(lay)
        lay.rot_in2_block = wl.rot_in2
        lay._c = None
    x_bits, lg, r = run_forward(wl, lay, T)
    ids, w, offsets, perm_src = check_routing(wl, lg, r)
    experts = pick(offsets, n=2, seed=T + 40)
    check_experts(wl, x_bits, r, ids, offsets, perm_src, experts, synth.tier_map(wl))
    check_combine_property(wl, r)
    check_layer_forward_bits(wl, lay, x_bits, lg, r)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode_rot", "decode_rot512"])
def test_rotated_prefill_full_sampled(name):
    """The rotated decode layer (and its wide down-input form) at T = 4096
    with the prefill routing: x rotated per assignment, the grouped GEMM's raw
    products, the middle rotation, and the combine rotating the down outputs
    back.  Sampled experts' rows against the oracle (the busiest, a random one
    and the least busy), the combine through its property."""
    import copy
    import dataclasses
    base = synth.WORKLOADS[name]
    # the prefill batch's seed slot and routing; the layer's weights and
    # signs (looked up by name for the oracle) are unchanged
    wl = dataclasses.replace(base, cfg=2, T=(4096,), logits="zipf", zipf_s=1.1)
    say("rotated prefill full", name)
    lay = layer("decode_rot")
    if base.rot_in2 != lay.rot_in2_block:
        lay = copy.copy(lay)
        lay.rot_in2_block = base.rot_in2
        lay._c = None
    x_bits, lg, r = run_forward(wl, lay, 4096)
    ids, w, offsets, perm_src = check_routing(wl, lg, r)
    counts = np.diff(offsets)
    experts = pick(offsets, n=2, seed=7)
    act = np.nonzero(counts > 0)[0]
    experts.append(int(act[np.argmin(counts[act])]))
    check_experts(wl, x_bits, r, ids, offsets, perm_src, experts, synth.tier_map(wl))
    check_combine_property(wl, r)
    check_layer_forward_bits(wl, lay, x_bits, lg, r)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["vq2x8", "vq"])
def test_vq_prefill_full_sampled(name):
    """VQ layers (2 x 8-bit codes with LDS codebooks; 16-bit codes from L2) at
    T = 4096 with the prefill routing: the grouped-GEMM path."""
    import dataclasses
    base = synth.WORKLOADS[name]
    wl = dataclasses.replace(base, cfg=2, T=(4096,), logits="zipf", zipf_s=1.1)
    say("vq prefill full", name)
    lay = layer(name)
    x_bits, lg, r = run_forward(wl, lay, 4096)
    ids, w, offsets, perm_src = check_routing(wl, lg, r)
    counts = np.diff(offsets)
    experts = pick(offsets, n=2, seed=5)
    act = np.nonzero(counts > 0)[0]
    experts.append(int(act[np.argmin(counts[act])]))
    check_experts(wl, x_bits, r, ids, offsets, perm_src, experts, synth.tier_map(wl))
    check_combine_property(wl, r)
