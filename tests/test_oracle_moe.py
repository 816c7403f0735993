"""Pins of the oracle's routing, permutation, expert FFN and combine: brute
force on tiny layers, closed forms, special cases and library routines.
CPU only."""

import itertools

import numpy as np
import pytest
import torch

import oracle
import synth


# ---------------------------------------------------------------- route

def test_route_brute_force_sorted():
    rs = np.random.default_rng(0)
    for E, k in [(8, 2), (16, 5), (64, 8), (7, 7)]:
        lg = rs.standard_normal((13, E)).astype(np.float32)
        # quantize a few logits so ties happen
        lg[::3] = np.round(lg[::3] * 2) / 2
        ids, w = oracle.route_topk(lg, k)
        for t in range(lg.shape[0]):
            order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))
            assert list(ids[t]) == order[:k]


def test_route_ties_lower_id_wins():
    lg = np.zeros((1, 10), np.float32)
    ids, w = oracle.route_topk(lg, 4)
    assert list(ids[0]) == [0, 1, 2, 3]
    assert np.allclose(w[0], 0.25, atol=0, rtol=1e-15)
    lg = np.array([[0.5, 1.0, 0.5, 2.0, 0.5, 0.5]], np.float32)
    ids, _ = oracle.route_topk(lg, 3)
    assert list(ids[0]) == [3, 1, 0]        # three-way tie for third place: lowest id
    lg = np.array([[-0.0, 0.0, -1.0, 0.0]], np.float32)
    ids, _ = oracle.route_topk(lg, 2)
    assert list(ids[0]) == [0, 1]           # -0.0 == +0.0


def test_route_weights_are_softmax_over_chosen():
    rs = np.random.default_rng(1)
    lg = rs.uniform(-4, 4, (50, 32)).astype(np.float32)
    ids, w = oracle.route_topk(lg, 6)
    sel = torch.from_numpy(np.take_along_axis(lg, ids.astype(np.int64), 1).astype(np.float64))
    ref = torch.softmax(sel, dim=1).numpy()
    assert np.max(np.abs(ref - w)) < 1e-15
    assert np.max(np.abs(w.sum(1) - 1)) < 1e-15
    # weights are non-increasing along the rank
    assert np.all(np.diff(w, axis=1) <= 0)


def test_route_k_equals_E_and_k1():
    lg = np.array([[3.0, -1.0, 2.0]], np.float32)
    ids, w = oracle.route_topk(lg, 3)
    assert list(ids[0]) == [0, 2, 1]
    ids, w = oracle.route_topk(lg, 1)
    assert list(ids[0]) == [0] and w[0, 0] == 1.0


def test_route_rejects_nan_and_bad_k():
    with pytest.raises(ValueError):
        oracle.route_topk(np.array([[np.nan, 1.0]], np.float32), 1)
    with pytest.raises(ValueError):
        oracle.route_topk(np.zeros((1, 4), np.float32), 5)


# ---------------------------------------------------------------- permute

def test_permute_matches_stable_argsort_and_invariants():
    rs = np.random.default_rng(2)
    for T, E, k in [(4, 8, 2), (37, 16, 3), (200, 256, 8), (0, 8, 2)]:
        ids = np.stack([rs.choice(E, size=k, replace=False) for _ in range(T)]) \
            if T else np.zeros((0, k), np.int64)
        counts, offsets, perm_src, inv_perm = oracle.permute(ids, E)
        flat = ids.reshape(-1)
        assert counts.sum() == T * k and offsets[E] == T * k and offsets[0] == 0
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert np.array_equal(np.diff(offsets), counts)
        assert np.array_equal(perm_src, np.argsort(flat, kind="stable"))
        assert np.array_equal(np.sort(perm_src), np.arange(T * k))
        assert np.array_equal(inv_perm[perm_src], np.arange(T * k))
        assert np.all(np.diff(flat[perm_src]) >= 0)


def test_permute_handworked():
    ids = np.array([[2, 0], [0, 1], [2, 1]])
    counts, offsets, perm_src, inv_perm = oracle.permute(ids, 4)
    # a: 0->e2 1->e0 2->e0 3->e1 4->e2 5->e1
    assert list(counts) == [2, 2, 2, 0]
    assert list(offsets) == [0, 2, 4, 6, 6]
    assert list(perm_src) == [1, 2, 3, 5, 0, 4]
    assert list(inv_perm) == [4, 0, 1, 2, 5, 3]


# ---------------------------------------------------------------- FFN / combine

def test_ffn_one_hot_input_picks_columns():
    """x = e_i: g = W_gate[:, i], u = W_up[:, i], y = W_down (silu(g) u).
    H != I so a transposed operand cannot pass."""
    rs = np.random.default_rng(3)
    H, I = 12, 5
    wg, wu = rs.standard_normal((I, H)), rs.standard_normal((I, H))
    wd = rs.standard_normal((H, I))
    for i in range(H):
        x = np.zeros((1, H))
        x[0, i] = 1.0
        y = oracle.expert_ffn(x, wg, wu, wd)
        g, u = wg[:, i], wu[:, i]
        h = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u
        want = np.zeros(H)
        for o in range(H):
            want[o] = sum(wd[o, c] * h[c] for c in range(I))
        assert np.allclose(y[0], want, rtol=1e-13, atol=1e-15)


def test_ffn_closed_form_constant_weights():
    """All weights = s: g = u = s*sum(x), h = silu(g)*g, y_o = s*I*h."""
    H, I, s = 32, 16, 0.0078125
    rs = np.random.default_rng(4)
    x = rs.standard_normal((3, H))
    W13 = np.full((I, H), s)
    W2 = np.full((H, I), s)
    y = oracle.expert_ffn(x, W13, W13, W2)
    g = s * x.sum(1)
    h = g * g / (1 + np.exp(-g))
    assert np.allclose(y, (s * I * h)[:, None] * np.ones((1, H)), rtol=1e-13)


def test_ffn_zero_weights_give_exact_zero():
    x = np.ones((2, 16))
    y = oracle.expert_ffn(x, np.zeros((8, 16)), np.zeros((8, 16)), np.zeros((16, 8)))
    assert np.all(y == 0)


def test_ffn_silu_saturation_no_nan():
    x = np.array([[1000.0, -1000.0]])
    wg = np.array([[1.0, 0.0], [-1.0, 0.0]])
    wu = np.array([[1.0, 0.0], [1.0, 0.0]])      # u = (1000, 1000)
    wd = np.eye(2)
    y = oracle.expert_ffn(x, wg, wu, wd)
    assert np.all(np.isfinite(y))
    # g = (1000, -1000): silu(1000) * 1000 = 1e6 exactly in fp64, silu(-1000) = 0
    assert y[0, 0] == 1e6 and y[0, 1] == 0.0


def test_combine_handworked():
    y = np.arange(2 * 3 * 2, dtype=np.float64).reshape(2, 3, 2)
    w = np.array([[0.5, 0.25, 0.25], [1.0, 0.0, 0.0]])
    out = oracle.combine(y, w)
    assert np.array_equal(out[0], 0.5 * y[0, 0] + 0.25 * y[0, 1] + 0.25 * y[0, 2])
    assert np.array_equal(out[1], y[1, 0])


def _tiny_layer(E=8, H=64, I=32, seed=0):
    rs = np.random.default_rng(seed)
    W = {}
    for e in range(E):
        mats = []
        for shape in [(I, H), (I, H), (H, I)]:
            w = (rs.standard_normal(shape) * 0.02).astype(np.float32)
            c, s = oracle.nvfp4_quantize(w)
            mats.append(oracle.nvfp4_dequant(c, s))
        W[e] = tuple(mats)
    return W


def test_forward_equals_dense_masked_form():
    """out[t] = sum_e [e in topk(t)] w_te FFN_e(x_t), evaluated densely over
    every expert."""
    E, k, H, I, T = 8, 2, 64, 32, 5
    W = _tiny_layer(E, H, I)
    rs = np.random.default_rng(1)
    x_bits = synth.f32_to_bf16_bits(rs.standard_normal((T, H)).astype(np.float32))
    lg = rs.standard_normal((T, E)).astype(np.float32)
    out, ids, w, y = oracle.forward(x_bits, lg, k, lambda e: W[e])
    x = oracle.bf16_bits_to_f64(x_bits)
    dense = np.zeros((T, H))
    for e in range(E):
        ye = oracle.expert_ffn(x, *W[e])
        for t in range(T):
            for j in range(k):
                if ids[t, j] == e:
                    dense[t] += w[t, j] * ye[t]
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-15)


def test_forward_closed_form_unit_codes():
    """Every code = 1.0 (code 2) and every scale byte the same s: each expert
    has W = s everywhere, so g = u = s*sum(x), h = silu(g) g, y = s I h for
    every chosen expert and out = y (the weights sum to 1)."""
    E, k, H, I, T = 4, 2, 32, 16, 3
    sb = 0x30                            # E4M3 0x30 = 0.5
    s = float(oracle.e4m3_decode(sb))
    codes13 = np.full((I, H // 2), 0x22, np.uint8)
    codes2 = np.full((H, I // 2), 0x22, np.uint8)
    W13 = oracle.nvfp4_dequant(codes13, np.full((I, H // 16), sb, np.uint8))
    W2 = oracle.nvfp4_dequant(codes2, np.full((H, I // 16), sb, np.uint8))
    assert np.all(W13 == s) and np.all(W2 == s)
    rs = np.random.default_rng(2)
    x_bits = synth.f32_to_bf16_bits(rs.standard_normal((T, H)).astype(np.float32))
    lg = rs.standard_normal((T, E)).astype(np.float32)
    out, ids, w, y = oracle.forward(x_bits, lg, k, lambda e: (W13, W13, W2))
    x = oracle.bf16_bits_to_f64(x_bits)
    g = s * x.sum(1)
    h = g * g / (1 + np.exp(-g))
    want = (s * I * h)[:, None] * np.ones((1, H))
    assert np.allclose(out, want, rtol=1e-12)


def test_forward_k1_is_expert_output():
    E, H, I, T = 8, 64, 32, 4
    W = _tiny_layer(E, H, I, seed=5)
    rs = np.random.default_rng(6)
    x_bits = synth.f32_to_bf16_bits(rs.standard_normal((T, H)).astype(np.float32))
    lg = rs.standard_normal((T, E)).astype(np.float32)
    out, ids, w, y = oracle.forward(x_bits, lg, 1, lambda e: W[e])
    assert np.all(w == 1.0)
    assert np.array_equal(out, y[:, 0])
    x = oracle.bf16_bits_to_f64(x_bits)
    for t in range(T):
        # BLAS may sum in another order for a different row count
        assert np.allclose(y[t, 0], oracle.expert_ffn(x[t:t + 1], *W[ids[t, 0]])[0],
                           rtol=1e-12, atol=1e-16)


def test_forward_all_zero_scales_expert_outputs_zero():
    E, k, H, I, T = 4, 2, 32, 16, 3
    Z13 = oracle.nvfp4_dequant(np.full((I, H // 2), 0x77, np.uint8), np.zeros((I, H // 16), np.uint8))
    Z2 = oracle.nvfp4_dequant(np.full((H, I // 2), 0x77, np.uint8), np.zeros((H, I // 16), np.uint8))
    rs = np.random.default_rng(3)
    x_bits = synth.f32_to_bf16_bits(rs.standard_normal((T, H)).astype(np.float32))
    lg = rs.standard_normal((T, E)).astype(np.float32)
    out, *_ = oracle.forward(x_bits, lg, k, lambda e: (Z13, Z13, Z2))
    assert np.all(out == 0)


# ---------------------------------------------------------------- synth recipes

def test_hot_bias_gives_expected_share():
    wl = synth.MIXED
    beta = synth.hot_bias(wl.E, wl.k, wl.n_hot, wl.hot_share)
    assert 0 < beta < 1
    # Monte Carlo check of the recipe (not of the method)
    rs = np.random.default_rng(0)
    hot = np.zeros(wl.E, bool)
    hot[:wl.n_hot] = True
    lg = rs.random((20000, wl.E)) + beta * hot
    top = np.argpartition(-lg, wl.k, axis=1)[:, :wl.k]
    share = hot[top].mean()
    assert abs(share - wl.hot_share) < 0.01


def test_synth_is_deterministic():
    a = synth.logits(synth.DECODE, 8)
    b = synth.logits(synth.DECODE, 8)
    assert np.array_equal(a, b)
    x = synth.activations(synth.TINY, 4)
    assert x.dtype == np.uint16 and x.shape == (4, 256)
    tm = synth.tier_map(synth.MIXED)
    assert (tm == synth.FMT_NVFP4).sum() == 108 and (tm == synth.FMT_VQ).sum() == 148


# ------------------------------------------------------------ shared expert

def test_shared_expert_alone_when_routed_outputs_vanish():
    # routed experts with all-zero weights: the forward is the shared FFN
    rs = np.random.default_rng(21)
    T, E, k, H, I = 5, 6, 2, 32, 16
    x = synth.f32_to_bf16_bits(rs.standard_normal((T, H)).astype(np.float32))
    lg = rs.standard_normal((T, E)).astype(np.float32)
    zero = (np.zeros((I, H)), np.zeros((I, H)), np.zeros((H, I)))
    sh = (rs.standard_normal((I, H)) * 0.1, rs.standard_normal((I, H)) * 0.1,
          rs.standard_normal((H, I)) * 0.1)
    out, ids, w, y = oracle.forward(x, lg, k, lambda e: zero, shared_weights=sh)
    assert np.all(y == 0)
    assert np.array_equal(out, oracle.expert_ffn(x, *sh))


def test_shared_expert_dense_form():
    # out = sum_e [e routed] w_te FFN_e(x_t) + FFN_s(x_t), computed densely
    rs = np.random.default_rng(22)
    T, E, k, H, I = 7, 5, 3, 24, 8
    x = synth.f32_to_bf16_bits(rs.standard_normal((T, H)).astype(np.float32))
    lg = rs.standard_normal((T, E)).astype(np.float32)
    Ws = {e: (rs.standard_normal((I, H)) * 0.2, rs.standard_normal((I, H)) * 0.2,
              rs.standard_normal((H, I)) * 0.2) for e in range(E)}
    sh = (rs.standard_normal((I, H)) * 0.2, rs.standard_normal((I, H)) * 0.2,
          rs.standard_normal((H, I)) * 0.2)
    out, ids, w, y = oracle.forward(x, lg, k, lambda e: Ws[e], shared_weights=sh)
    dense = oracle.expert_ffn(x, *sh)
    for e in range(E):
        m = (ids == e)
        wt = (w * m).sum(axis=1)
        dense = dense + wt[:, None] * oracle.expert_ffn(x, *Ws[e])
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-12)
    # and without the shared expert the routed part alone
    out0, *_ = oracle.forward(x, lg, k, lambda e: Ws[e])
    assert np.allclose(out - out0, oracle.expert_ffn(x, *sh), rtol=1e-12, atol=1e-12)
