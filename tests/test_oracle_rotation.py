"""Pins of the oracle's incoherence rotation ("GLM-5.3 Vision NestQuant 1.75-4
bit", Method: random signs + Hadamard-128 on both sides of each weight
matrix) against scipy's Hadamard matrix, dense Kronecker constructions, a
hand-worked case and the identities an orthonormal rotation must satisfy."""

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 256, 512])
def test_hadamard_is_scipys(n):
    assert np.array_equal(oracle.hadamard(n), scipy.linalg.hadamard(n))


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.hadamard(96)


def _dense_rotation(signs, block):
    n = len(signs)
    hb = scipy.linalg.hadamard(block) / np.sqrt(block)
    return np.kron(np.eye(n // block), hb) @ np.diag(np.asarray(signs, np.float64))


@pytest.mark.parametrize("n,block", [(256, 128), (384, 128), (16, 4), (8, 8), (512, 512),
                                     (1536, 512)])
def test_rotate_is_the_dense_block_rotation(n, block):
    rs = np.random.default_rng(n + block)
    s = np.where(rs.random(n) < 0.5, -1, 1)
    v = rs.standard_normal((3, n))
    R = _dense_rotation(s, block)
    assert np.allclose(oracle.rotate(v, s, block), v @ R.T, rtol=0, atol=1e-12)
    assert np.allclose(oracle.unrotate(v, s, block), v @ R, rtol=0, atol=1e-12)
    assert np.allclose(R @ R.T, np.eye(n), atol=1e-12)


def test_rotate_hand_worked():
    # signs (+1, -1), H_2 / sqrt(2) = [[1, 1], [1, -1]] / sqrt(2); v = (3, 5):
    # s * v = (3, -5) -> ((3 - 5), (3 + 5)) / sqrt(2) = (-sqrt(2), 4 sqrt(2))
    r = oracle.rotate(np.array([3.0, 5.0]), [1, -1], block=2)
    assert np.allclose(r, [-np.sqrt(2), 4 * np.sqrt(2)], rtol=0, atol=1e-15)
    assert np.allclose(oracle.unrotate(r, [1, -1], block=2), [3.0, 5.0], rtol=0, atol=1e-15)


def test_rotation_is_orthonormal():
    rs = np.random.default_rng(7)
    s = np.where(rs.random(6144) < 0.5, -1, 1)
    v = rs.standard_normal((4, 6144))
    r = oracle.rotate(v, s)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(v, axis=1), rtol=1e-13)
    assert np.allclose(oracle.unrotate(r, s), v, rtol=0, atol=1e-12)


def test_rotate_weights_dense():
    rs = np.random.default_rng(11)
    n_out, n_in = 256, 384
    so = np.where(rs.random(n_out) < 0.5, -1, 1)
    si = np.where(rs.random(n_in) < 0.5, -1, 1)
    W = rs.standard_normal((n_out, n_in))
    Ro, Ri = _dense_rotation(so, 128), _dense_rotation(si, 128)
    assert np.allclose(oracle.rotate_weights(W, so, si), Ro @ W @ Ri.T, atol=1e-12)
    assert np.allclose(oracle.unrotate_weights(W, so, si), Ro.T @ W @ Ri, atol=1e-12)
    assert np.allclose(oracle.unrotate_weights(oracle.rotate_weights(W, so, si), so, si), W,
                       atol=1e-12)


def test_rotate_weights_mixed_blocks_dense():
    """The wide down-input variant: block 512 on the input side, 128 on the
    output side, against the dense Kronecker rotations."""
    rs = np.random.default_rng(12)
    n_out, n_in = 256, 1024
    so = np.where(rs.random(n_out) < 0.5, -1, 1)
    si = np.where(rs.random(n_in) < 0.5, -1, 1)
    W = rs.standard_normal((n_out, n_in))
    Ro, Ri = _dense_rotation(so, 128), _dense_rotation(si, 512)
    assert np.allclose(oracle.rotate_weights(W, so, si, block_in=512), Ro @ W @ Ri.T, atol=1e-12)
    assert np.allclose(oracle.unrotate_weights(W, so, si, block_in=512), Ro.T @ W @ Ri,
                       atol=1e-12)
    # the sides are not interchangeable: the 128-block input rotation differs
    assert not np.allclose(oracle.unrotate_weights(W, so, si), Ro.T @ W @ Ri, atol=1e-3)
    # and the output side takes its own block
    W2 = rs.standard_normal((1024, 256))
    Ro2, Ri2 = _dense_rotation(si, 512), _dense_rotation(so, 128)
    assert np.allclose(oracle.unrotate_weights(W2, si, so, block_out=512), Ro2.T @ W2 @ Ri2,
                       atol=1e-12)


def test_rotate_512_factors_through_the_128_blocks():
    """Sylvester's order gives H_512 = H_4 (x) H_128, so the 512-block rotation
    is the 128-block rotation followed by a butterfly across the four 128-blocks
    of each 512-block (normalised by 1/2): the factorisation an online
    transform takes (two more butterfly stages after the 128-point ones)."""
    rs = np.random.default_rng(13)
    n = 1024
    s = np.where(rs.random(n) < 0.5, -1, 1)
    v = rs.standard_normal((4, n))
    r128 = oracle.rotate(v, s, 128).reshape(4, n // 512, 4, 128)
    cross = np.einsum("ij,rbjc->rbic", scipy.linalg.hadamard(4) / 2.0, r128).reshape(4, n)
    assert np.allclose(oracle.rotate(v, s, 512), cross, rtol=0, atol=1e-12)


@pytest.mark.parametrize("rot_in2", [128, 512])
def test_rotated_ffn_steps_equal_the_effective_weights(rot_in2):
    """The rotated layer's steps in order -- rotate x, product with the stored
    matrices, rotate the gate/up outputs back, SwiGLU, rotate h, product,
    rotate the output back -- equal the plain FFN with the effective weights
    R_out^T W_rot R_in that the oracle evaluates (also with the wide 512-block
    rotation on the down projection's input side)."""
    wl = synth.small_workload("rot_pin", E=2, k=1, H=256, I=512, T=5, rot=True, rot_in2=rot_in2)
    rs = np.random.default_rng(5)
    Wg, Wu, Wd = (rs.standard_normal((512, 256)) * 0.05, rs.standard_normal((512, 256)) * 0.05,
                  rs.standard_normal((256, 512)) * 0.05)
    s = {side: synth.rot_signs(wl, 1, side) for side in range(5)}
    b2 = wl.rot_in2
    x = rs.standard_normal((5, 256))
    xr = oracle.rotate(x, s[synth.ROT_IN13])
    g = oracle.unrotate(xr @ Wg.T, s[synth.ROT_OUT_GATE])
    u = oracle.unrotate(xr @ Wu.T, s[synth.ROT_OUT_UP])
    h = g * u / (1 + np.exp(-g))
    y = oracle.unrotate(oracle.rotate(h, s[synth.ROT_IN2], b2) @ Wd.T, s[synth.ROT_OUT2])
    eff = (oracle.unrotate_weights(Wg, s[synth.ROT_OUT_GATE], s[synth.ROT_IN13]),
           oracle.unrotate_weights(Wu, s[synth.ROT_OUT_UP], s[synth.ROT_IN13]),
           oracle.unrotate_weights(Wd, s[synth.ROT_OUT2], s[synth.ROT_IN2], block_in=b2))
    assert np.allclose(oracle.expert_ffn(x, *eff), y, rtol=0, atol=1e-12)
    # and a matrix stored rotated from plain weights gives back the plain FFN
    rot = (oracle.rotate_weights(Wg, s[synth.ROT_OUT_GATE], s[synth.ROT_IN13]),
           oracle.rotate_weights(Wu, s[synth.ROT_OUT_UP], s[synth.ROT_IN13]),
           oracle.rotate_weights(Wd, s[synth.ROT_OUT2], s[synth.ROT_IN2], block_in=b2))
    eff2 = (oracle.unrotate_weights(rot[0], s[synth.ROT_OUT_GATE], s[synth.ROT_IN13]),
            oracle.unrotate_weights(rot[1], s[synth.ROT_OUT_UP], s[synth.ROT_IN13]),
            oracle.unrotate_weights(rot[2], s[synth.ROT_OUT2], s[synth.ROT_IN2], block_in=b2))
    assert np.allclose(oracle.expert_ffn(x, *eff2), oracle.expert_ffn(x, Wg, Wu, Wd), atol=1e-12)


def test_rotation_spreads_an_outlier():
    """What the rotation is for: one large input channel is spread evenly over
    its 128-block (every entry of a rotated one-hot vector has magnitude
    1/sqrt(128))."""
    s = np.ones(256)
    e = np.zeros(256)
    e[37] = 1.0
    r = oracle.rotate(e, s)
    assert np.allclose(np.abs(r[:128]), 1 / np.sqrt(128), rtol=0, atol=1e-15)
    assert np.all(r[128:] == 0)
    # the wide block spreads it over all 512 entries of its block
    e2 = np.zeros(1024)
    e2[600] = 1.0
    r2 = oracle.rotate(e2, np.ones(1024), 512)
    assert np.allclose(np.abs(r2[512:]), 1 / np.sqrt(512), rtol=0, atol=1e-15)
    assert np.all(r2[:512] == 0)
