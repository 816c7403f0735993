"""Oracle: the incoherence rotation of rotated-format expert weights, in float64.

TEST INFRASTRUCTURE ONLY -- see oracle/__init__.py.

"GLM-5.3 Vision NestQuant 1.75-4 bit", Method: random signs and a
Hadamard-128 transform on both sides of each weight matrix.  Read here as the
orthonormal block-diagonal rotation

    R = blockdiag(H_b / sqrt(b), ...) @ diag(s),   s in {+1, -1}^N,   b = 128,

on each side of a matrix: the stored (then quantized) matrix is
W_rot = R_out W R_in^T, so that W = R_out^T W_rot R_in and the layer computes
W x = R_out^T (W_rot (R_in x)): the input is rotated online before the product
with the stored matrix and the output rotated back after it.  The random
signs are the only per-matrix data (one vector per side).

What the rotated expert computes is therefore the plain FFN with the effective
weights R_out^T Q(W_rot) R_in (Q = the stored format's decode); the oracle
takes that definition: it un-rotates the decoded matrix and evaluates the
ordinary expert FFN.  (Reading: gate and up share their input-side rotation,
because they share their input; every other side has its own signs.)

The same Method names a wider variant for the down projection of some layers:
its input side takes random signs and one Hadamard-512 per tensor-parallel
shard of the intermediate dimension, with a flat (uniform) input-channel
scale.  Read here as the same rotation with block b = 512 on that one side
(R_in = blockdiag(H_512 / sqrt(512)) diag(s)); the scale is the rotation's own
normalisation, no per-channel factor.  Every side therefore takes its own
block: `rotate_weights` / `unrotate_weights` accept block_out and block_in.
"""

import numpy as np

BLOCK = 128


def hadamard(n):
    """The n x n Hadamard matrix of Sylvester's construction, entries +-1
    (H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]); n a power of two."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate(v, signs, block=BLOCK):
    """R v along the last axis: each block of `block` entries of (s * v) times
    H_block / sqrt(block)."""
    v = np.asarray(v, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    n = v.shape[-1]
    if n % block:
        raise ValueError("length must be a multiple of the block")
    hb = hadamard(block) / np.sqrt(block)
    w = (v * s).reshape(v.shape[:-1] + (n // block, block))
    return (w @ hb.T).reshape(v.shape)


def unrotate(v, signs, block=BLOCK):
    """R^T v along the last axis: (H_block / sqrt(block)) per block, then the
    signs."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    if n % block:
        raise ValueError("length must be a multiple of the block")
    hb = hadamard(block) / np.sqrt(block)
    w = v.reshape(v.shape[:-1] + (n // block, block)) @ hb
    return w.reshape(v.shape) * np.asarray(signs, dtype=np.float64)


def rotate_weights(w, s_out, s_in, block_out=BLOCK, block_in=BLOCK):
    """W_rot = R_out W R_in^T for W [n_out, n_in], R_out of block block_out and
    R_in of block block_in."""
    a = rotate(np.asarray(w, dtype=np.float64), s_in, block_in)     # rows: W R_in^T
    return rotate(a.T, s_out, block_out).T                           # columns: R_out (.)


def unrotate_weights(w_rot, s_out, s_in, block_out=BLOCK, block_in=BLOCK):
    """R_out^T W_rot R_in for W_rot [n_out, n_in]: the effective weights of a
    rotated matrix (blocks as in rotate_weights)."""
    a = unrotate(np.asarray(w_rot, dtype=np.float64), s_in, block_in)   # rows: W_rot R_in
    return unrotate(a.T, s_out, block_out).T                             # columns: R_out^T (.)
