"""Oracle: routing, permutation, expert FFN and combine, in float64.

TEST INFRASTRUCTURE ONLY -- see oracle/__init__.py.

The forward is the plain definition, token by token:
    out[t] = sum_{j=0}^{k-1} w[t, j] * FFN_{ids[t, j]}(x_t)
    FFN_e(x) = W_down[e] (silu(W_gate[e] x) * (W_up[e] x))
with ids/w from a top-k over the router logits and softmax weights
renormalised over the chosen experts.
  * 256 routed experts, 8 active per token: GLM-5-NVFP4-MTP, "Model Description".
  * gate, up and down projections of each expert: GLM-5-NVFP4-MTP,
    "What's quantized".
  * routers kept exact / in fp32: GLM-5.3-EXL3-TR3-3.42bpw, "What is
    quantized" (mlp.gate carried byte-exact) and GLM-5.3-Flash-TR3-8bpw (K8),
    introduction (routers in native precision) -- so router logits are fp32
    inputs here.
  * the combine order matters for the bits (GLM-5.3-Flash-TR3-8bpw (K8),
    "Fidelity" and "Excess over control"), so it is fixed: ascending j.
"""

import numpy as np

from .formats import bf16_bits_to_f64


def route_topk(logits, k):
    """Top-k experts per token and their renormalised softmax weights.

    Experts are ordered by (logit descending, expert id ascending); -0.0 and
    +0.0 compare equal; NaN logits are rejected.  ids[t, j] is the expert of
    rank j.  w[t, j] = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), in float64
    from the fp32 logits.
    """
    lg = np.asarray(logits, dtype=np.float32)
    if lg.ndim != 2:
        raise ValueError("logits must be [T, E]")
    T, E = lg.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    if np.isnan(lg).any():
        raise ValueError("NaN logit")
    l64 = lg.astype(np.float64)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    eid = np.arange(E)
    for t in range(T):
        # lexsort: last key is primary.  -l puts larger logits first; the
        # expert id breaks ties (lower id first).  -(+0.0) == -(-0.0).
        order = np.lexsort((eid, -l64[t]))
        sel = order[:k]
        ids[t] = sel
        lsel = l64[t, sel]
        ex = np.exp(lsel - lsel[0])
        w[t] = ex / ex.sum()
    return ids, w


def permute(ids, E):
    """Group the T*k assignments by expert.

    a = t*k + j is the flat index of assignment (t, j), e_a = ids[t, j].
    counts[e] = #{a : e_a = e}; offsets = exclusive prefix sum of counts
    (offsets[E] = T*k); perm_src lists, expert by expert in ascending e, the
    assignments of that expert in ascending a; inv_perm[perm_src[i]] = i.
    """
    ids = np.asarray(ids, dtype=np.int64)
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    perm_src = np.concatenate(
        [np.nonzero(flat == e)[0] for e in range(E)] + [np.zeros(0, np.int64)]
    ).astype(np.int64)
    inv_perm = np.empty_like(perm_src)
    inv_perm[perm_src] = np.arange(perm_src.size)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm_src.astype(np.int32), inv_perm.astype(np.int32))


def expert_ffn(x, w_gate, w_up, w_down):
    """y = W_down (silu(g) * u), g = W_gate x, u = W_up x, for each row of x.

    x float64 [M, H] (or bf16 bits as uint16, widened exactly); W_gate and
    W_up [I, H], W_down [H, I] float64.  silu(g) * u = g * u / (1 + e^-g).
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x = bf16_bits_to_f64(x)
    x = x.astype(np.float64)
    g = x @ np.asarray(w_gate, dtype=np.float64).T
    u = x @ np.asarray(w_up, dtype=np.float64).T
    with np.errstate(over="ignore"):
        h = g * u / (1.0 + np.exp(-g))
    return h @ np.asarray(w_down, dtype=np.float64).T


def combine(y, w):
    """out[t] = sum_{j=0}^{k-1} w[t, j] * y[t, j], summed in ascending j.

    y float64 [T, k, H]; w float64 [T, k]."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, k, H = y.shape
    out = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        out += w[:, j, None] * y[:, j, :]
    return out


def combine_shared(y, w, y_shared):
    """The routed combine followed by the shared expert's output:
    out[t] = (sum_{j=0}^{k-1} w[t, j] * y[t, j]) + y_shared[t], the routed sum
    in ascending j first.  (GLM-5.3-EXL3-TR3-3.42bpw, What is quantized: the
    layers carry BF16 shared experts next to the routed ones; every token
    passes through the shared expert with weight 1.  Adding it after the
    routed sum is a reading.)"""
    return combine(y, w) + np.asarray(y_shared, dtype=np.float64)


def forward(x_bits, logits, k, expert_weights, shared_weights=None):
    """The whole routed-expert forward for T tokens.

    x_bits uint16 bf16 bits [T, H]; logits fp32 [T, E]; expert_weights(e) ->
    (W_gate [I, H], W_up [I, H], W_down [H, I]) float64, called once per
    touched expert; shared_weights: None or the shared expert's (W_gate, W_up,
    W_down) float64.  Returns (out [T, H], ids [T, k], w [T, k],
    y [T, k, H]) where y[t, j] = FFN_{ids[t, j]}(x_t); with a shared expert,
    out adds FFN_shared(x_t) after the routed sum.
    """
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    ids, w = route_topk(logits, k)
    T = x.shape[0]
    H = x.shape[1]
    y = np.zeros((T, k, H), dtype=np.float64)
    for e in np.unique(ids):
        wg, wu, wd = expert_weights(int(e))
        tt, jj = np.nonzero(ids == e)
        y[tt, jj] = expert_ffn(x[tt], wg, wu, wd)
    if shared_weights is None:
        return combine(y, w), ids, w, y
    return combine_shared(y, w, expert_ffn(x, *shared_weights)), ids, w, y
