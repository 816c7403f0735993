"""Seeded synthetic inputs for the routed-expert MoE workloads.

This module is shared by the oracle side (tests, CPU baseline) and the HIP
side (tests, bench).  It only draws random inputs -- logits, activations,
fp32 expert weights, VQ codes/codebooks/scales, tier maps -- and rounds them
to their storage types.  It holds none of the method's arithmetic: no format
encoding, no routing, no FFN.

Seeds: numpy PCG64 seeded by SeedSequence([20260711, cfg, kind, expert, proj,
rep]).  The tuple mirrors the (layer, expert, projection, rank) seed scheme
and seed base of GLM-5.3-EXL3-TR3-3.42bpw ("What is quantized": deterministic,
data-free encode).

Workloads (names used throughout tests/ and bench.py):
  tiny    E=8,   k=2, H=256,  I=128,  T=4     NVFP4 from N(0, 0.02) fp32,
                                              logits N(0,1)
  decode  E=256, k=8, H=6144, I=2048, T in {1, 8, 32}, NVFP4 layer,
                                              logits U[0,1)
  prefill same layer as decode, T=4096, Zipf(1.1) expert popularity
  vq      E=256, k=8, H=6144, I=2048, T=8, 2-bit AQLM-style VQ,
                                              logits U[0,1)
  mixed   108 NVFP4 + 148 VQ experts (seeded tier map), T in {8, 32},
          20 hot experts receive 60% of assignments in expectation
Activations are bf16 ~ N(0, 1) in all of them.
"""

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 20260711

# kinds of random stream
KIND_W = 0
KIND_LOGITS = 1
KIND_X = 2
KIND_VQ_CODES = 3
KIND_VQ_CODEBOOK = 4
KIND_VQ_SCALES = 5
KIND_TIER = 6
KIND_HOT = 7
KIND_ZIPF_RANK = 8
KIND_VQ8_CODES = 9
KIND_VQ8_CODEBOOK = 10
KIND_SHARED = 11
KIND_ROT_SIGNS = 12
KIND_VQ_CODEBOOK_EXPERT = 13

# sides of a rotated expert that carry their own random signs
ROT_IN13, ROT_OUT_GATE, ROT_OUT_UP, ROT_IN2, ROT_OUT2 = 0, 1, 2, 3, 4

PROJ_GATE, PROJ_UP, PROJ_DOWN = 0, 1, 2

FMT_NVFP4 = 1
FMT_VQ = 2
FMT_VQ8 = 3
FMT_BF16 = 4
FMT_NVFP4R = 5      # nested two-level NVFP4 (base plane + residual plane)
FMT_VQ8_M1 = 6      # small-codebook VQ at an explicit rate: 1, 2 or 3 codes
FMT_VQ8_M2 = 7      # (bits per weight) per 8-weight group
FMT_VQ8_M3 = 8
# the share of each VQ rate among a layer's experts: the module counts of the
# 1-, 2- and 3-bit modules of "GLM-5.2 mixed-bit VQ (AQLM) ~1.90 bpw", What it
# is (every module is one projection of one expert; here one rate per expert)
VQ8_RATE_COUNTS = (29456, 12441, 15703)
NVFP4R_SHIFT = 8    # residual-plane exponent of the nested layers


def rng(cfg, kind, expert=0, proj=0, rep=0):
    ss = np.random.SeedSequence([SEED_BASE, int(cfg), int(kind), int(expert),
                                 int(proj), int(rep)])
    return np.random.Generator(np.random.PCG64(ss))


# --------------------------------------------------------------------------
# storage-type rounding of drawn values
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x):
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_to_f16_bits(x):
    """Round to IEEE binary16 (numpy's cast: nearest, ties to even)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


# --------------------------------------------------------------------------
# workload shapes
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    cfg: int            # seed slot of the routing/activation streams
    E: int
    k: int
    H: int
    I: int
    T: tuple
    fmt: str            # "nvfp4", "vq", "vq8", "bf16", "mixed" (NVFP4 + VQ), "mixed3"
                        # (+ VQ8), "nv_bf16" (NVFP4 + BF16), "nested" (NVFP4 base
                        # tier, some experts lifted to two-level NVFP4) or "vqmix"
                        # (small-codebook VQ experts at 1, 2 and 3 bits per weight)
    logits: str         # "normal", "uniform", "zipf" or "hot"
    weight_cfg: int = 1     # seed slot of the NVFP4 weights
    vq_cfg: int = 3         # seed slot of the VQ codes/codebooks/scales
    n_nvfp4: int = 0        # mixed only
    n_hot: int = 0
    hot_share: float = 0.0
    zipf_s: float = 0.0
    vq8_m: int = 0          # codes per 8-weight group of the small-codebook VQ
    shared: bool = False    # the layer has a BF16 shared expert
    rot: bool = False       # expert weights stored rotated (signs + Hadamard-128)
    rot_in2: int = 128      # Hadamard block of the down projection's input side
                            # of a rotated layer: 128, or 512 (the wide variant)
    extra: dict = field(default_factory=dict, compare=False, hash=False)


TINY = Workload("tiny", 0, 8, 2, 256, 128, (4,), "nvfp4", "normal", weight_cfg=0)
DECODE = Workload("decode", 1, 256, 8, 6144, 2048, (1, 8, 32), "nvfp4", "uniform")
PREFILL = Workload("prefill", 2, 256, 8, 6144, 2048, (4096,), "nvfp4", "zipf",
                   zipf_s=1.1)
VQ = Workload("vq", 3, 256, 8, 6144, 2048, (8,), "vq", "uniform")
MIXED = Workload("mixed", 4, 256, 8, 6144, 2048, (8, 32), "mixed", "hot",
                 n_nvfp4=108, n_hot=20, hot_share=0.6)

# small-codebook VQ decode layers (1 and 2 bits per weight), T = 8
VQ1 = Workload("vq1", 5, 256, 8, 6144, 2048, (8,), "vq8", "uniform", vq_cfg=5, vq8_m=1)
VQ2X8 = Workload("vq2x8", 6, 256, 8, 6144, 2048, (8,), "vq8", "uniform", vq_cfg=6, vq8_m=2)
# the 3-bit module: three uint8 codes per group into three 256-entry codebooks
VQ3X8 = Workload("vq3x8", 8, 256, 8, 6144, 2048, (8,), "vq8", "uniform", vq_cfg=8, vq8_m=3)

# small-codebook VQ experts at mixed rates (1, 2 and 3 bits per weight, in the
# proportions of the page's module counts), three shared codebooks per
# projection, T = 8
VQMIX = Workload("vqmix", 10, 256, 8, 6144, 2048, (8,), "vqmix", "uniform", vq_cfg=10, vq8_m=3)

# the NVFP4 decode and prefill layers with a BF16 shared expert of the same
# intermediate size (the routed experts, routing and tokens are those of
# DECODE / PREFILL: same seed slots)
# the decode layer with rotated NVFP4 experts: the stored matrices (the NVFP4
# source weights) are taken to be in the rotated domain, W_rot ~ N(0, 0.02)
DECODE_ROT = Workload("decode_rot", 7, 256, 8, 6144, 2048, (1, 8, 32), "nvfp4", "uniform",
                      weight_cfg=1, rot=True)
# the same with the wide down-input rotation (signs + one Hadamard-512 per
# 512 intermediate channels on the down projection's input side); same seed
# slot: same stored matrices and signs
DECODE_ROT512 = Workload("decode_rot512", 7, 256, 8, 6144, 2048, (1, 8, 32), "nvfp4", "uniform",
                         weight_cfg=1, rot=True, rot_in2=512)
DECODE_SHARED = Workload("decode_shared", 1, 256, 8, 6144, 2048, (1, 8, 32), "nvfp4", "uniform",
                         shared=True)
# the decode layer's NVFP4 experts (same source weights) held nested: every
# expert's two-level record resident, the 20 hot experts (60% of the
# assignments) lifted to the two-level tier, the rest on their base planes
NESTED = Workload("nested", 9, 256, 8, 6144, 2048, (8, 32), "nested", "hot", weight_cfg=1,
                  n_hot=20, hot_share=0.6)
PREFILL_SHARED = Workload("prefill_shared", 2, 256, 8, 6144, 2048, (4096,), "nvfp4", "zipf",
                          zipf_s=1.1, shared=True)

WORKLOADS = {w.name: w for w in (TINY, DECODE, PREFILL, VQ, MIXED, VQ1, VQ2X8, VQ3X8, DECODE_SHARED,
                                 PREFILL_SHARED, DECODE_ROT, DECODE_ROT512, NESTED, VQMIX)}


def small_workload(name, E, k, H, I, T, fmt="nvfp4", logits="normal", cfg=100,
                   n_nvfp4=0, n_hot=0, hot_share=0.0, zipf_s=0.0, vq8_m=0, shared=False,
                   rot=False, rot_in2=128):
    """A property-test workload with its own seed slot."""
    return Workload(name, cfg, E, k, H, I, (T,), fmt, logits, weight_cfg=cfg,
                    vq_cfg=cfg, n_nvfp4=n_nvfp4, n_hot=n_hot, hot_share=hot_share,
                    zipf_s=zipf_s, vq8_m=vq8_m, shared=shared, rot=rot, rot_in2=rot_in2)


# --------------------------------------------------------------------------
# activations and logits
# --------------------------------------------------------------------------

def activations(wl, T, rep=0):
    """bf16 ~ N(0, 1) activations [T, H] as uint16 bits."""
    x = rng(wl.cfg, KIND_X, 0, T, rep).standard_normal((T, wl.H), dtype=np.float32)
    return f32_to_bf16_bits(x)


def logits(wl, T, rep=0):
    """fp32 router logits [T, E] following the workload's recipe."""
    g = rng(wl.cfg, KIND_LOGITS, 0, T, rep)
    if wl.logits == "normal":
        return g.standard_normal((T, wl.E), dtype=np.float32)
    if wl.logits == "uniform":
        return g.random((T, wl.E), dtype=np.float32)
    if wl.logits == "zipf":
        return zipf_logits(wl, g, T)
    if wl.logits == "hot":
        hot = hot_experts(wl)
        beta = np.float32(hot_bias(wl.E, wl.k, wl.n_hot, wl.hot_share))
        lg = g.random((T, wl.E), dtype=np.float32)
        lg[:, hot] += beta
        return lg
    raise ValueError(wl.logits)


def zipf_popularity(wl):
    """p_e proportional to r_e^-s over a seeded permutation r of ranks 1..E."""
    ranks = rng(wl.cfg, KIND_ZIPF_RANK).permutation(wl.E) + 1
    p = ranks.astype(np.float64) ** (-wl.zipf_s)
    return p / p.sum()


def zipf_logits(wl, g, T):
    """ln p_e + Gumbel(0, 1) noise, fp32: the top-k of these samples k experts
    without replacement with probability proportional to p (Gumbel-top-k)."""
    p = zipf_popularity(wl)
    u = g.random((T, wl.E))
    u = np.clip(u, 1e-300, None)
    gumbel = -np.log(-np.log(u))
    return (np.log(p)[None, :] + gumbel).astype(np.float32)


def hot_experts(wl):
    return np.sort(rng(wl.cfg, KIND_HOT).choice(wl.E, size=wl.n_hot, replace=False))


def hot_bias(E, k, n_hot, share, n_quad=4000):
    """Bias b added to the U[0,1) logits of n_hot experts so that, in
    expectation, a fraction `share` of the top-k picks are hot.

    A hot expert with value y (uniform on [b, 1+b)) is picked iff at most k-1
    of the other experts exceed y: Binomial(n_hot-1, 1+b-y) hot ones plus
    Binomial(E-n_hot, max(0, 1-y)) cold ones.  The expected hot share is
    n_hot/k * P(picked); b is found by bisection (the share grows with b).
    """
    from scipy.stats import binom

    def expected_share(b):
        y = b + (np.arange(n_quad) + 0.5) / n_quad
        qh = np.clip(1.0 + b - y, 0.0, 1.0)
        qc = np.clip(1.0 - y, 0.0, 1.0)
        j = np.arange(k)
        ph = binom.pmf(j[None, :], n_hot - 1, qh[:, None])       # [n, k]
        pc = binom.pmf(j[None, :], E - n_hot, qc[:, None])
        # P(Nh + Nc <= k-1) = sum_{a+c<=k-1} ph[a] pc[c]
        cpc = np.cumsum(pc, axis=1)
        prob = np.zeros(n_quad)
        for a in range(k):
            prob += ph[:, a] * cpc[:, k - 1 - a]
        return n_hot / k * prob.mean()

    lo, hi = 0.0, 1.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if expected_share(mid) < share:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


# --------------------------------------------------------------------------
# expert weights
# --------------------------------------------------------------------------

def proj_shape(wl, proj):
    return (wl.I, wl.H) if proj in (PROJ_GATE, PROJ_UP) else (wl.H, wl.I)


def nvfp4_source_weights(wl, expert, proj):
    """fp32 ~ N(0, 0.02) weights [n, kin] of one projection of one expert,
    before NVFP4 quantization (W_gate, W_up: [I, H]; W_down: [H, I])."""
    n, kin = proj_shape(wl, proj)
    z = rng(wl.weight_cfg, KIND_W, expert, proj).standard_normal((n, kin),
                                                                 dtype=np.float32)
    return z * np.float32(0.02)


def rot_sign_len(wl, side):
    return wl.H if side in (ROT_IN13, ROT_OUT2) else wl.I


def rot_signs(wl, expert, side):
    """The random signs (+1 / -1, int8) of one side of a rotated expert's
    matrices (ROT_IN13: the gate/up input, shared by both; ROT_OUT_GATE,
    ROT_OUT_UP; ROT_IN2, ROT_OUT2: the down projection's input and output)."""
    g = rng(wl.cfg, KIND_ROT_SIGNS, expert, side)
    return np.where(g.random(rot_sign_len(wl, side)) < 0.5, -1, 1).astype(np.int8)


def bf16_weights(wl, expert, proj):
    """Routed BF16-tier weights: the same N(0, 0.02) source weights as the
    NVFP4 tier, rounded to bf16 (nearest even), as uint16 bits."""
    return f32_to_bf16_bits(nvfp4_source_weights(wl, expert, proj))


def vq_codes(wl, expert, proj):
    """Uniform uint16 codes [n, kin/8] of one projection of one expert."""
    n, kin = proj_shape(wl, proj)
    return rng(wl.vq_cfg, KIND_VQ_CODES, expert, proj).integers(
        0, 65536, size=(n, kin // 8), dtype=np.uint16)


def vq_scales(wl, expert, proj):
    """fp16 per-output-channel scales ~ U(0.5, 1.5), as uint16 bits [n]."""
    n, _ = proj_shape(wl, proj)
    s = rng(wl.vq_cfg, KIND_VQ_SCALES, expert, proj).uniform(0.5, 1.5, size=n)
    return f32_to_f16_bits(s.astype(np.float32))


def vq_codebook(wl, proj, ncode=65536):
    """One fp16 codebook [ncode, 8] per projection type, shared by all the
    layer's experts; entries ~ N(0, 0.02); uint16 bits."""
    c = rng(wl.vq_cfg, KIND_VQ_CODEBOOK, 0, proj).standard_normal(
        (ncode, 8), dtype=np.float32) * np.float32(0.02)
    return f32_to_f16_bits(c)


def vq_codebook_expert(wl, expert, proj, ncode=65536):
    """An fp16 codebook [ncode, 8] of one expert's projection (the per-expert
    codebook variant); entries ~ N(0, 0.02); uint16 bits."""
    c = rng(wl.vq_cfg, KIND_VQ_CODEBOOK_EXPERT, expert, proj).standard_normal(
        (ncode, 8), dtype=np.float32) * np.float32(0.02)
    return f32_to_f16_bits(c)


def shared_weights_bf16(wl, proj):
    """The layer's BF16 shared expert: fp32 N(0, 0.02) rounded to bf16 (nearest
    even), as uint16 bits (W_gate, W_up: [I, H]; W_down: [H, I])."""
    n, kin = proj_shape(wl, proj)
    z = rng(wl.cfg, KIND_SHARED, 0, proj).standard_normal((n, kin), dtype=np.float32)
    return f32_to_bf16_bits(z * np.float32(0.02))


def vq8_rate(wl, expert):
    """Codes per 8-weight group of a small-codebook VQ expert: its explicit
    rate in a mixed-rate layer, else the layer's vq8_m."""
    if wl.fmt == "vqmix":
        return int(tier_map(wl)[expert]) - FMT_VQ8_M1 + 1
    return wl.vq8_m


def vq8_codes(wl, expert, proj):
    """Uniform uint8 codes [n, kin/8, M] of one projection of one expert
    (small-codebook VQ, M = the expert's codes per 8-weight group)."""
    n, kin = proj_shape(wl, proj)
    return rng(wl.vq_cfg, KIND_VQ8_CODES, expert, proj).integers(
        0, 256, size=(n, kin // 8, vq8_rate(wl, expert)), dtype=np.uint8)


def vq8_codebooks(wl, proj):
    """The fp16 codebooks [256, 8] of one projection type, shared by all the
    layer's experts: M = wl.vq8_m of them (an expert at rate m reads the first
    m); entries ~ N(0, 0.02 / sqrt(M)) so that a summed row has the spread of
    the 2-bit codebook's (N(0, 0.02 / sqrt(2)) in a mixed-rate layer, the
    middle rate's); uint16 bits."""
    M = wl.vq8_m
    sd = 0.02 / np.sqrt(2 if wl.fmt == "vqmix" else M)
    out = []
    for m in range(M):
        c = rng(wl.vq_cfg, KIND_VQ8_CODEBOOK, m, proj).standard_normal(
            (256, 8), dtype=np.float32) * np.float32(sd)
        out.append(f32_to_f16_bits(c))
    return out


def tier_map_hot(wl):
    """The mixed layer's tier map with its hot experts at the high tier: the
    n_hot hot experts and a seeded choice of n_nvfp4 - n_hot others are NVFP4,
    the rest VQ (the 4-bit tier goes to the experts that take most tokens)."""
    hot = hot_experts(wl)
    rest = np.setdiff1d(np.arange(wl.E), hot)
    others = rng(wl.cfg, KIND_TIER, 1).choice(rest, size=wl.n_nvfp4 - len(hot), replace=False)
    tm = np.full(wl.E, FMT_VQ, dtype=np.uint8)
    tm[hot] = FMT_NVFP4
    tm[others] = FMT_NVFP4
    return tm


def tier_map(wl):
    """Per-expert format tag (FMT_NVFP4 / FMT_VQ / FMT_VQ8 / FMT_BF16 /
    FMT_NVFP4R), uint8 [E]."""
    if wl.fmt == "nvfp4":
        return np.full(wl.E, FMT_NVFP4, dtype=np.uint8)
    if wl.fmt == "bf16":
        return np.full(wl.E, FMT_BF16, dtype=np.uint8)
    if wl.fmt == "nv_bf16":
        tm = np.full(wl.E, FMT_BF16, dtype=np.uint8)
        tm[rng(wl.cfg, KIND_TIER).choice(wl.E, size=wl.n_nvfp4, replace=False)] = FMT_NVFP4
        return tm
    if wl.fmt == "vq":
        return np.full(wl.E, FMT_VQ, dtype=np.uint8)
    if wl.fmt == "vq8":
        return np.full(wl.E, FMT_VQ8, dtype=np.uint8)
    if wl.fmt == "vqmix":
        # rates 1, 2, 3 over a seeded permutation of the experts, in the
        # proportions of the page's module counts (largest remainders)
        share = np.array(VQ8_RATE_COUNTS, np.float64) / sum(VQ8_RATE_COUNTS)
        n = np.floor(share * wl.E).astype(np.int64)
        rem = share * wl.E - n
        n[np.argsort(-rem, kind="stable")[: wl.E - int(n.sum())]] += 1
        perm = rng(wl.cfg, KIND_TIER).permutation(wl.E)
        tm = np.empty(wl.E, dtype=np.uint8)
        tm[perm[: n[0]]] = FMT_VQ8_M1
        tm[perm[n[0]: n[0] + n[1]]] = FMT_VQ8_M2
        tm[perm[n[0] + n[1]:]] = FMT_VQ8_M3
        return tm
    if wl.fmt == "nested":
        # the hot experts (or n_nvfp4 seeded ones) on the two-level tier
        tm = np.full(wl.E, FMT_NVFP4, dtype=np.uint8)
        up = (hot_experts(wl) if wl.n_hot
              else rng(wl.cfg, KIND_TIER).choice(wl.E, size=wl.n_nvfp4, replace=False))
        tm[up] = FMT_NVFP4R
        return tm
    g = rng(wl.cfg, KIND_TIER)
    tm = np.full(wl.E, FMT_VQ, dtype=np.uint8)
    nv = g.choice(wl.E, size=wl.n_nvfp4, replace=False)
    tm[nv] = FMT_NVFP4
    if wl.fmt == "mixed3":
        # half of the remaining experts take the small-codebook VQ
        rest = np.flatnonzero(tm == FMT_VQ)
        tm[g.choice(rest, size=len(rest) // 2, replace=False)] = FMT_VQ8
    return tm
