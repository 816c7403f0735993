"""Oracle: number formats of the expert weights (decode and the NVFP4 encoder).

TEST INFRASTRUCTURE ONLY -- see oracle/__init__.py.  numpy, float64.

NVFP4 (GLM-5-NVFP4-MTP, "Model Description": 4-bit weights with blockwise FP8
scales per 16 elements) is read as:
  * element codes in FP4 E2M1 (1 sign bit, 2 exponent bits with bias 1,
    1 mantissa bit; exponent field 0 is subnormal) -- the OCP Microscaling
    (MX) v1.0 FP4 element type;
  * one scale per 16 contiguous input elements of an output row, stored in
    FP8 E4M3 as defined by the OCP 8-bit floating point spec (E4M3FN: bias 7,
    subnormals, no infinities, S.1111.111 is NaN, max 448);
  * encoder: scale = amax/6 rounded to nearest-even E4M3, then each element
    rounded to the nearest E2M1 magnitude (ties to even mantissa), saturating
    at 6; a zero scale makes every code zero; no negative zero is emitted.

AQLM-style VQ (GLM-5.2 mixed-bit VQ (AQLM) ~1.90 bpw, "What it is":
per-group codes into a shared codebook) is read as: groups of 8 consecutive
input weights, one uint16 code per group indexing a 65536 x 8 fp16 codebook,
and one fp16 scale per output channel: W[o, 8g+j] = S[o] * C[code[o, g], j].

The small-codebook VQ modules (the same page and section: the build mixes
modules of 1, 2 and 3 bits per weight, each coded as per-group indices into a
codebook that the experts share) are read as groups of 8 input weights with
M = 1, 2 or 3 uint8 codes each, code m indexing a 256 x 8 fp16 codebook C_m
shared by the layer's experts, the rows summed (additive codebooks, as in
AQLM): W[o, 8g+j] = S[o] * sum_m C_m[code[o, g, m], j].  M codes per group
are M bits per weight.  The pages do not give these code shapes; they are
this reading's.
"""

import numpy as np


# --------------------------------------------------------------------------
# raw bit helpers (reading stored 16-bit floats; no rounding involved)
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64, exactly (bf16 is the top half
    of an IEEE binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits):
    """IEEE binary16 bit patterns (uint16) -> float64, exactly."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# --------------------------------------------------------------------------
# FP4 E2M1
# --------------------------------------------------------------------------

def e2m1_decode(codes):
    """Decode 4-bit E2M1 codes (0..15) to float64.

    Bit layout s.ee.m, exponent bias 1.  Exponent field 0 is subnormal:
    value = (-1)^s * m * 2^(1-1) * 0.5; otherwise (-1)^s * 2^(e-1) * (1 + m/2).
    (Element type of NVFP4; GLM-5-NVFP4-MTP, "Model Description".)
    """
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 15)):
        raise ValueError("E2M1 code out of range")
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    sub = m * 0.5
    nrm = np.ldexp(1.0 + m / 2.0, e - 1)
    mag = np.where(e == 0, sub, nrm)
    return np.where(s == 1, -mag, mag).astype(np.float64)


# magnitudes of the 8 non-negative codes, indexed by the 3 magnitude bits
E2M1_MAGNITUDES = e2m1_decode(np.arange(8))


# --------------------------------------------------------------------------
# FP8 E4M3 (OCP E4M3FN)
# --------------------------------------------------------------------------

def e4m3_decode(b):
    """Decode FP8 E4M3FN bytes to float64 (NaN for S.1111.111).

    s = b>>7, e = (b>>3)&15, m = b&7.  e == 0: (-1)^s * m * 2^-9 (subnormal);
    otherwise (-1)^s * (1 + m/8) * 2^(e-7).  Block-scale type of NVFP4
    (GLM-5-NVFP4-MTP, "Model Description": FP8 scales).
    """
    b = np.asarray(b).astype(np.int64)
    if np.any((b < 0) | (b > 255)):
        raise ValueError("E4M3 byte out of range")
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    sub = np.ldexp(m.astype(np.float64), -9)
    nrm = np.ldexp(1.0 + m / 8.0, e - 7)
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(np.float64)


def e4m3_finite_table():
    """The 127 finite non-negative E4M3 values, indexed by their byte 0..126
    (ascending: for non-negative E4M3 the byte order is the value order)."""
    return e4m3_decode(np.arange(127))


def e4m3_encode(v):
    """Round non-negative float64 values to E4M3 bytes: nearest finite value,
    ties to the even byte (= even mantissa), values above 448 saturate to 448.

    Written as a brute-force search over all 127 non-negative finite values.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(v < 0):
        raise ValueError("e4m3_encode takes finite, non-negative values")
    table = e4m3_finite_table()
    flat = v.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    codes = np.arange(127)
    chunk = 1 << 15
    for s in range(0, flat.size, chunk):
        x = flat[s:s + chunk, None]
        d = np.abs(x - table[None, :])
        out[s:s + chunk] = _nearest_even(d, codes)
    return out.reshape(v.shape)


def _nearest_even(dist, idx):
    """Per row of `dist`, the index with the smallest distance; on a tie the
    even index wins (the two tied candidates are neighbours, one even)."""
    dmin = dist.min(axis=1, keepdims=True)
    cand = dist == dmin
    even = cand & (idx[None, :] % 2 == 0)
    has_even = even.any(axis=1)
    pick_even = np.argmax(even, axis=1)
    pick_any = np.argmax(cand, axis=1)
    return np.where(has_even, pick_even, pick_any)


# --------------------------------------------------------------------------
# NVFP4 encode / decode
# --------------------------------------------------------------------------

def nvfp4_quantize(w):
    """Quantize an fp32 matrix w [n, kin] (kin % 16 == 0) to NVFP4.

    Per output row and per block of 16 contiguous input elements:
      amax = max |w|;  S = E4M3(amax / 6)  (division in float64);
      S == 0  -> every code in the block is 0;
      else code magnitude m = argmin_m | |w|/S - mag[m] |, ties -> even m,
      above 6 -> 6; sign bit = (w < 0 and m != 0).
    Returns canonical bytes: codes uint8 [n, kin/2] (element 2i in the low
    nibble of byte i) and scales uint8 [n, kin/16].
    (GLM-5-NVFP4-MTP, "Model Description".)
    """
    w = np.asarray(w)
    if w.ndim != 2 or w.shape[1] % 16 != 0:
        raise ValueError("w must be [n, kin] with kin % 16 == 0")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    n, kin = w.shape
    w64 = w.astype(np.float64)
    blocks = w64.reshape(n, kin // 16, 16)
    amax = np.abs(blocks).max(axis=2)
    scale_b = e4m3_encode(amax / 6.0)
    S = e4m3_decode(scale_b)

    mags = E2M1_MAGNITUDES
    midx = np.arange(8)
    a = np.abs(blocks)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(S[:, :, None] > 0, a / np.where(S > 0, S, 1.0)[:, :, None], 0.0)
    rf = r.reshape(-1)
    m = np.empty(rf.shape, dtype=np.int64)
    chunk = 1 << 18
    for s in range(0, rf.size, chunk):
        d = np.abs(rf[s:s + chunk, None] - mags[None, :])
        m[s:s + chunk] = _nearest_even(d, midx)
    m = m.reshape(blocks.shape)
    m = np.where(S[:, :, None] > 0, m, 0)
    sign = (blocks < 0) & (m != 0)
    code = (m | (sign.astype(np.int64) << 3)).reshape(n, kin)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale_b.astype(np.uint8)


def nvfp4_unpack_codes(codes):
    """Canonical packed codes [n, kin/2] -> 4-bit codes [n, kin]."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty((c.shape[0], c.shape[1] * 2), dtype=np.int64)
    out[:, 0::2] = c & 0xF
    out[:, 1::2] = c >> 4
    return out


def nvfp4_dequant(codes, scales):
    """W[o, k] = E2M1(code[o, k]) * E4M3(scale[o, k // 16]) in float64."""
    c = nvfp4_unpack_codes(codes)
    n, kin = c.shape
    s = e4m3_decode(np.asarray(scales, dtype=np.uint8))
    if s.shape != (n, kin // 16):
        raise ValueError("scale shape mismatch")
    return e2m1_decode(c) * np.repeat(s, 16, axis=1)


# --------------------------------------------------------------------------
# Nested two-level NVFP4 (a base plane plus a residual plane)
# --------------------------------------------------------------------------

def nvfp4_residual_quantize(w, shift):
    """The two planes of a nested two-level NVFP4 matrix.

    "GLM-5.3 Vision NestQuant 1.75-4 bit", introduction and Method: each
    expert has a base plus a residual plane that lifts it to the higher tier;
    the residual is coded on what the base leaves.  Reading (their base and
    residual are trellis codes; here both planes are NVFP4): base =
    nvfp4_quantize(w); residual = nvfp4_quantize(r) with r = (w - base value)
    * 2^shift, exact in float64 and rounded once to fp32.  The power of two
    brings the residual's small block maxima into the normal range of the
    E4M3 scales (without it most of them round to a zero scale).  Returns
    ((base codes, base scales), (residual codes, residual scales)).
    """
    w = np.asarray(w, dtype=np.float32)
    if not 0 <= shift <= 14:
        raise ValueError("shift must be in [0, 14]")
    bc, bs = nvfp4_quantize(w)
    r = np.ldexp(w.astype(np.float64) - nvfp4_dequant(bc, bs), shift).astype(np.float32)
    rc, rs = nvfp4_quantize(r)
    return (bc, bs), (rc, rs)


def nvfp4r_dequant(base, res, shift):
    """W = base value + residual value * 2^-shift (NVFP4 decodes), float64."""
    return nvfp4_dequant(*base) + np.ldexp(nvfp4_dequant(*res), -shift)


# --------------------------------------------------------------------------
# AQLM-style VQ decode
# --------------------------------------------------------------------------

def vq_dequant(codes, scales_f16, codebook_f16):
    """W[o, 8g + j] = S[o] * C[code[o, g], j] in float64.

    codes uint16 [n, kin/8]; scales_f16 uint16 bits [n]; codebook_f16 uint16
    bits [ncode, 8].  (GLM-5.2 mixed-bit VQ (AQLM) ~1.90 bpw, "What it is".)
    """
    codes = np.asarray(codes, dtype=np.uint16)
    C = f16_bits_to_f64(np.asarray(codebook_f16, dtype=np.uint16))
    S = f16_bits_to_f64(np.asarray(scales_f16, dtype=np.uint16))
    n, g = codes.shape
    if C.ndim != 2 or C.shape[1] != 8:
        raise ValueError("codebook must be [ncode, 8]")
    if S.shape != (n,):
        raise ValueError("scale shape mismatch")
    rows = C[codes.astype(np.int64)]          # [n, g, 8]
    return (S[:, None, None] * rows).reshape(n, g * 8)


def vq8_dequant(codes, scales_f16, codebooks_f16):
    """W[o, 8g + j] = S[o] * sum_m C_m[code[o, g, m], j] in float64.

    codes uint8 [n, kin/8, M]; scales_f16 uint16 bits [n]; codebooks_f16: M
    arrays of uint16 bits [256, 8] (C_0, C_1, ...).  The sum of the M fp16
    rows is exact in float64; the product with S rounds once (float64).
    (GLM-5.2 mixed-bit VQ (AQLM) ~1.90 bpw, "What it is": 1/2/3-bit modules
    with per-group codes and shared codebooks; the M x 8-bit code shape is a
    reading, see the module docstring.)
    """
    codes = np.asarray(codes, dtype=np.uint8)
    S = f16_bits_to_f64(np.asarray(scales_f16, dtype=np.uint16))
    if codes.ndim != 3:
        raise ValueError("codes must be [n, kin/8, M]")
    n, g, M = codes.shape
    if len(codebooks_f16) != M:
        raise ValueError("one codebook per code of a group")
    if S.shape != (n,):
        raise ValueError("scale shape mismatch")
    acc = np.zeros((n, g, 8), dtype=np.float64)
    for m in range(M):
        C = f16_bits_to_f64(np.asarray(codebooks_f16[m], dtype=np.uint16))
        if C.shape != (256, 8):
            raise ValueError("codebook must be [256, 8]")
        acc += C[codes[:, :, m].astype(np.int64)]
    return (S[:, None, None] * acc).reshape(n, g * 8)


def vq8_rate_dequant(codes, scales_f16, layer_codebooks_f16):
    """An expert of rate m in a layer of small-codebook VQ experts at mixed
    rates: W[o, 8g + j] = S[o] * sum_{i<m} C_i[code[o, g, i], j], with m =
    codes.shape[2] (1, 2 or 3 codes per group, m bits per weight) and C_i the
    i-th of the layer's codebooks for this projection.

    (GLM-5.2 mixed-bit VQ (AQLM) ~1.90 bpw, "What it is": one layer's modules
    run at 1, 2 and 3 bits, chosen per module by a loss-aware allocation,
    each indexing shared codebooks.)  Reading: the layer keeps up to three
    256 x 8 codebooks per projection, shared by every expert of the layer,
    and an expert at rate m uses the first m of them; rates are per expert
    (all three projections of an expert at one rate).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.ndim != 3 or not 1 <= codes.shape[2] <= 3:
        raise ValueError("codes must be [n, kin/8, m] with m = 1, 2 or 3")
    m = codes.shape[2]
    if len(layer_codebooks_f16) < m:
        raise ValueError("the layer holds fewer codebooks than the expert's rate")
    return vq8_dequant(codes, scales_f16, list(layer_codebooks_f16)[:m])

