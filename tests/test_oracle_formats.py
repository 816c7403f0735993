"""Pins of the oracle's format code (E2M1, E4M3, NVFP4 encoder, VQ decode)
against facts fixed outside the oracle: published value tables, a library
cast, hand-worked blocks, brute force and closed forms; the 16-bit float
widening of activations, codebooks and scales.  CPU only."""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import nvfp4_unpack_codes


def _read_table(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


# ------------------------------------------------- 16-bit activations
#
# The oracle widens every bf16 activation (and fp16 codebook entry / scale)
# with bf16_bits_to_f64 / f16_bits_to_f64.  Both are pinned over all 65,536
# bit patterns against (a) torch's own bfloat16 / float16 types and (b) the
# IEEE field decode written out here: sign, biased exponent, fraction, with
# exponent field 0 subnormal and the all-ones field infinity (fraction 0) or
# NaN.  bf16 = 1 + 8 + 7 bits, bias 127 (the top half of a binary32); fp16 =
# 1 + 5 + 10 bits, bias 15.


def _ieee_fields_decode(bits, ebits, fbits):
    bits = np.asarray(bits, dtype=np.int64)
    bias = (1 << (ebits - 1)) - 1
    s = (bits >> (ebits + fbits)) & 1
    e = (bits >> fbits) & ((1 << ebits) - 1)
    f = bits & ((1 << fbits) - 1)
    emax = (1 << ebits) - 1
    mag = np.where(e == 0, np.ldexp(f.astype(np.float64), 1 - bias - fbits),
                   np.ldexp((f + (1 << fbits)).astype(np.float64), e - bias - fbits))
    mag = np.where((e == emax) & (f == 0), np.inf, mag)
    mag = np.where((e == emax) & (f != 0), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _same_f64(got, want):
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_bf16_widening_all_patterns_vs_torch_and_fields():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    ref_t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    _same_f64(got, ref_t)
    _same_f64(got, _ieee_fields_decode(bits, 8, 7))
    # named points: 1.0, -2.0, the smallest subnormal, the largest finite, +-inf
    named = {0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133,
             0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127, 0x7F80: np.inf, 0xFF80: -np.inf}
    for b, v in named.items():
        assert oracle.bf16_bits_to_f64(np.uint16(b)) == v, hex(b)
    assert np.signbit(oracle.bf16_bits_to_f64(np.uint16(0x8000)))


def test_f16_widening_all_patterns_vs_torch_and_fields():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_bits_to_f64(bits)
    ref_t = torch.from_numpy(bits.view(np.int16)).view(torch.float16).double().numpy()
    _same_f64(got, ref_t)
    _same_f64(got, _ieee_fields_decode(bits, 5, 10))
    named = {0x3C00: 1.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24, 0x0400: 2.0 ** -14,
             0xFC00: -np.inf}
    for b, v in named.items():
        assert oracle.f16_bits_to_f64(np.uint16(b)) == v, hex(b)


# ---------------------------------------------------------------- E2M1

def test_e2m1_value_set_matches_published_table(golden_dir):
    rows = _read_table(os.path.join(golden_dir, "e2m1_values.txt"))
    assert len(rows) == 16
    for code, val in rows:
        got = oracle.e2m1_decode(int(code))
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def test_e2m1_sign_symmetry_and_monotone():
    v = oracle.e2m1_decode(np.arange(16))
    assert np.array_equal(v[8:], -v[:8])
    assert np.all(np.diff(v[:8]) > 0)
    assert np.array_equal(oracle.E2M1_MAGNITUDES, v[:8])


# ---------------------------------------------------------------- E4M3

def test_e4m3_named_values(golden_dir):
    for hx, val in _read_table(os.path.join(golden_dir, "e4m3_facts.txt")):
        got = float(oracle.e4m3_decode(int(hx, 16)))
        if val == "nan":
            assert math.isnan(got), hx
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), hx


def test_e4m3_decode_exhaustive_vs_torch_cast():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_e4m3_encode_roundtrip_all_finite_nonneg():
    b = np.arange(127)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(b)), b)


def test_e4m3_encode_midpoints_go_to_even():
    t = oracle.e4m3_finite_table()
    mids = (t[:-1] + t[1:]) / 2
    enc = oracle.e4m3_encode(mids)
    lo = np.arange(126)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(enc, want)
    # just above / below a midpoint goes to the nearer neighbour
    assert np.array_equal(oracle.e4m3_encode(np.nextafter(mids, np.inf)), lo + 1)
    assert np.array_equal(oracle.e4m3_encode(np.nextafter(mids, -np.inf)), lo)


def test_e4m3_encode_edges():
    assert oracle.e4m3_encode(2.0 ** -10) == 0            # tie 0 | 2^-9 -> even (0)
    assert oracle.e4m3_encode(np.nextafter(2.0 ** -10, 1)) == 1
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(463.9) == 0x7E
    assert oracle.e4m3_encode(1e6) == 0x7E                 # saturate
    assert oracle.e4m3_encode(0.0) == 0


def test_e4m3_encode_vs_torch_cast_random():
    rs = np.random.default_rng(1)
    v = np.concatenate([
        rs.uniform(0, 448, 20000),
        np.exp(rs.uniform(np.log(2.0 ** -12), np.log(448.0), 20000)),
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(v.astype(np.float64))
    assert np.array_equal(ref, got)


# ---------------------------------------------------------------- NVFP4

def _handworked(golden_dir):
    out = []
    with open(os.path.join(golden_dir, "nvfp4_handworked.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, vals, sb, cb = [p.strip() for p in line.split("|")]
            v = [float.fromhex(t) if "0x" in t else float(t) for t in vals.split()]
            out.append((name, np.array(v, dtype=np.float32), int(sb, 16),
                        [int(c, 16) for c in cb.split()]))
    return out


def test_nvfp4_handworked_blocks(golden_dir):
    blocks = _handworked(golden_dir)
    assert len(blocks) == 7
    for name, v, sb, cb in blocks:
        assert np.all(v.astype(np.float64) == v)  # fixture values are fp32-exact or fp32-rounded
        codes, scales = oracle.nvfp4_quantize(v[None, :])
        assert scales[0, 0] == sb, (name, hex(scales[0, 0]))
        assert list(codes[0]) == cb, (name, [hex(c) for c in codes[0]])
    # the same blocks side by side in one row, and stacked in rows
    V = np.concatenate([b[1] for b in blocks])[None, :]
    codes, scales = oracle.nvfp4_quantize(V)
    assert list(scales[0]) == [b[2] for b in blocks]
    assert list(codes[0]) == sum((b[3] for b in blocks), [])
    codes2, scales2 = oracle.nvfp4_quantize(np.stack([b[1] for b in blocks]))
    assert list(scales2[:, 0]) == [b[2] for b in blocks]


def _brute_force_check(w, codes, scales):
    """Every element's code is a nearest E2M1 value times S (among all 16
    codes), ties to an even mantissa, no negative zero; the scale is a nearest
    E4M3 value to amax/6 (among all 127), ties to even."""
    n, kin = w.shape
    table = oracle.e4m3_finite_table()
    vals16 = oracle.e2m1_decode(np.arange(16))
    c = nvfp4_unpack_codes(codes)
    for o in range(n):
        for b in range(kin // 16):
            blk = w[o, 16 * b:16 * b + 16].astype(np.float64)
            t = np.abs(blk).max() / 6.0
            d = np.abs(table - t)
            best = np.nonzero(d == d.min())[0]
            sb = int(scales[o, b])
            assert sb in best
            if len(best) == 2:
                assert sb % 2 == 0
            S = table[sb]
            for i in range(16):
                code = int(c[o, 16 * b + i])
                if S == 0:
                    assert code == 0
                    continue
                err = np.abs(blk[i] - vals16 * S)
                cands = np.nonzero(err == err.min())[0]
                assert code in cands, (o, b, i, blk[i], S, code, cands)
                mags = set(int(x) & 7 for x in cands)
                if len(mags) == 2:
                    assert (code & 7) % 2 == 0
                if code & 7 == 0:
                    assert code == 0      # no negative zero


def test_nvfp4_brute_force_random_blocks():
    rs = np.random.default_rng(7)
    w = (rs.standard_normal((24, 256)) * 0.02).astype(np.float32)
    # crafted rows: exact midpoints times S, a lone nonzero, tiny blocks
    w[0, :16] = np.float32(2.0 ** -7) * np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5,
                                                   -6, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5],
                                                  dtype=np.float32)
    w[1, :16] = 0
    w[1, 16:32] = 0
    w[1, 20] = np.float32(-0.013)
    w[2, :16] = np.float32(1e-4) * rs.standard_normal(16).astype(np.float32)
    w[3, :] = np.float32(100.0) * rs.standard_normal(256).astype(np.float32)
    codes, scales = oracle.nvfp4_quantize(w)
    _brute_force_check(w, codes, scales)


def test_nvfp4_error_bound_invariant():
    rs = np.random.default_rng(11)
    w = (rs.standard_normal((64, 512)) * 0.02).astype(np.float32)
    codes, scales = oracle.nvfp4_quantize(w)
    deq = oracle.nvfp4_dequant(codes, scales)
    S = np.repeat(oracle.e4m3_decode(scales), 16, axis=1)
    mags = oracle.E2M1_MAGNITUDES
    halfgap = np.max(np.diff(mags)) / 2         # 1.0 (between 4 and 6)
    a = np.abs(w.astype(np.float64))
    sat = a > 6 * S
    err = np.abs(w - deq)
    assert np.all(err[~sat] <= halfgap * S[~sat] + 0)
    # saturated elements decode to +-6 S
    assert np.all(np.abs(deq[sat]) == 6 * S[sat])
    # sign agreement wherever the decoded value is nonzero
    nz = deq != 0
    assert np.all(np.sign(deq[nz]) == np.sign(w[nz]))


# ---------------------------------------------------- nested two-level NVFP4

def test_nvfp4r_representable_matrix_has_zero_residual():
    """A matrix of NVFP4 values whose every block holds a +-6 code (so its
    scale is recovered exactly) is its own base: the residual plane is all
    zero codes and zero scales, and the two-level value is the matrix."""
    rs = np.random.default_rng(21)
    n, kin = 8, 64
    codes = rs.integers(0, 16, size=(n, kin)).astype(np.uint8)
    codes[:, ::16] = 7                                   # a +6 in every block
    sb = rs.integers(0x20, 0x60, size=(n, kin // 16)).astype(np.uint8)   # normal E4M3
    w = oracle.e2m1_decode(codes) * np.repeat(oracle.e4m3_decode(sb), 16, axis=1)
    assert np.all(w.astype(np.float32) == w)
    for shift in (0, 8):
        (bc, bs), (rc, rscale) = oracle.nvfp4_residual_quantize(w.astype(np.float32), shift)
        assert np.array_equal(oracle.nvfp4_dequant(bc, bs), w)
        assert np.all(rc == 0) and np.all(rscale == 0)
        assert np.array_equal(oracle.nvfp4r_dequant((bc, bs), (rc, rscale), shift), w)


def test_nvfp4r_error_bound_and_nesting():
    """The base plane is the plain NVFP4 quantization (the nested tier's
    bytes), and the two-level error obeys the NVFP4 bound on the residual:
    with S the residual block's E4M3 scale and a its largest |r|, an element
    not past 6 S is within S (half the widest E2M1 gap) of r, one past it
    within |r| - 6 S; scaled back by 2^-shift, plus r's fp32 rounding."""
    rs = np.random.default_rng(22)
    w = (rs.standard_normal((32, 512)) * 0.02).astype(np.float32)
    shift = 8
    (bc, bs), (rc, rsc) = oracle.nvfp4_residual_quantize(w, shift)
    c0, s0 = oracle.nvfp4_quantize(w)
    assert np.array_equal(bc, c0) and np.array_equal(bs, s0)
    base = oracle.nvfp4_dequant(bc, bs)
    r64 = np.ldexp(w.astype(np.float64) - base, shift)
    r = r64.astype(np.float32).astype(np.float64)
    S = np.repeat(oracle.e4m3_decode(rsc), 16, axis=1)
    q = oracle.nvfp4_dequant(rc, rsc)
    sat = np.abs(r) > 6 * S
    err = np.abs(r - q)
    assert np.all(err[~sat] <= S[~sat])
    assert np.all(err[sat] <= np.abs(r[sat]) - 6 * S[sat] + 1e-30)
    two = oracle.nvfp4r_dequant((bc, bs), (rc, rsc), shift)
    bound = np.ldexp(np.where(sat, np.abs(r) - 6 * S, S) + np.abs(r64 - r), -shift)
    assert np.all(np.abs(w - two) <= bound * (1 + 1e-12))
    # the residual plane cuts the error of N(0, 0.02) weights by an order of
    # magnitude (its scales are in E4M3's normal range at this shift)
    assert np.sqrt(np.mean((w - two) ** 2)) < np.sqrt(np.mean((w - base) ** 2)) / 8


def test_nvfp4r_shift_zero_loses_small_residuals():
    """Without the power of two the residual's block maxima fall below the
    smallest E4M3 scale and most residual blocks get scale 0 (why the layer
    carries an exponent for the residual plane)."""
    rs = np.random.default_rng(23)
    w = (rs.standard_normal((16, 256)) * 0.02).astype(np.float32)
    (_, _), (_, rsc0) = oracle.nvfp4_residual_quantize(w, 0)
    (_, _), (_, rsc8) = oracle.nvfp4_residual_quantize(w, 8)
    assert np.mean(rsc0 == 0) > 0.5 and np.all(rsc8 != 0)
    with pytest.raises(ValueError):
        oracle.nvfp4_residual_quantize(w, 15)


def test_nvfp4_zero_blocks_and_zero_scale():
    w = np.zeros((2, 32), dtype=np.float32)
    w[1, 16:] = np.float32(3 * 2.0 ** -11)   # amax/6 = 2^-12 -> scale 0 -> all codes 0
    codes, scales = oracle.nvfp4_quantize(w)
    assert np.all(codes == 0) and np.all(scales == 0)
    assert np.all(oracle.nvfp4_dequant(codes, scales) == 0)


def test_nvfp4_products_exact_in_bf16_and_f16():
    vals = oracle.e2m1_decode(np.arange(16))
    sc = oracle.e4m3_finite_table()
    prod = (vals[:, None] * sc[None, :]).reshape(-1)
    as32 = prod.astype(np.float32)
    assert np.array_equal(as32.astype(np.float64), prod)
    bf = torch.from_numpy(as32).to(torch.bfloat16).to(torch.float64).numpy()
    f16 = torch.from_numpy(as32).to(torch.float16).to(torch.float64).numpy()
    assert np.array_equal(bf, prod)
    assert np.array_equal(f16, prod)


def test_nvfp4_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.nvfp4_quantize(np.zeros((2, 24), np.float32))
    w = np.zeros((1, 16), np.float32)
    w[0, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.nvfp4_quantize(w)


# ---------------------------------------------------------------- VQ

def _f16(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def test_vq_codebook_identity_recovers_codes():
    ncode = 65536
    c = np.arange(ncode)
    cb = np.zeros((ncode, 8), dtype=np.float64)
    cb[:, 0] = c >> 8
    cb[:, 1] = c & 255
    cb[:, 2:] = np.arange(2, 8)[None, :]
    rs = np.random.default_rng(3)
    codes = rs.integers(0, ncode, size=(5, 12), dtype=np.uint16)
    W = oracle.vq_dequant(codes, _f16(np.ones(5)), _f16(cb))
    Wg = W.reshape(5, 12, 8)
    rec = (Wg[:, :, 0] * 256 + Wg[:, :, 1]).astype(np.int64)
    assert np.array_equal(rec, codes.astype(np.int64))
    assert np.all(Wg[:, :, 2:] == np.arange(2, 8)[None, None, :])


def test_vq_power_of_two_scales_shift_rows():
    rs = np.random.default_rng(5)
    cb = _f16(rs.standard_normal((256, 8)) * 0.02)
    codes = rs.integers(0, 256, size=(6, 4), dtype=np.uint16)
    p = np.array([-3, -1, 0, 1, 2, 5])
    W = oracle.vq_dequant(codes, _f16(2.0 ** p), cb)
    C = cb.view(np.float16).astype(np.float64)
    for o in range(6):
        for g in range(4):
            assert np.array_equal(W[o, 8 * g:8 * g + 8], np.ldexp(C[codes[o, g]], p[o]))


def test_vq_one_hot_codebook_rows():
    cb = np.zeros((16, 8))
    for r in range(16):
        cb[r, r % 8] = r + 1
    codes = np.array([[3, 11, 0]], dtype=np.uint16)
    W = oracle.vq_dequant(codes, _f16([0.5]), _f16(cb))
    want = np.zeros(24)
    want[0 + 3] = 2.0
    want[8 + 3] = 6.0
    want[16 + 0] = 0.5
    assert np.array_equal(W[0], want)


def test_vq_product_exact_in_fp32():
    rs = np.random.default_rng(9)
    cb = _f16(rs.standard_normal((4096, 8)) * 0.02)
    sc = _f16(rs.uniform(0.5, 1.5, 64))
    codes = rs.integers(0, 4096, size=(64, 32), dtype=np.uint16)
    W = oracle.vq_dequant(codes, sc, cb)
    assert np.array_equal(W.astype(np.float32).astype(np.float64), W)


# ------------------------------------------------------ small-codebook VQ

def test_vq8_identity_codebooks_recover_both_codes():
    # C_0[c] = 256 c and C_1[c] = c in every column (both exact in fp16):
    # the summed row is 256 c0 + c1, which gives back both codes
    c = np.arange(256, dtype=np.float64)
    cb0 = _f16(np.repeat((256 * c)[:, None], 8, axis=1))
    cb1 = _f16(np.repeat(c[:, None], 8, axis=1))
    rs = np.random.default_rng(11)
    codes = rs.integers(0, 256, size=(7, 9, 2), dtype=np.uint8)
    W = oracle.vq8_dequant(codes, _f16(np.ones(7)), [cb0, cb1]).reshape(7, 9, 8)
    v = W[:, :, 0].astype(np.int64)
    assert np.array_equal(v >> 8, codes[:, :, 0]) and np.array_equal(v & 255, codes[:, :, 1])
    assert np.all(W == W[:, :, :1])


def test_vq8_single_codebook_is_the_plain_lookup():
    # M = 1 is the 2-bit VQ decode restricted to a 256-entry codebook
    rs = np.random.default_rng(12)
    cb = _f16(rs.standard_normal((256, 8)) * 0.02)
    sc = _f16(rs.uniform(0.5, 1.5, 5))
    codes = rs.integers(0, 256, size=(5, 6, 1), dtype=np.uint8)
    W = oracle.vq8_dequant(codes, sc, [cb])
    assert np.array_equal(W, oracle.vq_dequant(codes[:, :, 0].astype(np.uint16), sc, cb))


def test_vq8_is_additive_over_codebooks():
    rs = np.random.default_rng(13)
    cbs = [_f16(rs.standard_normal((256, 8)) * 0.01) for _ in range(2)]
    codes = rs.integers(0, 256, size=(4, 5, 2), dtype=np.uint8)
    one = _f16(np.ones(4))
    W = oracle.vq8_dequant(codes, one, cbs)
    W0 = oracle.vq8_dequant(codes[:, :, :1], one, cbs[:1])
    W1 = oracle.vq8_dequant(codes[:, :, 1:], one, cbs[1:])
    assert np.array_equal(W, W0 + W1)   # fp16 rows of this range sum exactly


def test_vq8_one_hot_rows_and_power_of_two_scales():
    cb0 = np.zeros((256, 8))
    cb1 = np.zeros((256, 8))
    cb0[5, 2] = 3.0
    cb1[7, 6] = -1.5
    codes = np.array([[[5, 0], [0, 7], [5, 7]]], dtype=np.uint8)
    W = oracle.vq8_dequant(codes, _f16([4.0]), [_f16(cb0), _f16(cb1)])
    want = np.zeros(24)
    want[2] = 12.0
    want[8 + 6] = -6.0
    want[16 + 2], want[16 + 6] = 12.0, -6.0
    assert np.array_equal(W[0], want)


def test_vq8_rejects_bad_shapes():
    cb = _f16(np.zeros((256, 8)))
    with pytest.raises(ValueError):
        oracle.vq8_dequant(np.zeros((2, 3), np.uint8), _f16(np.ones(2)), [cb])
    with pytest.raises(ValueError):
        oracle.vq8_dequant(np.zeros((2, 3, 2), np.uint8), _f16(np.ones(2)), [cb])
    with pytest.raises(ValueError):
        oracle.vq8_dequant(np.zeros((2, 3, 1), np.uint8), _f16(np.ones(2)), [_f16(np.zeros((16, 8)))])


def test_vq8_three_codebooks_recover_all_codes():
    # the 3-bit module: C_0[c] = 256^2 c would overflow fp16, so use
    # C_0[c] = 16 c0, C_1[c] = c1 / 16 (c < 16 only: 4-bit codes in each), C_2
    # one-hot columns; the summed row gives back every code
    rs = np.random.default_rng(14)
    c = np.arange(256, dtype=np.float64)
    cb0 = _f16(np.repeat((16.0 * (c % 16))[:, None], 8, axis=1))
    cb1 = _f16(np.repeat(((c % 16) / 16.0)[:, None], 8, axis=1))
    cb2 = np.zeros((256, 8))
    for code in range(8):
        cb2[code, code] = 1024.0
    codes = np.stack([rs.integers(0, 16, size=(5, 6)), rs.integers(0, 16, size=(5, 6)),
                      rs.integers(0, 8, size=(5, 6))], axis=-1).astype(np.uint8)
    W = oracle.vq8_dequant(codes, _f16(np.ones(5)), [cb0, cb1, _f16(cb2)]).reshape(5, 6, 8)
    base = W.min(axis=2)                          # the column without the one-hot 1024
    assert np.array_equal(np.round(base // 16), codes[:, :, 0])
    assert np.array_equal(np.round((base % 16) * 16), codes[:, :, 1])
    assert np.array_equal(np.argmax(W, axis=2), codes[:, :, 2])
    # and it is the sum of the three single-codebook decodes
    one = _f16(np.ones(5))
    parts = [oracle.vq8_dequant(codes[:, :, j:j + 1], one, [cb][:1])
             for j, cb in enumerate([cb0, cb1, _f16(cb2)])]
    assert np.array_equal(W.reshape(5, 48), parts[0] + parts[1] + parts[2])


# ------------------------------------------- small-codebook VQ at mixed rates

def _rate_books(rs, scale=0.01):
    return [_f16(rs.standard_normal((256, 8)) * scale) for _ in range(3)]


def test_vq8_rate_uses_the_first_m_codebooks_only():
    """An expert at rate m reads codebooks 0..m-1 of the layer: changing the
    others leaves its weights unchanged, changing one it reads does not."""
    rs = np.random.default_rng(21)
    books = _rate_books(rs)
    other = _rate_books(rs)
    sc = _f16(rs.uniform(0.5, 1.5, 6))
    for m in (1, 2, 3):
        codes = rs.integers(0, 256, size=(6, 5, m), dtype=np.uint8)
        W = oracle.vq8_rate_dequant(codes, sc, books)
        swapped = books[:m] + other[m:]
        assert np.array_equal(W, oracle.vq8_rate_dequant(codes, sc, swapped)), m
        changed = list(books)
        changed[m - 1] = other[m - 1]
        assert not np.array_equal(W, oracle.vq8_rate_dequant(codes, sc, changed)), m


def test_vq8_rates_nest():
    """A rate-(m+1) expert is the rate-m expert of its first m codes plus the
    one-code lookup of its last code in codebook m (exact for these ranges)."""
    rs = np.random.default_rng(22)
    books = _rate_books(rs)
    one = _f16(np.ones(4))
    codes = rs.integers(0, 256, size=(4, 7, 3), dtype=np.uint8)
    for m in (1, 2):
        hi = oracle.vq8_rate_dequant(codes[:, :, :m + 1], one, books)
        lo = oracle.vq8_rate_dequant(codes[:, :, :m], one, books)
        last = oracle.vq8_dequant(codes[:, :, m:m + 1], one, [books[m]])
        assert np.array_equal(hi, lo + last), m


def test_vq8_rate_identity_codebooks_recover_codes():
    """Codebooks C_0[c] = 1024 (c % 16), C_1[c] = 32 (c % 16), C_2[c] = c % 16
    (every sum exact in fp16): each rate gives back all of its codes from the
    summed row, and a rate-1 expert is the plain lookup."""
    c = np.arange(256, dtype=np.float64) % 16
    books = [_f16(np.repeat((f * c)[:, None], 8, axis=1)) for f in (1024.0, 32.0, 1.0)]
    rs = np.random.default_rng(23)
    for m in (1, 2, 3):
        codes = rs.integers(0, 16, size=(5, 6, m), dtype=np.uint8)
        W = oracle.vq8_rate_dequant(codes, _f16(np.ones(5)), books).reshape(5, 6, 8)
        v = W[:, :, 0].astype(np.int64)
        for i, f in enumerate((1024, 32, 1)[:m]):
            assert np.array_equal((v // f) % 32 if f > 1 else v % 32, codes[:, :, i]), (m, i)
    cb = books[0]
    codes = rs.integers(0, 256, size=(3, 4, 1), dtype=np.uint8)
    sc = _f16([2.0, 0.5, 1.0])
    assert np.array_equal(oracle.vq8_rate_dequant(codes, sc, books),
                          oracle.vq_dequant(codes[:, :, 0].astype(np.uint16), sc, cb))


def test_vq8_rate_rejects_bad_rates():
    books = [_f16(np.zeros((256, 8)))] * 2
    with pytest.raises(ValueError):
        oracle.vq8_rate_dequant(np.zeros((2, 3, 3), np.uint8), _f16(np.ones(2)), books)
    with pytest.raises(ValueError):
        oracle.vq8_rate_dequant(np.zeros((2, 3, 4), np.uint8), _f16(np.ones(2)), books * 2)

