"""CPU tests of the C ABI library: it loads, exports every declared symbol,
its host packers match the oracle byte for byte, and its host-side argument
checks reject bad calls before any launch (no GPU is touched here)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import bit_quantized_moe_route_amd as moeq
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    txt = open(os.path.join(ROOT, "include", "moeq.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 14
    L = moeq.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", moeq.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    # the binding declares a prototype for every one of them
    assert set(names) == set(moeq._PROTOS)


def test_strerror():
    L = moeq.lib()
    for st in (0, -1, -2, -3, -4):
        assert L.moe_strerror(st)
    assert b"fail" in L.moe_strerror(-2) or b"unsupported" in L.moe_strerror(-2)


# ---------------------------------------------------------------- packers

@pytest.mark.parametrize("shape,seed", [((16, 256), 0), ((48, 6144), 1), ((96, 2048), 2),
                                        ((17, 32), 3)])
def test_quantize_nvfp4_matches_oracle(shape, seed):
    rs = np.random.default_rng(seed)
    w = (rs.standard_normal(shape) * 0.02).astype(np.float32)
    c, s = moeq.quantize_nvfp4(w)
    oc, os_ = oracle.nvfp4_quantize(w)
    assert np.array_equal(c, oc)
    assert np.array_equal(s, os_)


@pytest.mark.parametrize("shape,seed,shift", [((8, 64), 1, 8), ((48, 272), 2, 0), ((16, 128), 3, 14)])
def test_quantize_nvfp4_residual_matches_oracle(shape, seed, shift):
    """The library's two-plane quantizer (C) against the oracle's (numpy),
    byte for byte; its base plane is the plain NVFP4 quantization."""
    rs = np.random.default_rng(seed)
    w = (rs.standard_normal(shape) * 0.02).astype(np.float32)
    (bc, bs), (rc, rs_) = moeq.quantize_nvfp4_residual(w, shift)
    (obc, obs), (orc, ors) = oracle.nvfp4_residual_quantize(w, shift)
    for a, b in ((bc, obc), (bs, obs), (rc, orc), (rs_, ors)):
        assert np.array_equal(a, b)
    c, s = moeq.quantize_nvfp4(w)
    assert np.array_equal(bc, c) and np.array_equal(bs, s)
    with pytest.raises(moeq.MoeError):
        moeq.quantize_nvfp4_residual(w, 15)


def test_nvfp4r_record_layout():
    """A two-level record is the base plane's NVFP4 record followed by the
    residual plane's, each at the NVFP4 record size."""
    H, I = 272, 80
    rs = np.random.default_rng(4)
    parts = [moeq.quantize_nvfp4_residual((rs.standard_normal(sh) * 0.02).astype(np.float32))
             for sh in ((I, H), (I, H), (H, I))]
    base = [p[0] for p in parts]
    res = [p[1] for p in parts]
    w13, w2 = moeq.pack_nvfp4r_expert(base, res, H, I)
    n13, n2 = moeq.record_bytes(moeq.FMT_NVFP4, 0, H, I), moeq.record_bytes(moeq.FMT_NVFP4, 1, H, I)
    assert w13.shape[0] == 2 * n13 == moeq.record_bytes(moeq.FMT_NVFP4R, 0, H, I)
    assert w2.shape[0] == 2 * n2 == moeq.record_bytes(moeq.FMT_NVFP4R, 1, H, I)
    b13, b2 = moeq.pack_nvfp4_expert(*base, H, I)
    r13, r2 = moeq.pack_nvfp4_expert(*res, H, I)
    assert np.array_equal(w13[:n13], b13) and np.array_equal(w13[n13:], r13)
    assert np.array_equal(w2[:n2], b2) and np.array_equal(w2[n2:], r2)


def test_quantize_nvfp4_crafted_matches_oracle(golden_dir):
    rs = np.random.default_rng(5)
    rows = []
    for S in [2.0 ** -9, 3 * 2.0 ** -9, 2.0 ** -7, 0.171875, 1.0, 448.0]:
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6, 7, 0.1, 0.9, 4.4, -5, -0.25, 0, 6],
                        dtype=np.float64) * S
        rows.append(mids.astype(np.float32))
    rows.append(np.zeros(16, np.float32))
    rows.append((rs.standard_normal(16) * 1e-5).astype(np.float32))
    rows.append((rs.standard_normal(16) * 1e3).astype(np.float32))
    rows.append(np.array([np.float32(3 * 2.0 ** -11)] + [0] * 15, np.float32))
    w = np.stack(rows)
    c, s = moeq.quantize_nvfp4(w)
    oc, os_ = oracle.nvfp4_quantize(w)
    assert np.array_equal(c, oc) and np.array_equal(s, os_)
    # the hand-worked fixture blocks
    from tests.test_oracle_formats import _handworked
    for name, v, sb, cb in _handworked(golden_dir):
        c, s = moeq.quantize_nvfp4(v[None, :])
        assert s[0, 0] == sb and list(c[0]) == cb, name


_E2M1_POINTS = [0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, 7.0]


def _e4m3_value(byte):
    e, m = (byte >> 3) & 15, byte & 7
    return (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)


@settings(max_examples=400, deadline=None)
@given(data=st.data())
def test_quantize_nvfp4_adversarial_blocks_match_oracle(data):
    """Random blocks built on the encoder's decision points: a block scale
    from any finite positive E4M3 byte (subnormals included), elements at the
    E2M1 values and at the midpoints between them times that scale, each
    possibly nudged by one float32 ulp either way, with random signs and
    zeros: the library's encoder (C) and the oracle's (brute-force nearest
    value, numpy) give the same code and scale bytes."""
    rows = data.draw(st.integers(1, 4))
    blocks = []
    for _ in range(rows * 2):
        S = _e4m3_value(data.draw(st.integers(1, 126)))
        pts = data.draw(st.lists(st.sampled_from(_E2M1_POINTS), min_size=16, max_size=16))
        sign = data.draw(st.lists(st.booleans(), min_size=16, max_size=16))
        nudge = data.draw(st.lists(st.sampled_from([-1, 0, 0, 1]), min_size=16, max_size=16))
        v = np.array([(-p if sg else p) * S for p, sg in zip(pts, sign)], dtype=np.float32)
        for i, d in enumerate(nudge):
            if d:
                v[i] = np.nextafter(v[i], np.float32(np.inf if d > 0 else -np.inf), dtype=np.float32)
        blocks.append(v)
    w = np.stack(blocks).reshape(rows, 32)
    c, s = moeq.quantize_nvfp4(w)
    oc, os_ = oracle.nvfp4_quantize(w)
    assert np.array_equal(c, oc)
    assert np.array_equal(s, os_)


def test_quantize_nvfp4_rejects_nonfinite():
    w = np.zeros((2, 16), np.float32)
    w[1, 5] = np.inf
    with pytest.raises(moeq.MoeError) as ei:
        moeq.quantize_nvfp4(w)
    assert ei.value.status == moeq.MOE_EINVAL
    with pytest.raises(moeq.MoeError):
        moeq.quantize_nvfp4(np.zeros((2, 24), np.float32))


def _nv_record_offsets(n, kin, rg_step, rg_off):
    """(row, k) -> (byte offset of the code byte, nibble) and (row, block) ->
    scale byte offset, following the tile layout documented in moeq's
    internal header: 16 rows x 128 inputs per 1152-byte tile; lane L holds
    row L&15, inputs (L>>4)*32 .. +32 as 16 code bytes at 16L, and their two
    scales at 1024 + 2L."""
    nkb = (kin + 127) // 128
    code_off = np.empty((n, kin // 2), np.int64)
    scale_off = np.empty((n, kin // 16), np.int64)
    for row in range(n):
        g, r = divmod(row, 16)
        for kbyte in range(kin // 2):
            k = 2 * kbyte
            kb, kk = divmod(k, 128)
            L = r + 16 * (kk // 32)
            tile = (g * rg_step + rg_off) * nkb + kb
            code_off[row, kbyte] = tile * 1152 + L * 16 + (kk % 32) // 2
        for b in range(kin // 16):
            k = 16 * b
            kb, kk = divmod(k, 128)
            L = r + 16 * (kk // 32)
            tile = (g * rg_step + rg_off) * nkb + kb
            scale_off[row, b] = tile * 1152 + 1024 + 2 * L + (kk % 32) // 16
    return code_off, scale_off


@pytest.mark.parametrize("H,I", [(256, 128), (144, 48), (2304, 1152)])
def test_nvfp4_record_layout(H, I):
    rs = np.random.default_rng(H)
    mats = []
    for shape in [(I, H), (I, H), (H, I)]:
        w = (rs.standard_normal(shape) * 0.02).astype(np.float32)
        mats.append(moeq.quantize_nvfp4(w))
    w13, w2 = moeq.pack_nvfp4_expert(mats[0], mats[1], mats[2], H, I)
    assert w13.size == moeq.record_bytes(moeq.FMT_NVFP4, 0, H, I)
    for (codes, scales), rec, rg_step, rg_off in [(mats[0], w13, 2, 0), (mats[1], w13, 2, 1),
                                                   (mats[2], w2, 1, 0)]:
        n, kin = codes.shape[0], codes.shape[1] * 2
        co, so = _nv_record_offsets(n, kin, rg_step, rg_off)
        assert np.array_equal(rec[co], codes)
        assert np.array_equal(rec[so], scales)
    # everything else in the records is zero padding
    used = np.zeros(w13.size, bool)
    for (codes, scales), rg_off in [(mats[0], 0), (mats[1], 1)]:
        co, so = _nv_record_offsets(I, H, 2, rg_off)
        used[co.ravel()] = True
        used[so.ravel()] = True
    assert np.all(w13[~used] == 0)


def _finite_f16_bits(rs, n):
    """n random fp16 bit patterns of finite values (any sign, exponent field
    below all-ones)."""
    return (rs.integers(0, 0x7C00, n) | (rs.integers(0, 2, n) << 15)).astype(np.uint16)


def test_vq_record_layout():
    H, I = 272, 48
    rs = np.random.default_rng(0)
    parts = []
    for n, kin in [(I, H), (I, H), (H, I)]:
        parts.append((rs.integers(0, 65536, (n, kin // 8), dtype=np.uint16),
                      _finite_f16_bits(rs, n)))
    w13, w2 = moeq.pack_vq_expert(parts[0], parts[1], parts[2], H, I)
    for (codes, scales), rec, rg_step, rg_off, nrg in [(parts[0], w13, 2, 0, 2 * I // 16),
                                                       (parts[1], w13, 2, 1, 2 * I // 16),
                                                       (parts[2], w2, 1, 0, H // 16)]:
        n, ng = codes.shape
        kin = ng * 8
        nkb = (kin + 255) // 256
        r16 = rec[: nrg * nkb * 1024].view(np.uint16)
        for row in range(n):
            g, r = divmod(row, 16)
            for grp in range(ng):
                kb, kk = divmod(8 * grp, 256)
                L = r + 16 * (kk // 64)
                s = (kk % 64) // 8
                off = ((g * rg_step + rg_off) * nkb + kb) * 1024 + 16 * L + 2 * s
                assert r16[off // 2] == codes[row, grp]
    c13 = (2 * I // 16) * ((H + 255) // 256) * 1024
    assert np.array_equal(w13[c13:c13 + 2 * I].view(np.uint16), parts[0][1])
    assert np.array_equal(w13[c13 + 2 * I:c13 + 4 * I].view(np.uint16), parts[1][1])
    c2 = (H // 16) * ((I + 255) // 256) * 1024
    assert np.array_equal(w2[c2:c2 + 2 * H].view(np.uint16), parts[2][1])


@pytest.mark.parametrize("m", [1, 2, 3])
def test_vq8_record_layout(m):
    H, I = 272, 48
    rs = np.random.default_rng(m)
    parts = []
    for n, kin in [(I, H), (I, H), (H, I)]:
        parts.append((rs.integers(0, 256, (n, kin // 8, m), dtype=np.uint8),
                      _finite_f16_bits(rs, n)))
    w13, w2 = moeq.pack_vq8_expert(parts[0], parts[1], parts[2], H, I, m)
    assert w13.size == moeq.record_bytes(moeq.FMT_VQ8, 0, H, I, m) and w13.size % 256 == 0
    tb = 512 * m
    for (codes, scales), rec, rg_step, rg_off, nrg in [(parts[0], w13, 2, 0, 2 * I // 16),
                                                       (parts[1], w13, 2, 1, 2 * I // 16),
                                                       (parts[2], w2, 1, 0, H // 16)]:
        n, ng, _ = codes.shape
        kin = ng * 8
        nkb = (kin + 255) // 256
        for row in range(n):
            g, r = divmod(row, 16)
            for grp in range(ng):
                kb, kk = divmod(8 * grp, 256)
                L = r + 16 * (kk // 64)
                s = (kk % 64) // 8
                off = ((g * rg_step + rg_off) * nkb + kb) * tb + 8 * m * L + m * s
                assert np.array_equal(rec[off:off + m], codes[row, grp])
    c13 = (2 * I // 16) * ((H + 255) // 256) * tb
    assert np.array_equal(w13[c13:c13 + 2 * I].view(np.uint16), parts[0][1])
    assert np.array_equal(w13[c13 + 2 * I:c13 + 4 * I].view(np.uint16), parts[1][1])
    c2 = (H // 16) * ((I + 255) // 256) * tb
    assert np.array_equal(w2[c2:c2 + 2 * H].view(np.uint16), parts[2][1])
    with pytest.raises(moeq.MoeError):
        moeq.pack_vq8_expert(parts[0], parts[1], parts[2], H, I, 4)
    assert moeq.record_bytes(moeq.FMT_VQ8, 0, H, I, 4) == 0


@pytest.mark.parametrize("H,I", [(256, 128), (272, 48)])
def test_bf16_record_layout(H, I):
    # byte offset of weight (row, k) from the tile layout: 16-row groups, 128
    # inputs per 4096-byte tile, slice j = (k % 32) // 8 of 1 KB, lane
    # L = row % 16 + 16 * ((k % 128) // 32), 16 bytes per lane
    rs = np.random.default_rng(H + I)
    mats = [synth.f32_to_bf16_bits((rs.standard_normal(sh) * 0.02).astype(np.float32))
            for sh in [(I, H), (I, H), (H, I)]]
    w13, w2 = moeq.pack_bf16_expert(mats[0], mats[1], mats[2], H, I)
    assert w13.size == moeq.record_bytes(moeq.FMT_BF16, 0, H, I) and w13.size % 256 == 0
    assert w2.size == moeq.record_bytes(moeq.FMT_BF16, 1, H, I)
    used13 = np.zeros(w13.size // 2, bool)
    for w, rec, rg_step, rg_off, used in [(mats[0], w13, 2, 0, used13), (mats[1], w13, 2, 1, used13),
                                          (mats[2], w2, 1, 0, None)]:
        n, kin = w.shape
        nkb = (kin + 127) // 128
        row = np.arange(n)[:, None]
        k = np.arange(kin)[None, :]
        g, r = row // 16, row % 16
        kb, kk = k // 128, k % 128
        L = r + 16 * (kk // 32)
        tile = (g * rg_step + rg_off) * nkb + kb
        off = tile * 4096 + 1024 * ((kk % 32) // 8) + 16 * L + 2 * (kk % 8)
        assert np.array_equal(rec.view(np.uint16)[off // 2], w)
        if used is not None:
            used[(off // 2).ravel()] = True
    assert np.all(w13.view(np.uint16)[~used13] == 0)       # padding is zero


def test_pack_bf16_range():
    H, I = 32, 16
    z = np.zeros((I, H), np.uint16)
    d = np.zeros((H, I), np.uint16)
    big = z.copy()
    big[3, 5] = 0x477F                        # 65280: the largest bf16 <= 65504
    big[4, 6] = 0xC77F
    moeq.pack_bf16_expert(big, z, d, H, I)
    for bits in (0x4780, 0xC780, 0x7F80, 0xFF80, 0x7FC0):   # 65536, -65536, inf, -inf, nan
        bad = z.copy()
        bad[1, 2] = bits
        with pytest.raises(moeq.MoeError) as ei:
            moeq.pack_bf16_expert(z, bad, d, H, I)
        assert ei.value.status == moeq.MOE_EINVAL


def test_record_table_resident():
    tm = np.array([1, 2, 2, 3, 1, 3], np.uint8)
    rec = moeq.record_table_resident(tm)
    assert np.array_equal(rec >> 24, tm) and np.array_equal(rec & 0xFFFFFF, np.arange(6))
    with pytest.raises(moeq.MoeError) as ei:
        moeq.record_table_resident(np.array([1, 9], np.uint8))
    assert ei.value.status == moeq.MOE_EUNSUPPORTED


def test_record_table():
    tm = synth.tier_map(synth.MIXED)
    rec, counts = moeq.record_table(tm)
    assert counts == {1: 108, 2: 148, 3: 0, 4: 0, 5: 0, 6: 0, 7: 0, 8: 0}
    for fmt in (1, 2):
        sel = np.nonzero(tm == fmt)[0]
        assert np.all(rec[sel] >> 24 == fmt)
        assert np.array_equal(rec[sel] & 0xFFFFFF, np.arange(sel.size))
    tm3 = synth.tier_map(synth.small_workload("m3", E=40, k=4, H=64, I=32, T=4, fmt="mixed3",
                                              n_nvfp4=10, vq8_m=2))
    rec, counts = moeq.record_table(tm3)
    assert counts[1] == 10 and counts[3] == 15 and counts[2] == 15
    for fmt in (1, 2, 3):
        sel = np.nonzero(tm3 == fmt)[0]
        assert np.all(rec[sel] >> 24 == fmt)
        assert np.array_equal(rec[sel] & 0xFFFFFF, np.arange(sel.size))
    rec, counts = moeq.record_table(np.array([4, 1, 4], np.uint8))
    assert counts == {1: 1, 2: 0, 3: 0, 4: 2, 5: 0, 6: 0, 7: 0, 8: 0}
    assert list(rec) == [4 << 24, 1 << 24, (4 << 24) | 1]
    # small-codebook VQ experts at explicit rates: one pool (index space) each
    rec, counts = moeq.record_table(np.array([7, 6, 8, 7, 6, 1], np.uint8))
    assert counts[6] == 2 and counts[7] == 2 and counts[8] == 1 and counts[1] == 1
    assert list(rec) == [7 << 24, 6 << 24, 8 << 24, (7 << 24) | 1, (6 << 24) | 1, 1 << 24]
    rec, counts = moeq.record_table(np.array([5, 1, 5, 5], np.uint8))
    assert counts[5] == 3 and counts[1] == 1
    assert list(rec) == [5 << 24, 1 << 24, (5 << 24) | 1, (5 << 24) | 2]
    bad = tm.copy()
    bad[7] = 9
    with pytest.raises(moeq.MoeError) as ei:
        moeq.record_table(bad)
    assert ei.value.status == moeq.MOE_EUNSUPPORTED


# ---------------------------------------------------------------- host-side checks (no launch)

def test_route_rejects_bad_sizes_before_launch():
    L = moeq.lib()
    N = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)
    assert L.moe_route_topk(fake, 4, 0, 1, fake, fake, N) == moeq.MOE_EINVAL
    assert L.moe_route_topk(fake, 4, 8, 9, fake, fake, N) == moeq.MOE_EINVAL
    assert L.moe_route_topk(fake, 4, 2048, 8, fake, fake, N) == moeq.MOE_EINVAL
    assert L.moe_route_topk(fake, 4, 64, 17, fake, fake, N) == moeq.MOE_EINVAL
    assert L.moe_route_topk(N, 4, 8, 2, fake, fake, N) == moeq.MOE_EINVAL
    assert b"k must be" in L.moe_last_error() or L.moe_last_error()
    # T == 0 is a no-op that touches nothing
    assert L.moe_route_topk(N, 0, 8, 2, N, N, N) == moeq.MOE_OK
    assert L.moe_combine(N, N, N, 0, 2, 64, N, N) == moeq.MOE_OK
    assert L.moe_combine(fake, fake, fake, 3, 2, 66, fake, N) == moeq.MOE_EINVAL


def _fake_layer(fmt_host, H=256, I=128):
    d = moeq._QLayerC()
    d.E = len(fmt_host)
    d.H, d.I = H, I
    d.fmt_host = fmt_host.ctypes.data
    d.rec_dev = 0x1000
    for name in ("nvfp4_w13", "nvfp4_w2", "vq_w13", "vq_w2"):
        setattr(d, name, 0x100000)
    d.nvfp4_w13_stride = 1 << 20
    d.nvfp4_w2_stride = 1 << 20
    d.vq_w13_stride = 1 << 20
    d.vq_w2_stride = 1 << 20
    for p in range(3):
        d.vq_codebook[p] = 0x100000
    return d


def test_shared_ffn_and_combine_shared_host_checks():
    L = moeq.lib()
    fake = ctypes.c_void_p(0x1000)
    N = ctypes.c_void_p(0)
    d = _fake_layer(np.full(2, moeq.FMT_NVFP4, np.uint8))
    need = L.moe_shared_ffn_workspace_bytes(ctypes.byref(d), 4)
    assert need > 0
    assert L.moe_shared_ffn(ctypes.byref(d), fake, 4, fake, fake, need, N) == moeq.MOE_EINVAL
    assert b"E == 1" in L.moe_last_error()
    d = _fake_layer(np.full(1, moeq.FMT_BF16, np.uint8))
    d.bf16_w13 = d.bf16_w2 = 0x100000
    d.bf16_w13_stride = d.bf16_w2_stride = 1 << 20
    assert L.moe_shared_ffn(ctypes.byref(d), N, 0, N, N, 0, N) == moeq.MOE_OK   # T == 0
    assert L.moe_shared_ffn(ctypes.byref(d), fake, 4, fake, fake, need - 1,
                            N) == moeq.MOE_EWORKSPACE
    assert L.moe_shared_ffn(ctypes.byref(d), N, 4, fake, fake, need, N) == moeq.MOE_EINVAL
    d.bf16_w2 = None
    assert L.moe_shared_ffn(ctypes.byref(d), fake, 4, fake, fake, need, N) == moeq.MOE_EINVAL
    d.bf16_w2 = 0x100000
    d.bf16_w2_stride = 1000
    assert L.moe_shared_ffn(ctypes.byref(d), fake, 4, fake, fake, need, N) == moeq.MOE_EINVAL
    assert L.moe_combine_shared(N, N, N, N, 0, 2, 64, N, N) == moeq.MOE_OK
    assert L.moe_combine_shared(fake, fake, fake, N, 3, 2, 64, fake, N) == moeq.MOE_EINVAL
    assert L.moe_combine_shared(fake, fake, fake, fake, 3, 2, 66, fake, N) == moeq.MOE_EINVAL


def test_ffn_fails_closed_on_unknown_format():
    L = moeq.lib()
    fake = ctypes.c_void_p(0x1000)
    tm = np.full(8, moeq.FMT_NVFP4, np.uint8)
    tm[3] = 9
    d = _fake_layer(tm)
    st = L.moe_expert_ffn_q(ctypes.byref(d), fake, fake, fake, 4, 2, fake, fake, 1 << 20,
                            ctypes.c_void_p(0))
    assert st == moeq.MOE_EUNSUPPORTED
    assert b"expert 3" in L.moe_last_error()
    st = L.moe_dequant_q(ctypes.byref(d), 0, 0, fake, ctypes.c_void_p(0))
    assert st == moeq.MOE_EUNSUPPORTED


def test_ffn_rejects_bad_shapes_and_workspace():
    L = moeq.lib()
    fake = ctypes.c_void_p(0x1000)
    N = ctypes.c_void_p(0)
    tm = np.full(8, moeq.FMT_NVFP4, np.uint8)
    d = _fake_layer(tm, H=264, I=128)        # H % 16 != 0
    assert L.moe_expert_ffn_q(ctypes.byref(d), fake, fake, fake, 4, 2, fake, fake, 1 << 20,
                              N) == moeq.MOE_EUNSUPPORTED
    d = _fake_layer(tm)
    need = L.moe_ffn_workspace_bytes(ctypes.byref(d), 4, 2)
    assert need > 0
    assert L.moe_expert_ffn_q(ctypes.byref(d), fake, fake, fake, 4, 2, fake, ctypes.c_void_p(0x1000),
                              need - 1, N) == moeq.MOE_EWORKSPACE
    d.nvfp4_w13_stride = 1000                # not a multiple of 256 / too small
    assert L.moe_expert_ffn_q(ctypes.byref(d), fake, fake, fake, 4, 2, fake, ctypes.c_void_p(0x1000),
                              need, N) == moeq.MOE_EINVAL
    d = _fake_layer(tm)
    d.nvfp4_w2 = None                        # pool missing
    assert L.moe_expert_ffn_q(ctypes.byref(d), fake, fake, fake, 4, 2, fake, ctypes.c_void_p(0x1000),
                              need, N) == moeq.MOE_EINVAL
    d = _fake_layer(tm)
    assert L.moe_expert_ffn_q(ctypes.byref(d), N, N, N, 0, 2, N, N, 0, N) == moeq.MOE_OK  # T == 0
    assert L.moe_expert_ffn_q(ctypes.byref(d), fake, fake, fake, 4, 9, fake, fake, need,
                              N) == moeq.MOE_EINVAL  # k > E
    assert L.moe_dequant_q(ctypes.byref(d), 8, 0, fake, N) == moeq.MOE_EINVAL
    assert L.moe_dequant_q(ctypes.byref(d), 0, 3, fake, N) == moeq.MOE_EINVAL


def test_nvfp4r_layer_host_checks():
    """Two-level NVFP4 experts need their pools and a residual exponent in
    [0, 14]; checked before any launch."""
    L = moeq.lib()
    fake = ctypes.c_void_p(0x1000)
    N = ctypes.c_void_p(0)
    tm = np.array([1, 5, 5, 1], np.uint8)
    d = _fake_layer(tm)
    need = L.moe_ffn_workspace_bytes(ctypes.byref(d), 4, 2)
    assert L.moe_expert_ffn_q(ctypes.byref(d), fake, fake, fake, 4, 2, fake, fake, need,
                              N) == moeq.MOE_EINVAL            # NVFP4R pools NULL
    assert b"NVFP4R" in L.moe_last_error()
    d.nvfp4r_w13 = d.nvfp4r_w2 = 0x100000
    d.nvfp4r_w13_stride = d.nvfp4r_w2_stride = 1 << 20
    d.nvfp4r_shift = 15
    assert L.moe_expert_ffn_q(ctypes.byref(d), fake, fake, fake, 4, 2, fake, fake, need,
                              N) == moeq.MOE_EUNSUPPORTED
    assert b"nvfp4r_shift" in L.moe_last_error()
    d.nvfp4r_shift = 8
    d.nvfp4r_w2_stride = moeq.record_bytes(moeq.FMT_NVFP4, 1, 256, 128)   # one plane only
    assert L.moe_expert_ffn_q(ctypes.byref(d), fake, fake, fake, 4, 2, fake, fake, need,
                              N) == moeq.MOE_EINVAL


def test_nested_layer_host_side():
    """A nested layer (NVFP4 and two-level NVFP4 resident) built in host
    memory: the NVFP4 pools are the two-level records (same buffers and
    strides in the descriptor), the base planes are the plain NVFP4 records,
    set_residual rewrites only the residual halves, and set_tiers moves
    experts between the tags."""
    from bit_quantized_moe_route_amd.layers import build_layer
    E, H, I = 4, 256, 64
    rs = np.random.default_rng(31)
    W = {(e, p): (rs.standard_normal((I, H) if p < 2 else (H, I)) * 0.02).astype(np.float32)
         for e in range(E) for p in range(3)}
    tm = np.array([1, 5, 1, 5], np.uint8)
    lay = build_layer(E, H, I, tm, nvfp4_weights=lambda e, p: W[(e, p)], device="cpu",
                      workers=2, resident_formats={moeq.FMT_NVFP4, moeq.FMT_NVFP4R})
    assert lay.alias == {moeq.FMT_NVFP4: moeq.FMT_NVFP4R}
    for which in (0, 1):
        assert lay.pools[(1, which)] is lay.pools[(5, which)]
        assert lay.stride[(1, which)] == lay.stride[(5, which)]
    d = lay.c()
    assert d.nvfp4_w13 == d.nvfp4r_w13 and d.nvfp4_w2 == d.nvfp4r_w2
    assert d.nvfp4_w13_stride == d.nvfp4r_w13_stride and d.nvfp4r_shift == moeq.NVFP4R_SHIFT
    n13 = moeq.record_bytes(moeq.FMT_NVFP4, 0, H, I)
    n2 = moeq.record_bytes(moeq.FMT_NVFP4, 1, H, I)
    s13, s2 = lay.stride[(5, 0)], lay.stride[(5, 1)]
    p13, p2 = lay.pools[(5, 0)].numpy(), lay.pools[(5, 1)].numpy()
    for e in range(E):
        b13, b2 = moeq.pack_nvfp4_expert(*[moeq.quantize_nvfp4(W[(e, p)]) for p in range(3)], H, I)
        assert np.array_equal(p13[e * s13: e * s13 + n13], b13)
        assert np.array_equal(p2[e * s2: e * s2 + n2], b2)
    before = p13.copy(), p2.copy()
    lay.set_residual(2, np.full(n13, 7, np.uint8), np.full(n2, 9, np.uint8))
    changed13 = np.flatnonzero(before[0] != p13)
    changed2 = np.flatnonzero(before[1] != p2)
    assert changed13.min() >= 2 * s13 + n13 and changed13.max() < 2 * s13 + 2 * n13
    assert changed2.min() >= 2 * s2 + n2 and changed2.max() < 2 * s2 + 2 * n2
    lay.set_tiers(np.array([5, 5, 1, 1], np.uint8))
    assert list(lay.rec_host >> 24) == [5, 5, 1, 1]
    assert list(lay.rec_host & 0xFFFFFF) == [0, 1, 2, 3]
    assert lay.counts[1] == 2 and lay.counts[5] == 2


def test_layer_forward_host_checks():
    """moe_layer_forward: the step-by-step calls' checks, before any launch."""
    L = moeq.lib()
    fake = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x100000)          # 256-byte aligned stand-in
    N = ctypes.c_void_p(0)
    tm = np.full(8, moeq.FMT_NVFP4, np.uint8)
    d = _fake_layer(tm)
    need = L.moe_layer_forward_workspace_bytes(ctypes.byref(d), 4, 2)
    # at least the step-by-step path's buffers: expert-FFN workspace + y_perm
    assert need >= L.moe_ffn_workspace_bytes(ctypes.byref(d), 4, 2) + 4 * 2 * 256 * 4
    assert need % 256 == 0
    assert L.moe_layer_forward_workspace_bytes(None, 4, 2) == 0
    args = lambda T, k, nbytes, w=ws: (ctypes.byref(d), fake, fake, T, k, N, fake, fake, fake, w,
                                       nbytes, N)
    assert L.moe_layer_forward(*args(0, 2, 0, N)) == moeq.MOE_OK            # T == 0
    assert L.moe_layer_forward(*args(4, 2, need - 1)) == moeq.MOE_EWORKSPACE
    assert L.moe_layer_forward(*args(4, 2, need, ctypes.c_void_p(0x100010))) == moeq.MOE_EINVAL
    assert L.moe_layer_forward(*args(4, 9, need)) == moeq.MOE_EINVAL        # k > E
    assert L.moe_layer_forward(ctypes.byref(d), N, fake, 4, 2, N, fake, fake, fake, ws, need,
                               N) == moeq.MOE_EINVAL                          # x NULL
    assert L.moe_layer_forward(ctypes.byref(d), fake, fake, 4, 2, N, fake, fake, N, ws, need,
                               N) == moeq.MOE_EINVAL                          # out NULL
    bad = tm.copy()
    bad[5] = 9
    d = _fake_layer(bad)
    assert L.moe_layer_forward(*args(4, 2, need)) == moeq.MOE_EUNSUPPORTED
    assert b"expert 5" in L.moe_last_error()


# ---------------------------------------------------------------- rotation helpers

def test_rot_sign_bytes_and_packing():
    H, I = 256, 128
    assert moeq.rot_sign_bytes(H, I) == (2 * H + 3 * I) // 8
    assert moeq.rot_sign_bytes(250, 128) == 0
    rs = np.random.default_rng(3)
    secs = [np.where(rs.random(n) < 0.5, -1, 1).astype(np.int8) for n in (H, I, I, I, H)]
    b = moeq.pack_rot_signs(*secs, H, I)
    # bit i of byte j of a section = channel 8j + i is negative, sections in order
    bits = np.unpackbits(b, bitorder="little").astype(bool)
    want = np.concatenate([s < 0 for s in secs])
    assert np.array_equal(bits, want)
    bad = [x.copy() for x in secs]
    bad[3][5] = 0
    with pytest.raises(moeq.MoeError) as ei:
        moeq.pack_rot_signs(*bad, H, I)
    assert ei.value.status == moeq.MOE_EINVAL


@pytest.mark.parametrize("n_out,n_in,bo,bi", [(256, 384, 128, 128), (256, 1024, 128, 512),
                                               (512, 256, 512, 128)])
def test_rotate_matrix_matches_oracle(n_out, n_in, bo, bi):
    """The library's offline rotation (fp64 butterflies, one rounding to fp32)
    against the oracle's (fp64 block products): equal to within one fp32
    rounding, and the inverse rotation gives the matrix back; also with the
    wide 512-block on one side."""
    rs = np.random.default_rng(9 + n_in)
    w = (rs.standard_normal((n_out, n_in)) * 0.02).astype(np.float32)
    so = np.where(rs.random(n_out) < 0.5, -1, 1).astype(np.int8)
    si = np.where(rs.random(n_in) < 0.5, -1, 1).astype(np.int8)
    got = moeq.rotate_matrix(w, so, si, block_out=bo, block_in=bi)
    want = oracle.rotate_weights(w.astype(np.float64), so, si, block_out=bo, block_in=bi)
    assert np.all(np.abs(got - want) <= 2.0 ** -24 * np.abs(want) + 1e-45)
    back = oracle.unrotate_weights(got.astype(np.float64), so, si, block_out=bo, block_in=bi)
    assert np.allclose(back, w, rtol=0, atol=1e-8)
    if bo == bi == 128:
        assert np.array_equal(moeq.rotate_matrix(w, so, si), got)
    with pytest.raises(moeq.MoeError):
        moeq.rotate_matrix(w[:, :200], so, si[:200])
    with pytest.raises(moeq.MoeError):                       # blocks are 128 or 512
        moeq.rotate_matrix(w, so, si, block_in=256)
    with pytest.raises(moeq.MoeError):                       # 384 is no multiple of 512
        moeq.rotate_matrix(np.zeros((128, 384), np.float32), so[:128],
                           np.ones(384, np.int8), block_in=512)


def test_rotated_layer_host_checks():
    L = moeq.lib()
    fake = ctypes.c_void_p(0x1000)
    N = ctypes.c_void_p(0)
    tm = np.full(8, moeq.FMT_NVFP4, np.uint8)
    d = _fake_layer(tm, H=272, I=128)
    d.rot_signs = 0x2000                      # H not a multiple of 128
    need = L.moe_ffn_workspace_bytes(ctypes.byref(d), 4, 2)
    assert L.moe_expert_ffn_q(ctypes.byref(d), fake, fake, fake, 4, 2, fake, fake, need,
                              N) == moeq.MOE_EUNSUPPORTED
    d = _fake_layer(tm)
    plain = L.moe_ffn_workspace_bytes(ctypes.byref(d), 4, 2)
    d.rot_signs = 0x2000
    rot = L.moe_ffn_workspace_bytes(ctypes.byref(d), 4, 2)
    # rotated: x' [T*k, H] fp16 + g | u [T*k, 2I] fp32 + h [T*k, I] fp16, 256-aligned
    assert rot == 4 * 2 * 256 * 2 + 4 * 2 * 2 * 128 * 4 + 4 * 2 * 128 * 2
    assert rot > plain
    assert L.moe_expert_ffn_q(ctypes.byref(d), fake, fake, fake, 4, 2, fake, fake, rot - 1,
                              N) == moeq.MOE_EWORKSPACE
    # the down-input block: 0 / 128 / 512, and 512 needs I a multiple of 512
    for blk in (256, 64, -1, 1024):
        d = _fake_layer(tm)
        d.rot_signs = 0x2000
        d.rot_in2_block = blk
        assert L.moe_expert_ffn_q(ctypes.byref(d), fake, fake, fake, 4, 2, fake, fake, rot,
                                  N) == moeq.MOE_EUNSUPPORTED
    d = _fake_layer(tm)                       # I = 128
    d.rot_signs = 0x2000
    d.rot_in2_block = 512
    assert L.moe_expert_ffn_q(ctypes.byref(d), fake, fake, fake, 4, 2, fake, fake, rot,
                              N) == moeq.MOE_EUNSUPPORTED
    assert b"512" in L.moe_last_error()
    one = _fake_layer(np.full(1, moeq.FMT_NVFP4, np.uint8))
    one.rot_signs = 0x2000
    assert L.moe_shared_ffn(ctypes.byref(one), fake, 4, fake, fake, 1 << 24,
                            N) == moeq.MOE_EUNSUPPORTED


def test_layer_forward_shared_host_checks():
    """moe_layer_forward_shared rejects on the host, before any launch: a
    shared layer with E != 1 or another H, a short workspace; T = 0 is a no-op."""
    import ctypes
    L = moeq.lib()
    E, H, I = 8, 256, 128
    fmt = (ctypes.c_uint8 * E)(*([1] * E))
    rec = ctypes.c_void_p(16)            # never dereferenced on the host
    lay = moeq._QLayerC()
    lay.E, lay.H, lay.I = E, H, I
    lay.fmt_host = ctypes.cast(fmt, ctypes.c_void_p)
    lay.rec_dev = rec
    lay.nvfp4_w13 = lay.nvfp4_w2 = ctypes.c_void_p(256)
    lay.nvfp4_w13_stride = L.moe_record_bytes(1, 0, H, I)
    lay.nvfp4_w2_stride = L.moe_record_bytes(1, 1, H, I)
    sfmt = (ctypes.c_uint8 * 2)(4, 4)   # two tags, so that E = 2 below reads valid memory
    sh = moeq._QLayerC()
    sh.E, sh.H, sh.I = 1, H, I
    sh.fmt_host = ctypes.cast(sfmt, ctypes.c_void_p)
    sh.rec_dev = rec
    sh.bf16_w13 = sh.bf16_w2 = ctypes.c_void_p(256)
    sh.bf16_w13_stride = L.moe_record_bytes(4, 0, H, I)
    sh.bf16_w2_stride = L.moe_record_bytes(4, 1, H, I)
    p = ctypes.c_void_p(256)
    need = L.moe_layer_forward_shared_workspace_bytes(ctypes.byref(lay), ctypes.byref(sh), 2, 2)
    assert need >= L.moe_layer_forward_workspace_bytes(ctypes.byref(lay), 2, 2) + 2 * H * 4
    call = lambda s, T, ws_bytes: L.moe_layer_forward_shared(
        ctypes.byref(lay), ctypes.byref(s), p, p, T, 2, p, p, p, p, ws_bytes, None)
    assert call(sh, 0, 0) == moeq.MOE_OK
    assert call(sh, 2, need - 1) == moeq.MOE_EWORKSPACE
    sh.H = 512
    assert call(sh, 2, need) == moeq.MOE_EINVAL
    sh.H = H
    sh.E = 2
    assert call(sh, 2, need) == moeq.MOE_EINVAL


# ------------------------------------------------- packer input validation

def _nv_mats(H, I, seed):
    rs = np.random.default_rng(seed)
    return [moeq.quantize_nvfp4((rs.standard_normal(shape) * 0.02).astype(np.float32))
            for shape in [(I, H), (I, H), (H, I)]]


@pytest.mark.parametrize("bad", [0x7F, 0xFF])
def test_pack_nvfp4_rejects_e4m3_nan_scales(bad):
    H, I = 256, 128
    mats = _nv_mats(H, I, 5)
    for which in range(3):
        m = [(c, sc.copy()) for c, sc in mats]
        m[which][1][3, 1] = bad
        with pytest.raises(moeq.MoeError) as ei:
            moeq.pack_nvfp4_expert(m[0], m[1], m[2], H, I)
        assert ei.value.status == moeq.MOE_EINVAL
        assert b"NaN" in moeq.lib().moe_last_error()
        # the same byte in either plane of a two-level expert
        with pytest.raises(moeq.MoeError) as ei:
            moeq.pack_nvfp4r_expert(mats, m, H, I)
        assert ei.value.status == moeq.MOE_EINVAL
        with pytest.raises(moeq.MoeError) as ei:
            moeq.pack_nvfp4r_expert(m, mats, H, I)
        assert ei.value.status == moeq.MOE_EINVAL
    # the largest finite bytes (+-448) and negative scales are values, not errors
    m = [(c, sc.copy()) for c, sc in mats]
    m[0][1][0, 0], m[1][1][0, 0], m[2][1][0, 0] = 0x7E, 0xFE, 0x88
    moeq.pack_nvfp4_expert(m[0], m[1], m[2], H, I)


@pytest.mark.parametrize("bad", [0x7C00, 0xFC00, 0x7E00, 0xFFFF])
def test_pack_vq_rejects_nonfinite_scales(bad):
    H, I = 256, 128
    rs = np.random.default_rng(6)
    parts = [(rs.integers(0, 65536, (n, kin // 8), dtype=np.uint16), _finite_f16_bits(rs, n))
             for n, kin in [(I, H), (I, H), (H, I)]]
    parts8 = [(rs.integers(0, 256, (n, kin // 8, 2), dtype=np.uint8), _finite_f16_bits(rs, n))
              for n, kin in [(I, H), (I, H), (H, I)]]
    for which in range(3):
        p = [(c, sc.copy()) for c, sc in parts]
        p[which][1][7] = bad
        with pytest.raises(moeq.MoeError) as ei:
            moeq.pack_vq_expert(p[0], p[1], p[2], H, I)
        assert ei.value.status == moeq.MOE_EINVAL
        p8 = [(c, sc.copy()) for c, sc in parts8]
        p8[which][1][7] = bad
        with pytest.raises(moeq.MoeError) as ei:
            moeq.pack_vq8_expert(p8[0], p8[1], p8[2], H, I, 2)
        assert ei.value.status == moeq.MOE_EINVAL
    # the largest finite magnitude is accepted
    p = [(c, sc.copy()) for c, sc in parts]
    p[0][1][0], p[2][1][1] = 0x7BFF, 0xFBFF
    moeq.pack_vq_expert(p[0], p[1], p[2], H, I)


# ------------------------------------------------- workspace sizes

def _bf16_shared_layer(H, I):
    d = _fake_layer(np.full(1, moeq.FMT_BF16, np.uint8), H=H, I=I)
    d.bf16_w13 = d.bf16_w2 = 0x100000
    d.bf16_w13_stride = d.bf16_w2_stride = 1 << 30
    return d


def _al(n):
    return (n + 255) // 256 * 256


def test_shared_workspace_is_sized_for_the_path_that_runs():
    """The shared expert's decode path (T < 128) splits its gate/up inputs over
    nsplit workgroups and keeps nsplit x T x 2I fp32 partial sums; the
    grouped GEMM (T >= 128, NVFP4 or BF16) keeps none."""
    L = moeq.lib()
    H, I = 6144, 2048
    d = _bf16_shared_layer(H, I)
    # T = 4096 and 16384: x as fp16 and h only (no partial sums)
    for T in (4096, 16384):
        need = L.moe_shared_ffn_workspace_bytes(ctypes.byref(d), T)
        assert need == _al(T * H * 2) + _al(T * I * 2), T
    assert L.moe_shared_ffn_workspace_bytes(ctypes.byref(d), 4096) < 80 << 20
    # decode: I/16 = 128 row-pair groups per input split; 512 workgroups aimed
    # for -> 4 splits (and 48 input tiles of 128 allow up to 12)
    for T in (1, 8, 127):
        need = L.moe_shared_ffn_workspace_bytes(ctypes.byref(d), T)
        assert need == _al(T * H * 2) + _al(T * I * 2) + _al(4 * T * 2 * I * 4), T
    # a VQ shared expert keeps the decode path at every T (256-input tiles)
    dv = _fake_layer(np.full(1, moeq.FMT_VQ, np.uint8), H=H, I=I)
    need = L.moe_shared_ffn_workspace_bytes(ctypes.byref(dv), 4096)
    assert need == _al(4096 * H * 2) + _al(4096 * I * 2) + _al(4 * 4096 * 2 * I * 4)
    # a small layer: the split is capped by the input tiles (H = 256: 2 tiles
    # of 128 for 4 waves -> one split)
    ds = _bf16_shared_layer(256, 128)
    assert L.moe_shared_ffn_workspace_bytes(ctypes.byref(ds), 4) == (
        _al(4 * 256 * 2) + _al(4 * 128 * 2) + _al(1 * 4 * 2 * 128 * 4))
    # the one-call layer with a shared expert reserves the same shared part
    routed = _fake_layer(np.full(256, moeq.FMT_NVFP4, np.uint8), H=H, I=I)
    T, k = 4096, 8
    lw = L.moe_layer_forward_workspace_bytes(ctypes.byref(routed), T, k)
    tot = L.moe_layer_forward_shared_workspace_bytes(ctypes.byref(routed), ctypes.byref(d), T, k)
    assert tot == _al(lw) + _al(T * H * 2) + _al(T * I * 2) + _al(T * H * 4)
