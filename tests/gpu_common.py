"""Shared helpers of the GPU parity tests."""

import sys

import numpy as np

import oracle
import synth

ROW_TOL = 1e-2       # max |gpu - oracle| per row <= ROW_TOL * RMS(oracle row)
W_TOL = 1e-6         # router weights, absolute


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def assert_rows_close(gpu, ref, what, tol=ROW_TOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), what
    rms = np.sqrt(np.mean(ref * ref, axis=1))
    err = np.max(np.abs(gpu - ref), axis=1)
    zero = rms == 0
    assert np.all(gpu[zero] == 0), (what, "rows with zero oracle RMS must be exactly 0")
    rel = err[~zero] / rms[~zero]
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= tol, (what, "worst row rel err", worst)
    return worst


def build_small_layer(wl, device="cuda", resident_formats=None):
    """A QLayer for workload wl built by the library's packers from the
    seeded inputs (resident_formats: pack every expert in each of these
    formats, for tier switches)."""
    from bit_quantized_moe_route_amd.layers import build_layer

    fmt_host = synth.tier_map(wl)
    if wl.fmt == "nested" and resident_formats is None:
        # both tiers resident: the NVFP4 tier runs on the two-level records'
        # base planes
        resident_formats = {synth.FMT_NVFP4, synth.FMT_NVFP4R}
    used = set(np.unique(fmt_host).tolist()) | set(resident_formats or ())
    cbs = [synth.vq_codebook(wl, p) for p in range(3)] if synth.FMT_VQ in used else None
    vq8_tags = {synth.FMT_VQ8, synth.FMT_VQ8_M1, synth.FMT_VQ8_M2, synth.FMT_VQ8_M3}
    cbs8 = [synth.vq8_codebooks(wl, p) for p in range(3)] if used & vq8_tags else None
    return build_layer(
        wl.E, wl.H, wl.I, fmt_host,
        nvfp4_weights=lambda e, p: synth.nvfp4_source_weights(wl, e, p),
        vq_codes=lambda e, p: (synth.vq_codes(wl, e, p), synth.vq_scales(wl, e, p)),
        codebooks=cbs,
        vq8_codes=lambda e, p: (synth.vq8_codes(wl, e, p), synth.vq_scales(wl, e, p)),
        codebooks8=cbs8, vq8_m=wl.vq8_m,
        bf16_weights=lambda e, p: synth.bf16_weights(wl, e, p),
        device=device, workers=16, resident_formats=resident_formats,
        nvfp4r_shift=synth.NVFP4R_SHIFT,
        rot_signs=(lambda e: tuple(synth.rot_signs(wl, e, side) for side in range(5)))
        if wl.rot else None, rot_in2_block=wl.rot_in2)


def build_shared_layer(wl, device="cuda"):
    """The workload's BF16 shared expert as a one-expert QLayer."""
    from bit_quantized_moe_route_amd.layers import build_layer

    return build_layer(1, wl.H, wl.I, np.array([synth.FMT_BF16], np.uint8),
                       bf16_weights=lambda e, p: synth.shared_weights_bf16(wl, p),
                       device=device, workers=1)


def oracle_perm(ids, E):
    return oracle.permute(ids, E)
