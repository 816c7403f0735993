"""Oracle-side helpers for the parity tests and the CPU baseline: decode one
expert's weights from the seeded workload with the oracle's own encoder and
decoders, and evaluate the oracle FFN for given token rows.  Imports only
numpy, the oracle and the input generators (safe to run in spawned worker
processes that never touch the GPU)."""

import os

import numpy as np

import oracle
import synth


def expert_weights(wl, e, fmt=None):
    """(W_gate, W_up, W_down) float64 of expert e of workload wl, decoded by
    the oracle from the same seeded inputs the GPU layer was built from."""
    if fmt is None:
        fmt = int(synth.tier_map(wl)[e])
    mats = []
    for p in (synth.PROJ_GATE, synth.PROJ_UP, synth.PROJ_DOWN):
        if fmt == synth.FMT_NVFP4:
            c, s = oracle.nvfp4_quantize(synth.nvfp4_source_weights(wl, e, p))
            mats.append(oracle.nvfp4_dequant(c, s))
        elif fmt == synth.FMT_NVFP4R:
            base, res = oracle.nvfp4_residual_quantize(synth.nvfp4_source_weights(wl, e, p),
                                                       synth.NVFP4R_SHIFT)
            mats.append(oracle.nvfp4r_dequant(base, res, synth.NVFP4R_SHIFT))
        elif fmt == synth.FMT_BF16:
            mats.append(oracle.bf16_bits_to_f64(synth.bf16_weights(wl, e, p)))
        elif fmt == synth.FMT_VQ8:
            mats.append(oracle.vq8_dequant(synth.vq8_codes(wl, e, p), synth.vq_scales(wl, e, p),
                                           synth.vq8_codebooks(wl, p)))
        elif fmt in (synth.FMT_VQ8_M1, synth.FMT_VQ8_M2, synth.FMT_VQ8_M3):
            mats.append(oracle.vq8_rate_dequant(synth.vq8_codes(wl, e, p),
                                                synth.vq_scales(wl, e, p),
                                                synth.vq8_codebooks(wl, p)))
        else:
            mats.append(oracle.vq_dequant(synth.vq_codes(wl, e, p), synth.vq_scales(wl, e, p),
                                          synth.vq_codebook(wl, p)))
    if wl.rot:
        # rotated storage: the effective weights are R_out^T W_rot R_in
        s = {side: synth.rot_signs(wl, e, side) for side in range(5)}
        mats = [oracle.unrotate_weights(mats[0], s[synth.ROT_OUT_GATE], s[synth.ROT_IN13]),
                oracle.unrotate_weights(mats[1], s[synth.ROT_OUT_UP], s[synth.ROT_IN13]),
                oracle.unrotate_weights(mats[2], s[synth.ROT_OUT2], s[synth.ROT_IN2],
                                        block_in=wl.rot_in2)]
    return tuple(mats)


def stored_weights(wl, e, fmt=None):
    """The decoded matrices as stored (rotated for a rotated layer)."""
    import dataclasses
    return expert_weights(dataclasses.replace(wl, rot=False), e, fmt)


def shared_weights(wl):
    """(W_gate, W_up, W_down) float64 of the layer's BF16 shared expert."""
    return tuple(oracle.bf16_bits_to_f64(synth.shared_weights_bf16(wl, p))
                 for p in (synth.PROJ_GATE, synth.PROJ_UP, synth.PROJ_DOWN))


def expert_rows(args):
    """Oracle FFN outputs of expert e for the given bf16 token rows."""
    wl_name, e, x_bits, fmt = args
    wl = synth.WORKLOADS[wl_name] if isinstance(wl_name, str) else wl_name
    W = expert_weights(wl, e, fmt)
    return oracle.expert_ffn(x_bits, *W)


def pool_map(jobs, workers=None):
    """Run expert_rows over jobs in spawned processes (numpy only)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    if workers is None:
        workers = 8
    workers = max(1, min(len(jobs), workers, len(os.sched_getaffinity(0))))
    if workers == 1 or len(jobs) == 1:
        return [expert_rows(j) for j in jobs]
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(workers, mp_context=ctx, initializer=_one_blas_thread) as ex:
        return list(ex.map(expert_rows, jobs))


def _one_blas_thread():
    """Pool workers each take one core: BLAS limited to one thread."""
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)
