"""Loading a packed expert layer onto the GPU.

Weights come from caller-supplied providers (one projection of one expert at
a time), are encoded and laid out by the library's host packers
(moe_quantize_nvfp4, moe_pack_*_expert) on a thread pool, and are copied
into the layer's device pools.  One expert is resident in host memory per
worker at a time.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import (FMT_BF16, FMT_NVFP4, FMT_NVFP4R, FMT_VQ, FMT_VQ8, FMT_VQ8_RATES, PROJ_DOWN,
               PROJ_GATE, PROJ_UP, vq8_rate,
               QLayer, pack_bf16_expert, pack_nvfp4_expert, pack_nvfp4r_expert, pack_vq8_expert,
               pack_vq_expert, quantize_nvfp4, quantize_nvfp4_residual)


def build_layer(E, H, I, fmt_host, nvfp4_weights=None, vq_codes=None, codebooks=None,
                codebook_stride=0, vq8_codes=None, codebooks8=None, vq8_m=0, bf16_weights=None,
                device="cuda", workers=8, resident_formats=None, rot_signs=None,
                nvfp4r_shift=None, rot_in2_block=128):
    """Build a QLayer.

    nvfp4_weights(e, proj) -> fp32 [n, kin] source weights of an NVFP4 expert
        (proj 0 = gate [I, H], 1 = up [I, H], 2 = down [H, I]), also of a
        nested two-level NVFP4 expert (its base and residual planes are
        quantized from them).
    vq_codes(e, proj) -> (codes uint16 [n, kin/8], scales fp16 bits uint16 [n])
        of a VQ expert.
    codebooks: three uint16 arrays (fp16 bits) [65536 * n_books, 8] for gate,
        up, down.
    vq8_codes(e, proj) -> (codes uint8 [n, kin/8, m], scales fp16 bits [n])
        of a small-codebook VQ expert (m = vq8_m for FMT_VQ8, the tag's rate
        for FMT_VQ8_M1..3); codebooks8: for gate, up, down a list of uint16
        arrays [256, 8], as many as the layer's largest rate.
    bf16_weights(e, proj) -> bf16 bits uint16 [n, kin] of a BF16 expert (a
        routed BF16-tier expert, or the one expert of a shared-expert layer).
    resident_formats: None, or the formats every expert is packed in (slot e of
        each of those pools), for a layer whose tiers change at run time
        (QLayer.set_tiers); {FMT_NVFP4, FMT_NVFP4R} (with others or not) makes
        the layer nested: NVFP4-tier experts run on the base planes of their
        two-level records.
    nvfp4r_shift: the residual-plane exponent of two-level NVFP4 experts
        (default NVFP4R_SHIFT).
    rot_signs(e) -> (s_in13 [H], s_out_gate [I], s_out_up [I], s_in2 [I],
        s_out2 [H]) int8 +-1: the layer's matrices are stored rotated (the
        providers above return the rotated matrices) and these are each
        expert's signs.
    rot_in2_block: the Hadamard block of the down projection's input side of
        a rotated layer (128, or 512 for the wide variant).
    """
    import torch

    from . import NVFP4R_SHIFT
    layer = QLayer(E, H, I, fmt_host, device=device, vq8_m=vq8_m,
                   resident_formats=resident_formats,
                   nvfp4r_shift=NVFP4R_SHIFT if nvfp4r_shift is None else nvfp4r_shift)
    host = {}
    for key, pool in layer.pools.items():
        if pool is not None and key[0] not in layer.alias:
            host[key] = np.zeros(pool.numel(), np.uint8)

    def one(e):
        if layer.resident is not None:
            for fmt in sorted(layer.resident):
                if fmt not in layer.alias:   # a nested layer's base planes
                    pack_one(e, fmt, e)
        else:
            pack_one(e, int(layer.fmt_host[e]), layer.record_index(e))

    def pack_one(e, fmt, idx):
        s13, s2 = layer.stride[(fmt, 0)], layer.stride[(fmt, 1)]
        dst13 = host[(fmt, 0)][idx * s13: idx * s13 + s13]
        dst2 = host[(fmt, 1)][idx * s2: idx * s2 + s2]
        if fmt == FMT_NVFP4:
            parts = [quantize_nvfp4(nvfp4_weights(e, p)) for p in (PROJ_GATE, PROJ_UP, PROJ_DOWN)]
            w13, w2 = pack_nvfp4_expert(parts[0], parts[1], parts[2], H, I)
        elif fmt == FMT_NVFP4R:
            parts = [quantize_nvfp4_residual(nvfp4_weights(e, p), layer.nvfp4r_shift)
                     for p in (PROJ_GATE, PROJ_UP, PROJ_DOWN)]
            w13, w2 = pack_nvfp4r_expert([q[0] for q in parts], [q[1] for q in parts], H, I)
        elif fmt == FMT_BF16:
            parts = [bf16_weights(e, p) for p in (PROJ_GATE, PROJ_UP, PROJ_DOWN)]
            w13, w2 = pack_bf16_expert(parts[0], parts[1], parts[2], H, I)
        elif fmt == FMT_VQ8 or fmt in FMT_VQ8_RATES:
            parts = [vq8_codes(e, p) for p in (PROJ_GATE, PROJ_UP, PROJ_DOWN)]
            w13, w2 = pack_vq8_expert(parts[0], parts[1], parts[2], H, I, vq8_rate(fmt, vq8_m))
        else:
            parts = [vq_codes(e, p) for p in (PROJ_GATE, PROJ_UP, PROJ_DOWN)]
            w13, w2 = pack_vq_expert(parts[0], parts[1], parts[2], H, I)
        dst13[:w13.shape[0]] = w13
        dst2[:w2.shape[0]] = w2

    with ThreadPoolExecutor(max(1, workers)) as ex:
        list(ex.map(one, range(E)))
    for key, arr in host.items():
        layer.pools[key].copy_(torch.from_numpy(arr))
    if rot_signs is not None:
        from . import pack_rot_signs
        layer.set_rot_signs(np.stack([pack_rot_signs(*rot_signs(e), H, I) for e in range(E)]),
                            in2_block=rot_in2_block)
    if layer.pools[(FMT_VQ, 0)] is not None:
        layer.set_codebooks(codebooks, codebook_stride)
    if any(layer.pools[(f, 0)] is not None for f in (FMT_VQ8,) + FMT_VQ8_RATES):
        layer.set_codebooks8(codebooks8)
    if layer.device.type == "cuda":
        torch.cuda.synchronize(layer.device)
    return layer
