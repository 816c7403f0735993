"""Plain, slow, obviously-correct CPU oracle for the routed-expert MoE forward
over low-bit expert weights.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may call it.  It shares no code, table or helper with the HIP library
(``bit_quantized_moe_route_amd``), and it never takes an input or an expected
value from that library.

Everything is numpy in float64.  Each function cites the passage of the pages
it follows:

* GLM-5-NVFP4-MTP, "Model Description" -- 256 experts per MoE layer, 8 active
  per token; NVFP4 = 4-bit codes with blockwise FP8 scales per 16 elements.
* GLM-5-NVFP4-MTP, "What's quantized" -- only the expert MLP (gate, up, down
  projections) is quantized.
* GLM-5.2 mixed-bit VQ (AQLM) ~1.90 bpw, "What it is" -- AQLM-style per-group
  codes into a shared codebook.
* GLM-5.3-Flash-TR3-8bpw (K8), "Fidelity" / "Excess over control" -- the
  expert-combine order changes the bits, so the combine order is fixed.
* GLM-5.3-EXL3-TR3-3.42bpw, "What is quantized" -- BF16 shared experts beside
  the routed ones.
* GLM-5.3 Vision NestQuant 1.75-4 bit, "Method" -- random signs and a
  Hadamard-128 transform on both sides of each weight matrix; introduction --
  a nested two-level format: a base plus a residual plane on top of it.

Where the pages are silent the oracle takes the plainest reading, stated in
the docstring of the function that makes it.

Parity status per function (what pins each one is in tests/test_oracle_*.py):
  e2m1_decode, e4m3_decode, e4m3_encode, nvfp4_quantize, nvfp4_dequant,
  vq_dequant, vq8_dequant, route_topk, permute, expert_ffn, combine,
  combine_shared, forward, hadamard, rotate, unrotate, rotate_weights,
  unrotate_weights, nvfp4_residual_quantize, nvfp4r_dequant,
  bf16_bits_to_f64, f16_bits_to_f64, vq8_rate_dequant
  -- all pinned.  vq8_dequant's arithmetic is pinned; its code shape (M
  8-bit codes per 8-weight group into M 256-entry codebooks whose rows are
  summed) is a reading the pages do not fix: parity unpinned for the shape;
  so is vq8_rate_dequant's reading that an expert at rate m uses the first
  m of the layer's shared codebooks.
"""

from .formats import (  # noqa: F401
    E2M1_MAGNITUDES,
    e2m1_decode,
    e4m3_decode,
    e4m3_encode,
    e4m3_finite_table,
    nvfp4_quantize,
    nvfp4_dequant,
    nvfp4_residual_quantize,
    nvfp4r_dequant,
    vq_dequant,
    vq8_dequant,
    vq8_rate_dequant,
    bf16_bits_to_f64,
    f16_bits_to_f64,
)
from .rotation import (  # noqa: F401
    hadamard,
    rotate,
    unrotate,
    rotate_weights,
    unrotate_weights,
)
from .moe import (  # noqa: F401
    route_topk,
    permute,
    expert_ffn,
    combine,
    combine_shared,
    forward,
)
