"""Seeded synthetic inputs for the attention forward workloads.

This module holds no attention arithmetic.  It only draws random tensors,
builds the length/page metadata and quantises K/V to OCP E4M3 bytes, so that
the CPU oracle and the HIP path consume exactly the same inputs.

Recipes (seed = 1000 + 10*config + subcase):
  * values: torch.randn (fp32) from a seeded CPU generator, rounded to bf16 RNE;
  * fp8 K/V caches: N(0,1) data divided by a per-tensor descale = amax/448 and
    cast with torch's float8_e4m3fn conversion (round to nearest even); the
    bytes are what both sides read, so the quantiser's rounding is not part of
    any comparison;
  * varlen lengths: uniform integers, with one forced zero length and at least
    three lengths that are not multiples of 64;
  * paged caches: head-major pages [num_pages, Hkv, page_size, D] whose
    placement is a seeded random permutation (the block table);
  * block masks: uint8 [B*Hq, nQB, nKB], Bernoulli(p) or block-causal.
"""
from .gen import (  # noqa: F401
    to_vectorized,
    seed_for,
    randn_bf16,
    quantize_e4m3,
    varlen_lengths,
    cu_from_lengths,
    make_dense,
    make_varlen,
    make_paged,
    make_decode_lengths,
    bernoulli_block_mask,
    block_causal_mask,
    peaked_queries,
)
