"""CPU fp64 oracle for the FlashAttention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or
executes this package: only the test suite, the smoke check of the graft
entry point and the CPU-baseline leg of the benchmark may use it.  It shares
no code with the HIP library (no kernels, headers, helpers, tables or
constants) and imports nothing from it.

What it computes (all in float64, plain definitions, no blocking or fusion
beyond optional row chunking that does not change any result):

  * scores      s_ij = scale * <q_i, k_j>                      (softmax logits)
  * score mods  soft-cap  s <- c * tanh(s / c), then ALiBi s <- s - slope*|i' - j|
  * visibility  causal j <= i', window i'-W_l <= j <= i'+W_r, block mask tile != 0,
                with bottom-right alignment i' = i + (Skv - Sq)
  * result      LSE_i = log(sum_vis exp(s_ij)),  O_i = sum_vis exp(s_ij - LSE_i) v_j
                rows with no visible key give O_i = 0 and LSE_i = -inf
  * FP8 caches  OCP E4M3 (e4m3fn) bytes decoded bit-field by bit-field, times
                the per-tensor descale
  * split-KV    merging per-split (O_s, LSE_s) partials by their LSE weights
  * backward    dV = P^T dO, dS = P (dO V^T - Delta), dQ = scale dS K, dK = scale dS^T Q
                (oracle.backward)
  * KV write    E4M3 encoding (ties to even, saturating) of x / descale with the
                per-tensor descale amax/448, placed by a slot mapping into
                head-major or vectorised pages (oracle.kvcache)

Sources (pages of the method):
  * "Add forward LSE output to FlyDSL flash attention kernels" (FlyDSL PR 844),
    Summary and Changes: LSE is the per-row log-sum-exp normalisation statistic
    (natural log, in the scaled-logit domain), written for fully masked rows as
    -inf; split-K partials are finalised from per-split (m, l).
  * "SM90 TMA + mma.sync FlashAttention ..." (RL-Kernel PR 237), description:
    packed varlen [total_tokens, H, D] with cu_seqlens; the reference is an
    independent per-sequence masked softmax plus logsumexp; zero-length
    sequences are valid; default softmax scale 1/sqrt(D).
  * "Support paged FP8 Flash attention with asymmetric K/V head dim on gfx950"
    (FlyDSL PR 1066), overview and review: OCP E4M3 K/V with single-value
    descales, Q/K width 192 and V/O width 128, block_table paging, bottom-right
    causal alignment when query and key lengths differ, output zero when the
    softmax denominator is zero.
  * "flash_attention: prologue fusion, mma tensor cores, fp8 KV cache, flex
    attention + block sparsity" (fkl_python PR 7), part 4: ALiBi(slope),
    SoftCap(cap), SlidingWindow(W) score mods and a (bh, nQB, nKB) uint8 tile
    block mask whose inactive tiles contribute nothing.

Readings where the pages are silent are listed with each function.
Every function here is pinned by CPU tests (closed forms, brute force,
library special cases); none is "parity unpinned" except the *semantics* of
the score mods, which the pages name but print no values for.
"""
from .e4m3 import decode_e4m3, encode_e4m3  # noqa: F401
from .kvcache import amax_descale, quantize_rows, kv_cache_write  # noqa: F401
from .backward import attend_bwd, attention_bwd_dense, attention_bwd_varlen  # noqa: F401
from .attention import visible, attend, lse_merge  # noqa: F401
from .layouts import (  # noqa: F401
    attention_dense,
    attention_varlen,
    attention_paged,
    gather_paged,
    varlen_rows,
    paged_rows,
)
