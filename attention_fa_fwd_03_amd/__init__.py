"""MI355X (gfx950) FlashAttention forward: thin Python binding over libfa.so.

The functions here only marshal torch tensors into the C ABI declared in
include/fa.h; every step of the computation runs in the HIP kernels of
libfa.so.  Importing this package raises if the shared library has not been
built (python attention_fa_fwd_03_amd/build.py): there is no fallback path.
"""
from .binding import (  # noqa: F401
    FaError,
    FA_CAUSAL,
    FA_WINDOW,
    FA_ALIBI,
    FA_SOFTCAP,
    FA_BLOCK_MASK,
    FA_BF16,
    FA_FP8_E4M3,
    Mods,
    fa_fwd_dense,
    fa_fwd_varlen,
    fa_fwd_paged,
    fa_fwd_paged_noalloc,
    fa_fwd_paged_vec,
    FA_PAGES_HEAD_MAJOR,
    FA_PAGES_VECTORIZED,
    fa_fwd_paged_workspace_size,
    fa_kv_cache_write_fp8,
    fa_bwd_dense,
    fa_bwd_varlen,
    fa_bwd_workspace_size,
    fa_kv_cache_write_fp8_workspace_size,
    FA_SCALE_GIVEN,
    FA_SCALE_AMAX,
    fa_last_error,
    fa_abi_version,
    library_path,
    lib,
)
