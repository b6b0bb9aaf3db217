"""Shared test helpers: tensor conversion and oracle comparison."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances (max-abs).  bf16 inputs: O 2e-2, LSE 5e-3.  FP8 caches: O 6e-2
# against the oracle fed the same dequantised K/V; LSE 5e-3 (K is converted
# exactly from E4M3 to bf16 and Q stays bf16, so the logits carry only fp32
# accumulation error).
TOL_O_BF16 = 2e-2
TOL_LSE = 5e-3
TOL_O_FP8 = 6e-2


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a (CPU or device) tensor; uint8 stays uint8."""
    t = t.detach().cpu()
    if t.dtype == torch.uint8:
        return t.numpy()
    return t.to(torch.float64).numpy()


def compare(o_gpu, lse_gpu, o_ref, lse_ref, tol_o, tol_lse=TOL_LSE, what=""):
    """Element-wise comparison with exact handling of empty rows.

    o_gpu/o_ref: [..., Dv] rows aligned with lse_gpu/lse_ref [...].
    Rows the oracle marks empty (LSE = -inf) must have LSE exactly -inf and
    O exactly 0 on the GPU.  No NaN anywhere.
    """
    o_g, l_g = f64(o_gpu) if isinstance(o_gpu, torch.Tensor) else o_gpu, \
        f64(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    assert not np.isnan(o_g).any(), f"{what}: NaN in O"
    assert not np.isnan(l_g).any(), f"{what}: NaN in LSE"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l_g), empty), \
        f"{what}: -inf rows differ ({int(np.isneginf(l_g).sum())} vs {int(empty.sum())})"
    if empty.any():
        assert np.all(o_g[empty] == 0.0), f"{what}: empty rows must give O = 0"
    fin = ~empty
    err_l = float(np.max(np.abs(l_g[fin] - lse_ref[fin]))) if fin.any() else 0.0
    err_o = float(np.max(np.abs(o_g - o_ref))) if o_g.size else 0.0
    assert err_l <= tol_lse, f"{what}: LSE max-abs {err_l:.3e} > {tol_lse}"
    assert err_o <= tol_o, f"{what}: O max-abs {err_o:.3e} > {tol_o}"
    return err_o, err_l
