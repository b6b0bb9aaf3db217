"""FP8 E4M3 KV-cache write: quantise token-major K/V rows and place them in
paged caches.

Oracle (test infrastructure only).  Sources: "flash_attention: prologue
fusion, mma tensor cores, fp8 KV cache, flex attention + block sparsity"
(fkl_python PR 7), part 3: a GPU quantisation kernel turns K/V into E4M3
with a scale from the largest magnitude over 448; "Support paged FP8 Flash
attention with asymmetric K/V head dim on gfx950" (FlyDSL PR 1066), overview
and tests: per-tensor descale = amax / 448, paged caches addressed through
the block table, head-major or vectorised 5-D pages.

Readings (the pages give the scale rule, not the arithmetic order):
  * descale = max(amax / 448, 2^-126) in fp32 (the floor keeps 1/descale
    finite when every value is zero), amax = max |x| over all rows written;
    or a descale the caller gives;
  * code = E4M3(x * (1 / descale)), both operations fp32 rounded to nearest,
    the conversion ties-to-even and saturating at 448 (encode_e4m3);
  * token t goes to page slot_mapping[t] // page_size, slot
    slot_mapping[t] % page_size; a negative entry skips the token, as does
    one past the cache; with no rows at all nothing is written, descales
    included.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import E4M3_MAX, encode_e4m3

FLT_MIN = np.float32(2.0 ** -126)


def amax_descale(x) -> np.float32:
    """Per-tensor descale max(amax / 448, 2^-126), fp32."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    return max(np.float32(amax / np.float32(E4M3_MAX)), FLT_MIN)


def quantize_rows(x, descale) -> np.ndarray:
    """E4M3 codes of x * (1 / descale) (fp32 steps, see the module notes)."""
    inv = np.float32(1.0) / np.float32(descale)
    return encode_e4m3(np.asarray(x, dtype=np.float32) * inv)


def kv_cache_write(k, v, slot_mapping, k_cache, v_cache, page_size, layout="head_major",
                   k_descale=None, v_descale=None):
    """Write rows k [T,Hkv,Dqk], v [T,Hkv,Dv] (float values) into copies of
    the uint8 caches.  Descales None: computed from k / v (amax rule);
    otherwise used as given.  Returns (k_cache, v_cache, k_descale, v_descale).

    Layouts: head_major K/V [P,Hkv,page,D]; vectorized K [P,Hkv,Dqk/16,page,16],
    V [P,Hkv,page/16,Dv,16]."""
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    slot_mapping = np.asarray(slot_mapping, dtype=np.int64)
    kc, vc = np.array(k_cache, dtype=np.uint8, copy=True), np.array(v_cache, dtype=np.uint8, copy=True)
    if k.shape[0] == 0:                   # nothing to write: caches and descales untouched
        return kc, vc, k_descale, v_descale
    kd = amax_descale(k) if k_descale is None else np.float32(k_descale)
    vd = amax_descale(v) if v_descale is None else np.float32(v_descale)
    kq, vq = quantize_rows(k, kd), quantize_rows(v, vd)
    P = kc.shape[0]
    Dqk, Dv = k.shape[2], v.shape[2]
    for t, sl in enumerate(slot_mapping):
        if sl < 0 or sl >= P * page_size:
            continue
        p, s = divmod(int(sl), page_size)
        if layout == "head_major":
            kc[p, :, s, :] = kq[t]
            vc[p, :, s, :] = vq[t]
        else:
            for c in range(Dqk // 16):
                kc[p, :, c, s, :] = kq[t, :, 16 * c:16 * c + 16]
            vc[p, :, s // 16, :, s % 16] = vq[t]
    return kc, vc, kd, vd
