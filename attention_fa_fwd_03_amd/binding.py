"""ctypes marshalling of torch tensors into libfa.so (include/fa.h).

Each function takes already-allocated device tensors (outputs included),
checks the torch-level facts the C ABI cannot see (device residency, dtype,
contiguity, exact shapes), and passes raw pointers, sizes and the current HIP
stream.  All size/limit/aliasing validation and all computation happen in
libfa.so.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libfa.so")
if not os.path.exists(library_path):
    raise ImportError(f"{library_path} is missing: build it with `python attention_fa_fwd_03_amd/build.py`")
lib = ctypes.CDLL(library_path)

FA_CAUSAL, FA_WINDOW, FA_ALIBI, FA_SOFTCAP, FA_BLOCK_MASK = 1, 2, 4, 8, 16
FA_BF16, FA_FP8_E4M3 = 0, 1
_ERR = {-1: "FA_ERR_INVALID", -2: "FA_ERR_UNSUPPORTED", -3: "FA_ERR_LIMIT", -4: "FA_ERR_WORKSPACE", -5: "FA_ERR_HIP"}


class FaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERR.get(code, code)}: {msg}")
        self.code = code


class _FaMods(ctypes.Structure):
    _fields_ = [
        ("flags", ctypes.c_uint32),
        ("softmax_scale", ctypes.c_float),
        ("alibi_slope", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("window_left", ctypes.c_int64),
        ("window_right", ctypes.c_int64),
        ("block_mask", ctypes.c_void_p),
        ("mask_block_q", ctypes.c_int64),
        ("mask_block_k", ctypes.c_int64),
        ("mask_nqb", ctypes.c_int64),
        ("mask_nkb", ctypes.c_int64),
    ]


class _FaPagedOpts(ctypes.Structure):
    _fields_ = [
        ("q_dtype", ctypes.c_int),
        ("q_descale", ctypes.c_void_p),
        ("page_layout", ctypes.c_int32),
    ]


FA_PAGES_HEAD_MAJOR, FA_PAGES_VECTORIZED = 0, 1

_vp, _i64, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
lib.fa_fwd_dense.argtypes = [_vp] * 5 + [_i64] * 7 + [ctypes.POINTER(_FaMods), _vp]
lib.fa_fwd_dense.restype = ctypes.c_int
lib.fa_fwd_varlen.argtypes = [_vp] * 7 + [_i64] * 9 + [ctypes.POINTER(_FaMods), _vp]
lib.fa_fwd_varlen.restype = ctypes.c_int
lib.fa_fwd_paged.argtypes = ([_vp] * 8 + [_i64] * 11 + [ctypes.c_int, _vp, _vp, _vp, _sz,
                                                         ctypes.POINTER(_FaMods), _vp])
lib.fa_fwd_paged.restype = ctypes.c_int
lib.fa_fwd_paged_noalloc.argtypes = ([_vp] * 8 + [_i64] * 11 + [ctypes.c_int, _vp, _vp, ctypes.POINTER(_FaMods),
                                                                 _vp])
lib.fa_fwd_paged_noalloc.restype = ctypes.c_int
lib.fa_fwd_paged_vec.argtypes = lib.fa_fwd_paged.argtypes
lib.fa_fwd_paged_vec.restype = ctypes.c_int
lib.fa_fwd_paged_ex.argtypes = ([_vp] * 8 + [_i64] * 11 + [ctypes.c_int, _vp, _vp, _vp, _sz,
                                                            ctypes.POINTER(_FaPagedOpts), ctypes.POINTER(_FaMods), _vp])
lib.fa_fwd_paged_ex.restype = ctypes.c_int
lib.fa_kv_cache_write_fp8.argtypes = ([_vp] * 3 + [_i64] * 4 + [_vp, _vp, _i64, _i64, ctypes.c_int32, _vp, _vp,
                                                                 ctypes.c_int32, _vp, _sz, _vp])
lib.fa_kv_cache_write_fp8.restype = ctypes.c_int
lib.fa_kv_cache_write_fp8_workspace_size.argtypes = [_i64] * 4
lib.fa_kv_cache_write_fp8_workspace_size.restype = _sz
lib.fa_bwd_dense.argtypes = [_vp] * 9 + [_i64] * 7 + [ctypes.POINTER(_FaMods), _vp, _sz, _vp]
lib.fa_bwd_dense.restype = ctypes.c_int
lib.fa_bwd_varlen.argtypes = [_vp] * 11 + [_i64] * 9 + [ctypes.POINTER(_FaMods), _vp, _sz, _vp]
lib.fa_bwd_varlen.restype = ctypes.c_int
lib.fa_bwd_workspace_size.argtypes = [_i64, _i64]
lib.fa_bwd_workspace_size.restype = _sz
lib.fa_fwd_paged_workspace_size.argtypes = [_i64] * 9 + [ctypes.c_int]
lib.fa_fwd_paged_workspace_size.restype = _sz
lib.fa_last_error.argtypes = []
lib.fa_last_error.restype = ctypes.c_char_p
lib.fa_abi_version.argtypes = []
lib.fa_abi_version.restype = ctypes.c_int


def fa_last_error() -> str:
    return lib.fa_last_error().decode()


def fa_abi_version() -> int:
    return lib.fa_abi_version()


class Mods:
    """Python view of fa_mods (score mods and masks, values are runtime)."""

    def __init__(self, causal=False, window=None, alibi_slope=None, softcap=None,
                 block_mask=None, mask_block=(128, 128), scale=None):
        self.causal = causal
        self.window = window
        self.alibi_slope = alibi_slope
        self.softcap = softcap
        self.block_mask = block_mask
        self.mask_block = mask_block
        self.scale = scale

    def to_c(self) -> _FaMods:
        m = _FaMods()
        f = 0
        if self.causal:
            f |= FA_CAUSAL
        if self.window is not None:
            f |= FA_WINDOW
            m.window_left, m.window_right = int(self.window[0]), int(self.window[1])
        if self.alibi_slope is not None:
            f |= FA_ALIBI
            m.alibi_slope = float(self.alibi_slope)
        if self.softcap is not None:
            f |= FA_SOFTCAP
            m.softcap = float(self.softcap)
        if self.block_mask is not None:
            bm = self.block_mask
            _need(bm, "block_mask", torch.uint8)
            f |= FA_BLOCK_MASK
            m.block_mask = bm.data_ptr()
            m.mask_block_q, m.mask_block_k = int(self.mask_block[0]), int(self.mask_block[1])
            m.mask_nqb, m.mask_nkb = int(bm.shape[-2]), int(bm.shape[-1])
        m.flags = f
        m.softmax_scale = float(self.scale) if self.scale else 0.0
        return m


def _need(t, name, dtype=None, shape=None):
    # the common case in one expression; the explanation only on failure
    if (isinstance(t, torch.Tensor) and t.is_cuda and (dtype is None or t.dtype == dtype)
            and (shape is None or t.shape == tuple(shape)) and t.is_contiguous()):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


# the current stream's raw handle without building a torch Stream object
# (about 2 us per call otherwise); torch.cuda.current_stream where absent
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, dev):
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(dev.index if dev.index is not None else torch.cuda.current_device())
        return torch.cuda.current_stream(dev).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _mods(mods):
    if mods is None:
        return None
    return ctypes.byref(mods.to_c() if isinstance(mods, Mods) else mods)


def _check(rc):
    if rc != 0:
        raise FaError(rc, fa_last_error())


def fa_fwd_dense(q, k, v, o, lse, mods=None, stream=None):
    """O [B,Sq,Hq,Dv] and LSE [B,Hq,Sq] of dense BSHD attention (see include/fa.h)."""
    B, Sq, Hq, Dqk = q.shape
    Skv, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, Skv, Hkv, Dqk))
    _need(v, "v", torch.bfloat16, (B, Skv, Hkv, Dv))
    _need(o, "o", torch.bfloat16, (B, Sq, Hq, Dv))
    _need(lse, "lse", torch.float32, (B, Hq, Sq))
    _check(lib.fa_fwd_dense(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            B, Sq, Skv, Hq, Hkv, Dqk, Dv, _mods(mods), _stream(stream, q.device)))


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                  mods=None, stream=None):
    """O [Tq,Hq,Dv] and LSE [Hq,Tq] of packed varlen attention (see include/fa.h)."""
    Tq, Hq, Dqk = q.shape
    Tk, Hkv, Dv = k.shape[0], k.shape[1], v.shape[2]
    B = cu_seqlens_q.shape[0] - 1
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (Tk, Hkv, Dqk))
    _need(v, "v", torch.bfloat16, (Tk, Hkv, Dv))
    _need(o, "o", torch.bfloat16, (Tq, Hq, Dv))
    _need(lse, "lse", torch.float32, (Hq, Tq))
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, (B + 1,))
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, (B + 1,))
    _check(lib.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, Tq, Tk,
                             int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, Dqk, Dv,
                             _mods(mods), _stream(stream, q.device)))


def fa_fwd_paged_workspace_size(B, total_q, max_seqlen_q, max_seqlen_k, Hq, Hkv, d_qk, d_v, page_size,
                                kv_dtype=FA_FP8_E4M3) -> int:
    return int(lib.fa_fwd_paged_workspace_size(B, total_q, max_seqlen_q, max_seqlen_k, Hq, Hkv, d_qk, d_v,
                                               page_size, kv_dtype))


def fa_fwd_paged(q, k_cache, v_cache, o, lse, cu_seqlens_q, seqlen_k, block_table, max_seqlen_q, max_seqlen_k,
                 k_descale=None, v_descale=None, workspace=None, mods=None, stream=None, q_descale=None):
    """O [Tq,Hq,Dv] and LSE [Hq,Tq] over a paged cache (see include/fa.h).

    k_cache/v_cache: uint8 (FP8 E4M3 codes) or bf16, [num_pages, Hkv, page_size, D].
    q: bf16, or uint8 E4M3 codes with q_descale (fa_fwd_paged_ex).
    """
    P, Hkv, ps, Dqk = k_cache.shape
    Dv = v_cache.shape[3]
    fp8 = k_cache.dtype == torch.uint8
    cdt = torch.uint8 if fp8 else torch.bfloat16
    _need(k_cache, "k_cache", cdt, (P, Hkv, ps, Dqk))
    _need(v_cache, "v_cache", cdt, (P, Hkv, ps, Dv))
    _paged_call(FA_PAGES_HEAD_MAJOR, q, k_cache, v_cache, o, lse, cu_seqlens_q, seqlen_k, block_table,
                max_seqlen_q, max_seqlen_k, P, Hkv, ps, Dqk, Dv, fp8, k_descale, v_descale, workspace, mods, stream,
                q_descale)


def fa_fwd_paged_noalloc(q, k_cache, v_cache, o, lse, cu_seqlens_q, seqlen_k, block_table, max_seqlen_q,
                         max_seqlen_k, k_descale=None, v_descale=None, mods=None, stream=None):
    """fa_fwd_paged without a workspace (see include/fa.h): bf16 queries,
    head-major pages; the decode path's scratch is the library's static
    device array."""
    P, Hkv, ps, Dqk = k_cache.shape
    Dv = v_cache.shape[3]
    fp8 = k_cache.dtype == torch.uint8
    cdt = torch.uint8 if fp8 else torch.bfloat16
    _need(k_cache, "k_cache", cdt, (P, Hkv, ps, Dqk))
    _need(v_cache, "v_cache", cdt, (P, Hkv, ps, Dv))
    Tq, Hq = q.shape[0], q.shape[1]
    B = cu_seqlens_q.shape[0] - 1
    _need(q, "q", torch.bfloat16, (Tq, Hq, Dqk))
    _need(o, "o", torch.bfloat16, (Tq, Hq, Dv))
    _need(lse, "lse", torch.float32, (Hq, Tq))
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, (B + 1,))
    _need(seqlen_k, "seqlen_k", torch.int32, (B,))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B, max_pages], got {tuple(block_table.shape)}")
    if fp8:
        _need(k_descale, "k_descale", torch.float32)
        _need(v_descale, "v_descale", torch.float32)
    _check(lib.fa_fwd_paged_noalloc(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(), lse.data_ptr(),
        cu_seqlens_q.data_ptr(), seqlen_k.data_ptr(), block_table.data_ptr(),
        B, Tq, int(max_seqlen_q), int(max_seqlen_k), P, ps, block_table.shape[1], Hq, Hkv, Dqk, Dv,
        FA_FP8_E4M3 if fp8 else FA_BF16, k_descale.data_ptr() if fp8 else None,
        v_descale.data_ptr() if fp8 else None, _mods(mods), _stream(stream, q.device)))


def fa_fwd_paged_vec(q, k_cache, v_cache, o, lse, cu_seqlens_q, seqlen_k, block_table, max_seqlen_q,
                     max_seqlen_k, k_descale=None, v_descale=None, workspace=None, mods=None, stream=None,
                     q_descale=None):
    """fa_fwd_paged over vectorised FP8 pages (see include/fa.h).

    k_cache: uint8 [num_pages, Hkv, D_qk/16, page_size, 16];
    v_cache: uint8 [num_pages, Hkv, page_size/16, D_v, 16].
    """
    if k_cache.dim() != 5 or v_cache.dim() != 5:
        raise ValueError("vectorised caches are 5-D")
    P, Hkv, nc, ps, x = k_cache.shape
    Dqk = nc * x
    Dv = v_cache.shape[3]
    _need(k_cache, "k_cache", torch.uint8, (P, Hkv, Dqk // 16, ps, 16))
    _need(v_cache, "v_cache", torch.uint8, (P, Hkv, ps // 16, Dv, 16))
    _paged_call(FA_PAGES_VECTORIZED, q, k_cache, v_cache, o, lse, cu_seqlens_q, seqlen_k, block_table,
                max_seqlen_q, max_seqlen_k, P, Hkv, ps, Dqk, Dv, True, k_descale, v_descale, workspace, mods,
                stream, q_descale)


def _paged_call(layout, q, k_cache, v_cache, o, lse, cu_seqlens_q, seqlen_k, block_table, max_seqlen_q,
                max_seqlen_k, P, Hkv, ps, Dqk, Dv, fp8, k_descale, v_descale, workspace, mods, stream, q_descale):
    """bf16 queries go through fa_fwd_paged / fa_fwd_paged_vec, E4M3 queries
    (uint8) through fa_fwd_paged_ex."""
    Tq, Hq = q.shape[0], q.shape[1]
    B = cu_seqlens_q.shape[0] - 1
    q8 = q.dtype == torch.uint8
    _need(q, "q", torch.uint8 if q8 else torch.bfloat16, (Tq, Hq, Dqk))
    if q8:
        _need(q_descale, "q_descale", torch.float32)
    elif q_descale is not None:
        raise ValueError("q_descale is for uint8 (E4M3) queries")
    _need(o, "o", torch.bfloat16, (Tq, Hq, Dv))
    _need(lse, "lse", torch.float32, (Hq, Tq))
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, (B + 1,))
    _need(seqlen_k, "seqlen_k", torch.int32, (B,))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B, max_pages], got {tuple(block_table.shape)}")
    if fp8:
        _need(k_descale, "k_descale", torch.float32)
        _need(v_descale, "v_descale", torch.float32)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _need(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(), lse.data_ptr(),
            cu_seqlens_q.data_ptr(), seqlen_k.data_ptr(), block_table.data_ptr(),
            B, Tq, int(max_seqlen_q), int(max_seqlen_k), P, ps, block_table.shape[1],
            Hq, Hkv, Dqk, Dv, FA_FP8_E4M3 if fp8 else FA_BF16,
            k_descale.data_ptr() if fp8 else None, v_descale.data_ptr() if fp8 else None,
            ws_ptr or None, ws_bytes)
    if q8:
        opts = _FaPagedOpts(FA_FP8_E4M3, q_descale.data_ptr(), layout)
        _check(lib.fa_fwd_paged_ex(*args, ctypes.byref(opts), _mods(mods), _stream(stream, q.device)))
    else:
        fn = lib.fa_fwd_paged_vec if layout == FA_PAGES_VECTORIZED else lib.fa_fwd_paged
        _check(fn(*args, _mods(mods), _stream(stream, q.device)))


FA_SCALE_GIVEN, FA_SCALE_AMAX = 0, 1


def fa_kv_cache_write_fp8_workspace_size(T, Hkv, d_qk, d_v) -> int:
    return int(lib.fa_kv_cache_write_fp8_workspace_size(T, Hkv, d_qk, d_v))


def fa_kv_cache_write_fp8(k, v, slot_mapping, k_cache, v_cache, k_descale, v_descale, compute_scale=True,
                          workspace=None, stream=None):
    """Quantise bf16 rows k [T,Hkv,Dqk], v [T,Hkv,Dv] to E4M3 and write them
    into uint8 paged caches (see include/fa.h).  Caches: head-major 4-D
    [P,Hkv,page,D] or vectorised 5-D (K [P,Hkv,Dqk/16,page,16], V
    [P,Hkv,page/16,Dv,16]).  compute_scale: write per-tensor descales
    amax/448 first (needs a workspace); else use the ones given."""
    T, Hkv, Dqk = k.shape
    Dv = v.shape[2]
    _need(k, "k", torch.bfloat16)
    _need(v, "v", torch.bfloat16, (T, Hkv, Dv))
    _need(slot_mapping, "slot_mapping", torch.int64, (T,))
    _need(k_descale, "k_descale", torch.float32)
    _need(v_descale, "v_descale", torch.float32)
    if k_cache.dim() == 5:
        P, _, _, ps, _ = k_cache.shape
        _need(k_cache, "k_cache", torch.uint8, (P, Hkv, Dqk // 16, ps, 16))
        _need(v_cache, "v_cache", torch.uint8, (P, Hkv, ps // 16, Dv, 16))
        layout = FA_PAGES_VECTORIZED
    else:
        P, _, ps, _ = k_cache.shape
        _need(k_cache, "k_cache", torch.uint8, (P, Hkv, ps, Dqk))
        _need(v_cache, "v_cache", torch.uint8, (P, Hkv, ps, Dv))
        layout = FA_PAGES_HEAD_MAJOR
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _need(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib.fa_kv_cache_write_fp8(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), T, Hkv, Dqk, Dv,
                                     k_cache.data_ptr(), v_cache.data_ptr(), P, ps, layout,
                                     k_descale.data_ptr(), v_descale.data_ptr(),
                                     FA_SCALE_AMAX if compute_scale else FA_SCALE_GIVEN, ws_ptr or None, ws_bytes,
                                     _stream(stream, k.device)))


def fa_bwd_workspace_size(total_q, Hq) -> int:
    return int(lib.fa_bwd_workspace_size(total_q, Hq))


def _ws(workspace):
    if workspace is None:
        return None, 0
    _need(workspace, "workspace")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def fa_bwd_dense(q, k, v, o, dout, lse, dq, dk, dv, mods=None, workspace=None, stream=None):
    """dQ, dK, dV of the dense forward (see include/fa.h): q/o/dout/dq
    [B,Sq,Hq,D], k/v/dk/dv [B,Skv,Hkv,D] bf16, lse [B,Hq,Sq] fp32."""
    B, Sq, Hq, Dqk = q.shape
    _, Skv, Hkv, Dv = v.shape
    for t, n, shp in ((q, "q", None), (k, "k", (B, Skv, Hkv, Dqk)), (v, "v", None), (o, "o", (B, Sq, Hq, Dv)),
                      (dout, "dout", (B, Sq, Hq, Dv)), (dq, "dq", tuple(q.shape)), (dk, "dk", tuple(k.shape)),
                      (dv, "dv", tuple(v.shape))):
        _need(t, n, torch.bfloat16, shp)
    _need(lse, "lse", torch.float32, (B, Hq, Sq))
    ws, wsb = _ws(workspace)
    _check(lib.fa_bwd_dense(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Sq, Skv, Hq, Hkv, Dqk, Dv, _mods(mods),
                            ws, wsb, _stream(stream, q.device)))


def fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                  mods=None, workspace=None, stream=None):
    """dQ, dK, dV of the varlen forward: q/o/dout/dq [Tq,Hq,D], k/v/dk/dv
    [Tk,Hkv,D] bf16, lse [Hq,Tq] fp32."""
    Tq, Hq, Dqk = q.shape
    Tk, Hkv, Dv = v.shape
    B = cu_seqlens_q.shape[0] - 1
    for t, n, shp in ((q, "q", None), (k, "k", (Tk, Hkv, Dqk)), (v, "v", None), (o, "o", (Tq, Hq, Dv)),
                      (dout, "dout", (Tq, Hq, Dv)), (dq, "dq", tuple(q.shape)), (dk, "dk", tuple(k.shape)),
                      (dv, "dv", tuple(v.shape))):
        _need(t, n, torch.bfloat16, shp)
    _need(lse, "lse", torch.float32, (Hq, Tq))
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, (B + 1,))
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, (B + 1,))
    ws, wsb = _ws(workspace)
    _check(lib.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                             lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_seqlens_q.data_ptr(),
                             cu_seqlens_k.data_ptr(), B, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, Dqk,
                             Dv, _mods(mods), ws, wsb, _stream(stream, q.device)))
