"""Oracle drivers for the three tensor layouts: dense, packed varlen, paged.

Oracle (test infrastructure only).  Each driver gathers one (sequence, head)
at a time from its layout definition and calls attention.attend.

Layouts (readings of the pages, see the package docstring):
  * dense   Q [B,Sq,Hq,Dqk], K [B,Skv,Hkv,Dqk], V [B,Skv,Hkv,Dv];
            O [B,Sq,Hq,Dv], LSE [B,Hq,Sq];
  * varlen  Q [Tq,Hq,Dqk], K [Tk,Hkv,Dqk], V [Tk,Hkv,Dv] packed by
            cu_seqlens_q / cu_seqlens_k (int32 [B+1]); O [Tq,Hq,Dv], LSE [Hq,Tq];
  * paged   Q and O as varlen (cu_seqlens_q); key j of sequence b is slot
            j % page_size of physical page block_table[b, j // page_size] in
            head-major caches K [P,Hkv,page_size,Dqk], V [P,Hkv,page_size,Dv],
            or in the vectorized 5-D caches K [P,Hkv,Dqk/x,page_size,x],
            V [P,Hkv,page_size/x,Dv,x] (see gather_paged); seqlen_k[b] keys;
            FP8 caches hold OCP E4M3 codes scaled by a per-tensor descale;
            Q may be OCP E4M3 codes too (uint8) with its own descale
            ("Support paged FP8 Flash attention with asymmetric K/V head dim
            on gfx950", PR description: E4M3 Q/K/V with scalar descales).
  * GQA     q-head h reads kv-head h // (Hq / Hkv) (consecutive q-heads share
            a kv-head; the pages are silent, Hkv = 1 there).
  * scale   default 1/sqrt(Dqk) (RL-Kernel PR: default softmax scale).
  * block mask [B*Hq, nQB, nKB], row b*Hq + h for sequence b and q-head h.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .attention import visible, attend
from .e4m3 import decode_e4m3

ROW_CHUNK = 1024


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _mods_kw(mods):
    mods = dict(mods or {})
    return dict(
        causal=bool(mods.get("causal", False)),
        window=mods.get("window"),
        softcap=mods.get("softcap"),
        alibi_slope=mods.get("alibi_slope"),
        block_mask=mods.get("block_mask"),
        mask_block=tuple(mods.get("mask_block", (128, 128))),
        scale=mods.get("scale"),
    )


def _one_head(qh, kh, vh, sq, skv, rows, scale, m, bm_slice):
    """Rows `rows` of one (sequence, head): qh [len(rows), dqk], kh [skv, dqk], vh [skv, dv]."""
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.shape[0], vh.shape[1]))
    lse = np.full(rows.shape[0], -np.inf)
    for a in range(0, rows.shape[0], ROW_CHUNK):
        r = rows[a:a + ROW_CHUNK]
        vis = visible(sq, skv, r, causal=m["causal"], window=m["window"],
                      block_mask=bm_slice, mask_block=m["mask_block"])
        ip = r + (skv - sq)
        o[a:a + ROW_CHUNK], lse[a:a + ROW_CHUNK] = attend(
            qh[a:a + ROW_CHUNK], kh, vh, scale, vis,
            softcap=m["softcap"], alibi_slope=m["alibi_slope"], ip=ip)
    return o, lse


def _run(units, fn, workers):
    if workers and workers > 1:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, units))
    return [fn(u) for u in units]


def attention_dense(q, k, v, mods=None, workers=1):
    """Dense BSHD attention.  Returns (O [B,Sq,Hq,Dv], LSE [B,Hq,Sq]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Hq, Dqk = q.shape
    _, Skv, Hkv, Dv = v.shape
    m = _mods_kw(mods)
    scale = m["scale"] if m["scale"] else 1.0 / math.sqrt(Dqk)
    grp = Hq // Hkv
    o = np.zeros((B, Sq, Hq, Dv))
    lse = np.full((B, Hq, Sq), -np.inf)

    def unit(bh):
        b, h = bh
        g = h // grp
        bm = None if m["block_mask"] is None else np.asarray(m["block_mask"])[b * Hq + h]
        return _one_head(q[b, :, h], k[b, :, g], v[b, :, g], Sq, Skv, np.arange(Sq), scale, m, bm)

    units = [(b, h) for b in range(B) for h in range(Hq)]
    for (b, h), (ob, lb) in zip(units, _run(units, unit, workers)):
        o[b, :, h], lse[b, h] = ob, lb
    return o, lse


def attention_varlen(q, k, v, cu_q, cu_k, mods=None, workers=1):
    """Packed varlen attention.  Returns (O [Tq,Hq,Dv], LSE [Hq,Tq]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    B = cu_q.shape[0] - 1
    Tq, Hq, Dqk = q.shape
    _, Hkv, Dv = v.shape
    m = _mods_kw(mods)
    scale = m["scale"] if m["scale"] else 1.0 / math.sqrt(Dqk)
    grp = Hq // Hkv
    o = np.zeros((Tq, Hq, Dv))
    lse = np.full((Hq, Tq), -np.inf)

    def unit(bh):
        b, h = bh
        g = h // grp
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        bm = None if m["block_mask"] is None else np.asarray(m["block_mask"])[b * Hq + h]
        return _one_head(q[q0:q1, h], k[k0:k1, g], v[k0:k1, g], q1 - q0, k1 - k0,
                         np.arange(q1 - q0), scale, m, bm)

    units = [(b, h) for b in range(B) for h in range(Hq) if cu_q[b + 1] > cu_q[b]]
    for (b, h), (ob, lb) in zip(units, _run(units, unit, workers)):
        o[cu_q[b]:cu_q[b + 1], h], lse[h, cu_q[b]:cu_q[b + 1]] = ob, lb
    return o, lse


def varlen_rows(q, k, v, cu_q, cu_k, picks, mods=None):
    """Selected rows of packed varlen attention.

    picks: iterable of (b, h, i) with i the row within sequence b.
    Returns (O [n, Dv], LSE [n]) in the order of `picks`.
    """
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    Hq, Dqk = q.shape[1], q.shape[2]
    Hkv, Dv = v.shape[1], v.shape[2]
    m = _mods_kw(mods)
    scale = m["scale"] if m["scale"] else 1.0 / math.sqrt(Dqk)
    grp = Hq // Hkv
    picks = list(picks)
    o = np.zeros((len(picks), Dv))
    lse = np.full(len(picks), -np.inf)
    groups = {}
    for n, (b, h, i) in enumerate(picks):
        groups.setdefault((b, h), []).append((n, i))
    for (b, h), lst in groups.items():
        g = h // grp
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        rows = np.array([i for _, i in lst])
        bm = None if m["block_mask"] is None else np.asarray(m["block_mask"])[b * Hq + h]
        ob, lb = _one_head(_f64(q[q0 + rows, h]), _f64(k[k0:k1, g]), _f64(v[k0:k1, g]),
                           q1 - q0, k1 - k0, rows, scale, m, bm)
        for t, (n, _) in enumerate(lst):
            o[n], lse[n] = ob[t], lb[t]
    return o, lse


def paged_queries(q, q_descale=None):
    """Query values of a paged call: bf16 values as they are, or E4M3 codes
    (uint8) decoded and multiplied by the per-tensor q_descale."""
    q = np.asarray(q)
    if q.dtype == np.uint8:
        if q_descale is None:
            raise ValueError("E4M3 queries need q_descale")
        return decode_e4m3(q) * float(q_descale)
    if q_descale is not None:
        raise ValueError("q_descale applies to E4M3 queries only")
    return _f64(q)


def gather_paged(cache, block_row, length, g, descale=None, layout="head_major", kind="k"):
    """Token-major [length, D] float64 rows of kv-head g for one sequence.

    Key j is slot s = j % ps of page p = block_row[j // ps].  Layouts:
      * head_major  cache [P, Hkv, ps, D]: element (j, d) at [p, g, s, d];
      * vectorized  (the 5-D page layout of "Support paged FP8 Flash attention
        with asymmetric K/V head dim on gfx950", review of the interface:
        a K page is [Hkv, D/16, ps, 16] and a V page [Hkv, ps/16, Dv, 16],
        16 one-byte codes per vector; x = the last extent):
          kind "k": cache [P, Hkv, D/x, ps, x], element (j, d) at [p, g, d // x, s, d % x]
          kind "v": cache [P, Hkv, ps/x, Dv, x], element (j, d) at [p, g, s // x, d, s % x]
    FP8 caches (uint8) are decoded as OCP E4M3 and multiplied by `descale`
    in float64.
    """
    cache = np.asarray(cache)
    j = np.arange(length)
    if layout == "head_major":
        ps = cache.shape[2]
        pages = np.asarray(block_row, dtype=np.int64)[j // ps]
        raw = cache[pages, g, j % ps]
    elif layout == "vectorized" and kind == "k":
        x, ps = cache.shape[4], cache.shape[3]
        d = np.arange(cache.shape[2] * x)
        pages = np.asarray(block_row, dtype=np.int64)[j // ps]
        raw = cache[pages[:, None], g, (d // x)[None, :], (j % ps)[:, None], (d % x)[None, :]]
    elif layout == "vectorized" and kind == "v":
        x = cache.shape[4]
        ps = cache.shape[2] * x
        d = np.arange(cache.shape[3])
        pages = np.asarray(block_row, dtype=np.int64)[j // ps]
        s = j % ps
        raw = cache[pages[:, None], g, (s // x)[:, None], d[None, :], (s % x)[:, None]]
    else:
        raise ValueError(f"unknown paged layout {layout!r} / kind {kind!r}")
    if raw.dtype == np.uint8:
        out = decode_e4m3(raw)
        if descale is not None:
            out = out * float(descale)
        return out
    return _f64(raw)


def attention_paged(q, k_cache, v_cache, cu_q, seqlen_k, block_table, mods=None,
                    k_descale=None, v_descale=None, workers=1, layout="head_major", q_descale=None):
    """Paged-KV attention over either page layout (see gather_paged), with
    bf16 or E4M3 queries (see paged_queries).
    Returns (O [Tq,Hq,Dv], LSE [Hq,Tq]) in float64."""
    q = paged_queries(q, q_descale)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    seqlen_k = np.asarray(seqlen_k, dtype=np.int64)
    block_table = np.asarray(block_table, dtype=np.int64)
    B = cu_q.shape[0] - 1
    Tq, Hq, Dqk = q.shape
    Hkv, Dv = v_cache.shape[1], v_cache.shape[3]
    m = _mods_kw(mods)
    scale = m["scale"] if m["scale"] else 1.0 / math.sqrt(Dqk)
    grp = Hq // Hkv
    o = np.zeros((Tq, Hq, Dv))
    lse = np.full((Hq, Tq), -np.inf)

    def unit(bg):
        b, g = bg
        L = int(seqlen_k[b])
        kh = gather_paged(k_cache, block_table[b], L, g, k_descale, layout, "k")
        vh = gather_paged(v_cache, block_table[b], L, g, v_descale, layout, "v")
        q0, q1 = cu_q[b], cu_q[b + 1]
        res = []
        for h in range(g * grp, (g + 1) * grp):
            bm = None if m["block_mask"] is None else np.asarray(m["block_mask"])[b * Hq + h]
            res.append(_one_head(q[q0:q1, h], kh, vh, q1 - q0, L, np.arange(q1 - q0), scale, m, bm))
        return res

    units = [(b, g) for b in range(B) for g in range(Hkv) if cu_q[b + 1] > cu_q[b]]
    for (b, g), res in zip(units, _run(units, unit, workers)):
        for t, (ob, lb) in enumerate(res):
            h = g * grp + t
            o[cu_q[b]:cu_q[b + 1], h], lse[h, cu_q[b]:cu_q[b + 1]] = ob, lb
    return o, lse


def paged_rows(q, k_cache, v_cache, cu_q, seqlen_k, block_table, picks, mods=None,
               k_descale=None, v_descale=None, layout="head_major", q_descale=None):
    """Selected rows (b, h, i) of paged attention over either page layout;
    returns (O [n, Dv], LSE [n])."""
    q = paged_queries(q, q_descale)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    seqlen_k = np.asarray(seqlen_k, dtype=np.int64)
    block_table = np.asarray(block_table, dtype=np.int64)
    Hq, Dqk = q.shape[1], q.shape[2]
    Hkv, Dv = v_cache.shape[1], v_cache.shape[3]
    m = _mods_kw(mods)
    scale = m["scale"] if m["scale"] else 1.0 / math.sqrt(Dqk)
    grp = Hq // Hkv
    picks = list(picks)
    o = np.zeros((len(picks), Dv))
    lse = np.full(len(picks), -np.inf)
    groups = {}
    for n, (b, h, i) in enumerate(picks):
        groups.setdefault((b, h), []).append((n, i))
    gathered = {}
    for (b, h), lst in groups.items():
        g = h // grp
        L = int(seqlen_k[b])
        if (b, g) not in gathered:
            gathered = {(b, g): (gather_paged(k_cache, block_table[b], L, g, k_descale, layout, "k"),
                                 gather_paged(v_cache, block_table[b], L, g, v_descale, layout, "v"))}
        kh, vh = gathered[(b, g)]
        q0, q1 = cu_q[b], cu_q[b + 1]
        rows = np.array([i for _, i in lst])
        bm = None if m["block_mask"] is None else np.asarray(m["block_mask"])[b * Hq + h]
        ob, lb = _one_head(_f64(q[q0 + rows, h]), kh, vh, q1 - q0, L, rows, scale, m, bm)
        for t, (n, _) in enumerate(lst):
            o[n], lse[n] = ob[t], lb[t]
    return o, lse
