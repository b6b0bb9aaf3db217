"""Masked softmax attention of one (sequence, head), written from its definition.

Oracle (test infrastructure only).  fp64 numpy; a matrix product is the only
library primitive used as a step.

Readings taken where the pages leave a step open (each also listed in the
design notes of the repository):
  * query row i sees key j relative to i' = i + (Skv - Sq) (bottom-right
    alignment, the "cross_seqlen" causal mask of the paged FP8 PR review);
  * a row with no visible key has O = 0 and LSE = -inf (the paged PR's
    zero-denominator output and the LSE PR's "-inf rows");
  * LSE is the natural-log log-sum-exp of the scaled (and modded) logits
    (LSE PR: sm_scale*m + ln(l); RL-Kernel PR: "attention-domain" M + log L);
  * soft-cap is c*tanh(s/c) on the scaled logit and is applied before ALiBi;
    ALiBi subtracts slope*|i' - j| (one slope for every head);
  * window (W_l, W_r): visible iff i'-W_l <= j <= i'+W_r, a negative bound
    meaning unbounded on that side; SlidingWindow(W) is (W, 0);
  * block mask M[qb, kb] (already sliced to this sequence and head) with tile
    sizes (bq, bk): key j is visible to row i only if M[i // bq, j // bk] != 0.
"""
from __future__ import annotations

import numpy as np


def visible(sq: int, skv: int, rows=None, *, causal=False, window=None,
            block_mask=None, mask_block=(128, 128)) -> np.ndarray:
    """Boolean [len(rows), skv]: is key j visible to query row i.

    rows: query row indices within the sequence (default all of range(sq)).
    """
    i = np.arange(sq) if rows is None else np.asarray(rows, dtype=np.int64)
    ip = i + (skv - sq)
    j = np.arange(skv)
    vis = np.ones((i.shape[0], skv), dtype=bool)
    if causal:
        vis &= j[None, :] <= ip[:, None]
    if window is not None:
        wl, wr = window
        if wl is not None and wl >= 0:
            vis &= j[None, :] >= ip[:, None] - wl
        if wr is not None and wr >= 0:
            vis &= j[None, :] <= ip[:, None] + wr
    if block_mask is not None:
        bq, bk = mask_block
        bm = np.asarray(block_mask)
        vis &= bm[i[:, None] // bq, j[None, :] // bk] != 0
    return vis


def attend(q, k, v, scale, vis, *, softcap=None, alibi_slope=None, ip=None):
    """One sequence and head.

    q [n, dqk], k [m, dqk], v [m, dv] (float64), vis bool [n, m];
    ip [n]: aligned query positions i' (needed by ALiBi).
    Returns (o [n, dv], lse [n]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, m = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)                                   # scaled logits
    if softcap is not None:
        s = softcap * np.tanh(s / softcap)
    if alibi_slope is not None:
        j = np.arange(m)
        s = s - alibi_slope * np.abs(np.asarray(ip, dtype=np.float64)[:, None] - j[None, :])
    s = np.where(vis, s, -np.inf)
    nvis = vis.sum(axis=1)
    has = nvis > 0
    mx = np.where(has, np.max(np.where(vis, s, -np.inf), axis=1, initial=-np.inf), 0.0)
    e = np.where(vis, np.exp(s - mx[:, None]), 0.0)
    den = e.sum(axis=1)
    lse = np.where(has, mx + np.log(np.where(has, den, 1.0)), -np.inf)
    p = e / np.where(has, den, 1.0)[:, None]
    o = p @ v
    o[~has] = 0.0
    return o, lse


def lse_merge(parts):
    """Merge attention results computed over disjoint key subsets.

    parts: list of (o_s [n, dv], lse_s [n]) where o_s is normalised by its own
    denominator.  With m = max_s lse_s: LSE = m + log(sum_s exp(lse_s - m)) and
    O = sum_s exp(lse_s - LSE) * o_s.  Subsets with no visible key carry
    lse_s = -inf and weigh zero (LSE PR: split-K partials finalised from (m, l)).
    """
    lses = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])      # [S, n]
    outs = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])      # [S, n, dv]
    m = np.max(lses, axis=0)
    has = np.isfinite(m)
    mm = np.where(has, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - mm[None, :]), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(has, mm + np.log(np.where(has, tot, 1.0)), -np.inf)
    o = np.einsum("sn,snd->nd", w / np.where(has, tot, 1.0)[None, :], outs)
    o[~has] = 0.0
    return o, lse
