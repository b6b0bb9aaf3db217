"""Gradients of the attention forward pass, written from their definition.

Oracle (test infrastructure only).  fp64 numpy.  Sources: "SM90 TMA +
mma.sync FlashAttention, forward + backward (causal, varlen, LSE)"
(RL-Kernel PR 237), backward commit: a Delta preprocess plus dQ/dK/dV,
recomputing the probabilities from the forward's saved LSE; "Add forward LSE
output to FlyDSL flash attention kernels" (FlyDSL PR 844), Summary: LSE is
the statistic the backward pass needs to recompute P.

For one (sequence, head) with O = P V, P = softmax over the visible keys of
S = scale Q K^T, and an upstream gradient dO:
    dV = P^T dO,   dP = dO V^T,   Delta_i = sum_j P_ij dP_ij (= dO_i . O_i),
    dS = P * (dP - Delta),   dQ = scale dS K,   dK = scale dS^T Q.
GQA: dK and dV of a kv-head sum the contributions of its q-heads.

Readings: rows with no visible key have O = 0 and contribute nothing (all
their P are zero); the masks are the forward's causal (bottom-right) and
window visibility; score mods and block masks are not part of the backward.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import visible


def attend_bwd(q, k, v, do, scale, vis):
    """One sequence and head: q [n,dqk], k [m,dqk], v [m,dv], do [n,dv],
    vis bool [n,m].  Returns (dq, dk, dv) in float64."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    has = vis.any(axis=1)
    mx = np.where(has, np.max(s, axis=1, initial=-np.inf), 0.0)
    e = np.where(vis, np.exp(s - mx[:, None]), 0.0)
    den = np.where(has, e.sum(axis=1), 1.0)
    p = e / den[:, None]
    dv = p.T @ do
    dp = do @ v.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), dv


def _mask(mods):
    mods = dict(mods or {})
    return bool(mods.get("causal", False)), mods.get("window"), mods.get("scale")


def attention_bwd_dense(q, k, v, do, mods=None):
    """Dense BSHD: q [B,Sq,Hq,Dqk], k [B,Skv,Hkv,Dqk], v [B,Skv,Hkv,Dv],
    do [B,Sq,Hq,Dv].  Returns (dq, dk, dv) shaped like q, k, v (float64)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, Sq, Hq, Dqk = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    causal, window, scale = _mask(mods)
    scale = scale if scale else 1.0 / math.sqrt(Dqk)
    grp = Hq // Hkv
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    vis = visible(Sq, Skv, causal=causal, window=window)
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            a, c, e = attend_bwd(q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h], scale, vis)
            dq[b, :, h] = a
            dk[b, :, g] += c
            dv[b, :, g] += e
    return dq, dk, dv


def attention_bwd_varlen(q, k, v, do, cu_q, cu_k, mods=None):
    """Packed varlen: q [Tq,Hq,Dqk], k [Tk,Hkv,Dqk], v [Tk,Hkv,Dv], do [Tq,Hq,Dv]
    with cu_seqlens_q / cu_seqlens_k.  Returns (dq, dk, dv) (float64)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    Hq, Dqk = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    causal, window, scale = _mask(mods)
    scale = scale if scale else 1.0 / math.sqrt(Dqk)
    grp = Hq // Hkv
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(cu_q.shape[0] - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if q1 == q0 or k1 == k0:
            continue
        vis = visible(q1 - q0, k1 - k0, causal=causal, window=window)
        for h in range(Hq):
            g = h // grp
            a, c, e = attend_bwd(q[q0:q1, h], k[k0:k1, g], v[k0:k1, g], do[q0:q1, h], scale, vis)
            dq[q0:q1, h] = a
            dk[k0:k1, g] += c
            dv[k0:k1, g] += e
    return dq, dk, dv
