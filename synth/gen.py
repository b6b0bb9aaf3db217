"""Seeded generators for the attention workloads (no attention arithmetic here)."""
from __future__ import annotations

import math

import torch

E4M3_MAX = 448.0          # largest finite OCP E4M3 (e4m3fn) magnitude
E4M3_NAN_BYTE = 0x7F      # an E4M3 NaN encoding, used to poison unused cache bytes


def seed_for(config: int, subcase: int = 0) -> int:
    """Seed of workload `config`, sub-case `subcase`: 1000 + 10*config + subcase."""
    return 1000 + 10 * config + subcase


def _generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn_bf16(shape, seed: int, device="cpu") -> torch.Tensor:
    """N(0,1) drawn in fp32 from a seeded generator, rounded to bf16 (RNE)."""
    g = _generator(seed, device)
    return torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor OCP E4M3 quantisation with descale = amax/448.

    Returns (bytes uint8 with x's shape, descale fp32 tensor [1]) such that
    decode(bytes) * descale approximates x.  torch's float8_e4m3fn cast rounds
    to nearest even; both sides of every comparison read the returned bytes.
    """
    xf = x.float()
    amax = xf.abs().max()
    descale = (amax / E4M3_MAX).clamp_min(torch.finfo(torch.float32).tiny)
    q = (xf / descale).to(torch.float8_e4m3fn).view(torch.uint8)
    return q, descale.reshape(1).to(torch.float32)


def varlen_lengths(seed: int, n: int = 8, lo: int = 0, hi: int = 4096,
                   force_zero: bool = True, min_unaligned: int = 3, align: int = 64):
    """n lengths uniform in [lo, hi]; one forced to zero; resampled until at
    least `min_unaligned` of them are not multiples of `align`."""
    g = _generator(seed, "cpu")
    while True:
        lens = torch.randint(lo, hi + 1, (n,), generator=g)
        if force_zero:
            idx = int(torch.randint(0, n, (1,), generator=g))
            lens[idx] = 0
        if int(((lens % align) != 0).sum()) >= min_unaligned:
            return [int(v) for v in lens]


def make_decode_lengths(seed: int, n: int = 64, lo: int = 1024, hi: int = 32768):
    """Decode context lengths uniform in [lo, hi]."""
    g = _generator(seed, "cpu")
    return [int(v) for v in torch.randint(lo, hi + 1, (n,), generator=g)]


def cu_from_lengths(lengths) -> torch.Tensor:
    """Exclusive prefix sums [0, l0, l0+l1, ...] as int32."""
    cu = [0]
    for v in lengths:
        cu.append(cu[-1] + int(v))
    return torch.tensor(cu, dtype=torch.int32)


def make_dense(B, Sq, Skv, Hq, Hkv, Dqk, Dv, seed, device="cpu"):
    """Q [B,Sq,Hq,Dqk], K [B,Skv,Hkv,Dqk], V [B,Skv,Hkv,Dv], bf16 ~ N(0,1)."""
    return dict(
        q=randn_bf16((B, Sq, Hq, Dqk), seed, device),
        k=randn_bf16((B, Skv, Hkv, Dqk), seed + 100_000, device),
        v=randn_bf16((B, Skv, Hkv, Dv), seed + 200_000, device),
    )


def make_varlen(lengths_q, lengths_k, Hq, Hkv, Dqk, Dv, seed, device="cpu"):
    """Packed Q [Tq,Hq,Dqk], K [Tk,Hkv,Dqk], V [Tk,Hkv,Dv] bf16 plus int32 cu_seqlens."""
    cu_q = cu_from_lengths(lengths_q)
    cu_k = cu_from_lengths(lengths_k)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    return dict(
        q=randn_bf16((tq, Hq, Dqk), seed, device),
        k=randn_bf16((tk, Hkv, Dqk), seed + 100_000, device),
        v=randn_bf16((tk, Hkv, Dv), seed + 200_000, device),
        cu_q=cu_q.to(device), cu_k=cu_k.to(device),
        lengths_q=list(lengths_q), lengths_k=list(lengths_k),
    )


def make_paged(lengths_q, lengths_k, Hq, Hkv, Dqk, Dv, page_size, seed, device="cpu",
               kv_dtype="fp8", extra_pages=0, min_pages=0, place_high=0, poison=True, q_dtype="bf16"):
    """Paged K/V caches with head-major pages.

    K cache [num_pages, Hkv, page_size, Dqk], V cache [num_pages, Hkv, page_size, Dv]
    (uint8 E4M3 bytes for kv_dtype="fp8", bf16 otherwise).  Sequence b's
    logical page p lives at physical page block_table[b, p].  Physical pages
    are a seeded random sample of range(num_pages) where
    num_pages = max(min_pages, used + extra_pages).  `place_high` > 0 forces
    the first `place_high` used pages to the highest page ids (large offsets).
    Unused pages and the bytes past seqlen_k in a sequence's last page are
    filled with E4M3 NaN bytes (or bf16 NaN) when `poison` is set.
    q_dtype="fp8" quantises the same bf16 queries to E4M3 codes (uint8) with a
    per-tensor q_descale (amax/448); q_descale is None for bf16 queries.
    Returns dict(q, q_descale, k_cache, v_cache, cu_q, seqlen_k, block_table, k_descale,
    v_descale, num_pages, k_logical, v_logical) where *_logical are the
    token-major [Tk, Hkv, D] caches before paging (CPU, for reference only
    when small; None when the cache is large).
    """
    B = len(lengths_k)
    pages_per = [int(math.ceil(l / page_size)) for l in lengths_k]
    used = sum(pages_per)
    num_pages = max(int(min_pages), used + int(extra_pages), 1)
    max_pages = max(1, max(pages_per) if pages_per else 1)
    g = _generator(seed + 300_000, "cpu")
    if place_high:
        high = torch.arange(num_pages - place_high, num_pages)
        rest = torch.randperm(num_pages - place_high, generator=g)[: used - place_high]
        phys = torch.cat([high, rest])
        phys = phys[torch.randperm(used, generator=g)]
    else:
        phys = torch.randperm(num_pages, generator=g)[:used]
    block_table = torch.zeros((B, max_pages), dtype=torch.int32)
    pos = 0
    for b in range(B):
        n = pages_per[b]
        block_table[b, :n] = phys[pos:pos + n].to(torch.int32)
        pos += n

    cu_q = cu_from_lengths(lengths_q)
    tq, tk = int(cu_q[-1]), sum(int(l) for l in lengths_k)
    q = randn_bf16((tq, Hq, Dqk), seed, device)
    q_descale = None
    if q_dtype == "fp8":
        q, q_descale = quantize_e4m3(q)
    kf = torch.randn((tk, Hkv, Dqk), generator=_generator(seed + 100_000, device), device=device)
    vf = torch.randn((tk, Hkv, Dv), generator=_generator(seed + 200_000, device), device=device)
    if kv_dtype == "fp8":
        kq, k_descale = quantize_e4m3(kf)
        vq, v_descale = quantize_e4m3(vf)
        fill = E4M3_NAN_BYTE
        cdtype = torch.uint8
    else:
        kq, vq = kf.to(torch.bfloat16), vf.to(torch.bfloat16)
        k_descale = torch.ones(1, dtype=torch.float32)
        v_descale = torch.ones(1, dtype=torch.float32)
        fill = float("nan")
        cdtype = torch.bfloat16
    del kf, vf
    k_cache = torch.full((num_pages, Hkv, page_size, Dqk), fill if poison else 0, dtype=cdtype, device=device)
    v_cache = torch.full((num_pages, Hkv, page_size, Dv), fill if poison else 0, dtype=cdtype, device=device)
    # token t of sequence b, position j: physical page block_table[b, j // ps], slot j % ps
    if tk:
        tok_b = torch.repeat_interleave(torch.arange(B), torch.tensor([int(l) for l in lengths_k]))
        tok_j = torch.cat([torch.arange(int(l)) for l in lengths_k])
        tok_page = block_table[tok_b, tok_j // page_size].long().to(device)
        tok_slot = (tok_j % page_size).to(device)
        k_cache[tok_page, :, tok_slot, :] = kq
        v_cache[tok_page, :, tok_slot, :] = vq
    small = tk * Hkv * (Dqk + Dv) <= (1 << 26)
    return dict(
        q=q, q_descale=None if q_descale is None else q_descale.to(device),
        k_cache=k_cache, v_cache=v_cache,
        cu_q=cu_q.to(device),
        seqlen_k=torch.tensor([int(l) for l in lengths_k], dtype=torch.int32, device=device),
        block_table=block_table.to(device),
        k_descale=k_descale.to(device), v_descale=v_descale.to(device),
        num_pages=num_pages, page_size=page_size,
        lengths_q=list(lengths_q), lengths_k=list(lengths_k),
        k_logical=kq.cpu() if small else None, v_logical=vq.cpu() if small else None,
    )


def to_vectorized(d, x=16):
    """Copy of a make_paged() dict with its caches in the vectorized 5-D page
    layout: K [P, Hkv, Dqk/x, page_size, x], V [P, Hkv, page_size/x, Dv, x]
    (x elements of 16 bytes per vector).  A pure re-layout of the same bytes."""
    k, v = d["k_cache"], d["v_cache"]
    P, Hkv, ps, Dqk = k.shape
    Dv = v.shape[3]
    e = dict(d)
    e["k_cache"] = k.reshape(P, Hkv, ps, Dqk // x, x).permute(0, 1, 3, 2, 4).contiguous()
    e["v_cache"] = v.reshape(P, Hkv, ps // x, x, Dv).permute(0, 1, 2, 4, 3).contiguous()
    return e


def bernoulli_block_mask(bh, nqb, nkb, p, seed):
    """uint8 [bh, nqb, nkb]: 1 with probability p (seeded)."""
    g = _generator(seed + 400_000, "cpu")
    return (torch.rand((bh, nqb, nkb), generator=g) < p).to(torch.uint8)


def block_causal_mask(bh, nqb, nkb):
    """uint8 [bh, nqb, nkb]: 1 where key block <= query block."""
    qb = torch.arange(nqb)[:, None]
    kb = torch.arange(nkb)[None, :]
    return (kb <= qb).to(torch.uint8).expand(bh, nqb, nkb).contiguous()


def peaked_queries(key_rows: torch.Tensor, alpha: float) -> torch.Tensor:
    """Queries equal to alpha times given key rows (rounded to bf16).

    With alpha large, each query's softmax concentrates on the key it copies,
    which exposes any K/V pairing or row-permutation mistake."""
    return (key_rows.float() * alpha).to(torch.bfloat16)
