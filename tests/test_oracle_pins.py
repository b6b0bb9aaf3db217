"""Pins of the fp64 oracle against facts other than itself (CPU only).

Each test fixes part of the oracle with a closed form, a brute-force scalar
evaluation, a library special case, an invariant, or values printed in a
published specification / on the pages (fixtures under tests/golden/).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import f64
from oracle import attention as oatt
from oracle import layouts as olay

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


# ----------------------------------------------------------------------------- E4M3
def test_e4m3_golden_points():
    with open(os.path.join(GOLDEN, "e4m3_points.json")) as f:
        pts = json.load(f)["points"]
    codes = np.array([int(c, 16) for c, _ in pts], dtype=np.uint8)
    got = oracle.decode_e4m3(codes)
    for (c, want), g in zip(pts, got):
        if want == "nan":
            assert math.isnan(g), c
        else:
            assert g == want and math.copysign(1, g) == math.copysign(1, want), (c, g, want)


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


# ----------------------------------------------------------------------------- closed forms
def _counts(sq, skv, causal=False, window=None):
    """Visible-key counts per row from interval arithmetic (no mask matrix)."""
    out = []
    for i in range(sq):
        ip = i + skv - sq
        lo, hi = 0, skv - 1
        if causal:
            hi = min(hi, ip)
        if window is not None:
            wl, wr = window
            if wl >= 0:
                lo = max(lo, ip - wl)
            if wr >= 0:
                hi = min(hi, ip + wr)
        out.append(max(0, hi - lo + 1))
    return np.array(out)


@pytest.mark.parametrize("sq,skv,causal,window", [
    (17, 17, False, None), (17, 17, True, None), (9, 23, True, None), (23, 9, True, None),
    (31, 31, False, (5, 0)), (31, 31, True, (4, 2)), (12, 40, False, (3, 7)), (16, 16, False, (0, 0)),
])
def test_q_zero_gives_log_count_and_mean(sq, skv, causal, window):
    d, dv = 8, 5
    q = np.zeros((sq, d))
    k = rng.standard_normal((skv, d))
    v = rng.standard_normal((skv, dv))
    vis = oatt.visible(sq, skv, causal=causal, window=window)
    o, lse = oatt.attend(q, k, v, 0.3, vis)
    n = _counts(sq, skv, causal, window)
    for i in range(sq):
        if n[i] == 0:
            assert lse[i] == -np.inf and np.all(o[i] == 0)
            continue
        assert abs(lse[i] - math.log(n[i])) < 1e-12
        ip = i + skv - sq
        lo = 0 if window is None or window[0] < 0 else max(0, ip - window[0])
        mean = v[lo:lo + n[i]].mean(axis=0)
        assert np.allclose(o[i], mean, atol=1e-12)


def test_q_zero_block_mask_counts():
    sq = skv = 40
    bq, bk = 8, 16
    nqb, nkb = 5, 3
    bm = (rng.random((nqb, nkb)) < 0.5).astype(np.uint8)
    bm[2, :] = 0
    vis = oatt.visible(sq, skv, block_mask=bm, mask_block=(bq, bk))
    o, lse = oatt.attend(np.zeros((sq, 4)), rng.standard_normal((skv, 4)), rng.standard_normal((skv, 3)), 1.0, vis)
    for i in range(sq):
        n = sum(min(skv, (kb + 1) * bk) - kb * bk for kb in range(nkb) if bm[i // bq, kb])
        if n == 0:
            assert lse[i] == -np.inf
        else:
            assert abs(lse[i] - math.log(n)) < 1e-12


@pytest.mark.parametrize("slope", [0.0625, 0.5, 1.7])
def test_alibi_q_zero_geometric_series(slope):
    m = 37
    r = math.exp(-slope)
    vis = oatt.visible(m, m)
    _, lse = oatt.attend(np.zeros((m, 4)), rng.standard_normal((m, 4)), rng.standard_normal((m, 2)),
                         1.0, vis, alibi_slope=slope, ip=np.arange(m))
    for i in range(m):
        # sum_{d=0}^{i} r^d + sum_{d=1}^{m-1-i} r^d
        closed = (1 - r ** (i + 1)) / (1 - r) + r * (1 - r ** (m - 1 - i)) / (1 - r)
        assert abs(lse[i] - math.log(closed)) < 1e-12


def test_constant_v_gives_constant_output():
    sq, skv, d, dv = 19, 27, 16, 6
    c = rng.standard_normal(dv)
    v = np.tile(c, (skv, 1))
    for kw in [dict(), dict(causal=True), dict(window=(3, 1))]:
        vis = oatt.visible(sq, skv, **kw)
        o, lse = oatt.attend(rng.standard_normal((sq, d)) * 3, rng.standard_normal((skv, d)), v, 0.25, vis,
                             softcap=5.0, alibi_slope=0.1, ip=np.arange(sq) + skv - sq)
        has = vis.any(axis=1)
        assert np.allclose(o[has], c, atol=1e-12)


def test_single_visible_key_is_exact():
    sq, d, dv = 21, 8, 8
    q = rng.standard_normal((sq, d))
    k = rng.standard_normal((sq, d))
    v = rng.standard_normal((sq, dv))
    vis = oatt.visible(sq, sq, window=(0, 0))
    o, lse = oatt.attend(q, k, v, 0.5, vis)
    for i in range(sq):
        assert np.array_equal(o[i], v[i])
        assert abs(lse[i] - 0.5 * sum(q[i, t] * k[i, t] for t in range(d))) < 1e-12


def test_logit_shift_moves_lse_only():
    """An extra feature with q-value a and k-value 1 adds scale*a to every logit of
    the row: LSE moves by scale*a and O is unchanged."""
    sq, skv, d, dv = 11, 14, 6, 4
    q, k, v = rng.standard_normal((sq, d)), rng.standard_normal((skv, d)), rng.standard_normal((skv, dv))
    a = rng.standard_normal(sq) * 4
    vis = oatt.visible(sq, skv, causal=True)
    o1, l1 = oatt.attend(q, k, v, 0.7, vis)
    o2, l2 = oatt.attend(np.c_[q, a], np.c_[k, np.ones(skv)], v, 0.7, vis)
    has = vis.any(axis=1)
    assert np.allclose(o1, o2, atol=1e-12)
    assert np.allclose(l2[has] - l1[has], 0.7 * a[has], atol=1e-12)


def test_key_permutation_invariance():
    sq, skv, d, dv = 9, 30, 8, 5
    q, k, v = rng.standard_normal((sq, d)), rng.standard_normal((skv, d)), rng.standard_normal((skv, dv))
    perm = rng.permutation(skv)
    vis = np.ones((sq, skv), bool)
    o1, l1 = oatt.attend(q, k, v, 0.4, vis, softcap=3.0)
    o2, l2 = oatt.attend(q, k[perm], v[perm], 0.4, vis, softcap=3.0)
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


# ----------------------------------------------------------------------------- brute force
def _brute(q, k, v, scale, causal, window, softcap, slope, bm, mb):
    sq, skv = len(q), len(k)
    outs, lses = [], []
    for i in range(sq):
        ip = i + skv - sq
        logits = {}
        for j in range(skv):
            if causal and j > ip:
                continue
            if window is not None:
                if window[0] >= 0 and j < ip - window[0]:
                    continue
                if window[1] >= 0 and j > ip + window[1]:
                    continue
            if bm is not None and not bm[i // mb[0]][j // mb[1]]:
                continue
            s = scale * math.fsum(float(q[i][t]) * float(k[j][t]) for t in range(len(q[i])))
            if softcap is not None:
                s = softcap * math.tanh(s / softcap)
            if slope is not None:
                s -= slope * abs(ip - j)
            logits[j] = s
        if not logits:
            outs.append([0.0] * len(v[0]))
            lses.append(-math.inf)
            continue
        mx = max(logits.values())
        den = math.fsum(math.exp(s - mx) for s in logits.values())
        lse = mx + math.log(den)
        outs.append([math.fsum(math.exp(s - lse) * float(v[j][c]) for j, s in logits.items())
                     for c in range(len(v[0]))])
        lses.append(lse)
    return np.array(outs), np.array(lses)


CASES = [
    dict(causal=False, window=None, softcap=None, slope=None, bm=False),
    dict(causal=True, window=None, softcap=None, slope=None, bm=False),
    dict(causal=False, window=(3, 0), softcap=None, slope=None, bm=False),
    dict(causal=True, window=(2, 5), softcap=2.5, slope=None, bm=False),
    dict(causal=False, window=None, softcap=None, slope=0.3, bm=False),
    dict(causal=False, window=None, softcap=1.5, slope=0.2, bm=True),
    dict(causal=True, window=None, softcap=None, slope=None, bm=True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("sq,skv", [(13, 13), (7, 17), (17, 5)])
def test_brute_force_small(case, sq, skv):
    c = CASES[case]
    d, dv = 5, 3
    q, k, v = rng.standard_normal((sq, d)) * 2, rng.standard_normal((skv, d)), rng.standard_normal((skv, dv))
    mb = (4, 3)
    bm = (rng.random((math.ceil(sq / 4), math.ceil(skv / 3))) < 0.6).astype(np.uint8) if c["bm"] else None
    vis = oatt.visible(sq, skv, causal=c["causal"], window=c["window"], block_mask=bm, mask_block=mb)
    o, lse = oatt.attend(q, k, v, 0.45, vis, softcap=c["softcap"], alibi_slope=c["slope"],
                         ip=np.arange(sq) + skv - sq)
    ob, lb = _brute(q, k, v, 0.45, c["causal"], c["window"], c["softcap"], c["slope"], bm, mb)
    assert np.array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    assert np.allclose(lse[fin], lb[fin], atol=1e-12, rtol=0)
    assert np.allclose(o, ob, atol=1e-12, rtol=0)


def test_matches_torch_sdpa_fp64():
    """torch's CPU fp64 scaled_dot_product_attention with a boolean mask for O,
    and logsumexp of the masked logits for LSE."""
    B, Sq, Skv, Hq, Hkv, D = 2, 33, 47, 4, 2, 16
    q = torch.randn(B, Sq, Hq, D, dtype=torch.float64)
    k = torch.randn(B, Skv, Hkv, D, dtype=torch.float64)
    v = torch.randn(B, Skv, Hkv, D, dtype=torch.float64)
    for causal in (False, True):
        o, lse = oracle.attention_dense(q.numpy(), k.numpy(), v.numpy(), dict(causal=causal))
        mask = torch.from_numpy(oatt.visible(Sq, Skv, causal=causal))
        kk = k.repeat_interleave(Hq // Hkv, dim=2).transpose(1, 2)
        vv = v.repeat_interleave(Hq // Hkv, dim=2).transpose(1, 2)
        qq = q.transpose(1, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask).transpose(1, 2)
        logits = (qq @ kk.transpose(-1, -2)) / math.sqrt(D)
        ref_lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)
        has = mask.any(dim=-1)
        assert torch.allclose(torch.from_numpy(o)[:, has], ref[:, has], atol=1e-12)
        assert torch.allclose(torch.from_numpy(lse)[..., has], ref_lse[..., has], atol=1e-12)


# ----------------------------------------------------------------------------- degenerate mods
def test_degenerate_mods_reduce_to_plain():
    sq = skv = 24
    q, k, v = rng.standard_normal((sq, 8)), rng.standard_normal((skv, 8)), rng.standard_normal((skv, 4))
    full = np.ones((sq, skv), bool)
    o0, l0 = oatt.attend(q, k, v, 0.5, full)
    o1, l1 = oatt.attend(q, k, v, 0.5, full, alibi_slope=0.0, ip=np.arange(sq))
    o2, l2 = oatt.attend(q, k, v, 0.5, full, softcap=1e30)
    vis3 = oatt.visible(sq, skv, window=(sq, sq))
    vis4 = oatt.visible(sq, skv, block_mask=np.ones((2, 2), np.uint8), mask_block=(16, 16))
    for o, l in [(o1, l1), (o2, l2), oatt.attend(q, k, v, 0.5, vis3), oatt.attend(q, k, v, 0.5, vis4)]:
        assert np.allclose(o, o0, atol=1e-13) and np.allclose(l, l0, atol=1e-13)
    # block-causal with unit tiles is token causal
    bc = np.tril(np.ones((sq, skv), np.uint8))
    assert np.array_equal(oatt.visible(sq, skv, block_mask=bc, mask_block=(1, 1)),
                          oatt.visible(sq, skv, causal=True))


def test_lse_merge_identity():
    sq, skv, d, dv = 15, 50, 8, 6
    q, k, v = rng.standard_normal((sq, d)) * 2, rng.standard_normal((skv, d)), rng.standard_normal((skv, dv))
    vis = oatt.visible(sq, skv, causal=True)
    o, lse = oatt.attend(q, k, v, 0.5, vis)
    cuts = [0, 7, 7, 22, 50]          # includes an empty split
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        sub = np.zeros_like(vis)
        sub[:, a:b] = vis[:, a:b]
        parts.append(oatt.attend(q, k, v, 0.5, sub))
    om, lm = oatt.lse_merge(parts)
    fin = np.isfinite(lse)
    assert np.array_equal(fin, np.isfinite(lm))
    assert np.allclose(lm[fin], lse[fin], atol=1e-12) and np.allclose(om, o, atol=1e-12)


# ----------------------------------------------------------------------------- layouts
def _np(t):
    return t.float().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else t.numpy()


def test_varlen_equals_per_sequence_dense():
    import synth
    lens = [5, 0, 33, 64, 17]
    d = synth.make_varlen(lens, lens, 4, 2, 16, 16, seed=7)
    o, lse = oracle.attention_varlen(_np(d["q"]), _np(d["k"]), _np(d["v"]), d["cu_q"].numpy(), d["cu_k"].numpy(),
                                     dict(causal=True))
    cu = d["cu_q"].numpy()
    for b, L in enumerate(lens):
        if L == 0:
            continue
        sl = slice(cu[b], cu[b + 1])
        od, ld = oracle.attention_dense(_np(d["q"])[None, sl], _np(d["k"])[None, sl], _np(d["v"])[None, sl],
                                        dict(causal=True))
        assert np.array_equal(od[0], o[sl]) and np.array_equal(ld[0], lse[:, sl])


def test_paged_gather_index_arithmetic_and_placement_invariance():
    import synth
    lk = [70, 3, 128, 129]
    lq = [5, 3, 1, 40]
    d = synth.make_paged(lq, lk, 4, 2, 24, 16, page_size=16, seed=3, extra_pages=5)
    kc, vc = d["k_cache"].numpy(), d["v_cache"].numpy()
    bt = d["block_table"].numpy()
    # gather equals explicit page/slot arithmetic, bytes identical
    t0 = 0
    for b, L in enumerate(lk):
        for g in range(2):
            got = olay.gather_paged(kc, bt[b], L, g)
            want = np.stack([oracle.decode_e4m3(kc[bt[b][j // 16], g, j % 16]) for j in range(L)])
            assert np.array_equal(np.isnan(got), np.isnan(want)) and np.array_equal(np.nan_to_num(got), np.nan_to_num(want))
            assert np.array_equal(kc[bt[b][np.arange(L) // 16], g, np.arange(L) % 16], d["k_logical"][t0:t0 + L, g].numpy())
        t0 += L
    # result equals the varlen oracle on the logical (dequantised) KV
    kd = oracle.decode_e4m3(d["k_logical"].numpy()) * float(d["k_descale"])
    vd = oracle.decode_e4m3(d["v_logical"].numpy()) * float(d["v_descale"])
    cu_k = np.concatenate([[0], np.cumsum(lk)])
    mods = dict(causal=True)
    o1, l1 = oracle.attention_paged(_np(d["q"]), kc, vc, d["cu_q"].numpy(), d["seqlen_k"].numpy(), bt, mods,
                                    float(d["k_descale"]), float(d["v_descale"]))
    o2, l2 = oracle.attention_varlen(_np(d["q"]), kd, vd, d["cu_q"].numpy(), cu_k, mods)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert not np.isnan(o1).any()


def test_paged_4gib_golden_geometry():
    """The pages' >4 GiB case: a page id of ceil(2^32/8192) puts both K and V
    byte offsets past 2^32 for Hkv=1, page 64, K width 192 and V width 128 fp8."""
    with open(os.path.join(GOLDEN, "paged_4gib_geometry.json")) as f:
        gd = json.load(f)
    geo = gd["geometry"]
    kpb = geo["Hkv"] * geo["page_size"] * geo["d_qk"] * geo["bytes_per_elem"]
    vpb = geo["Hkv"] * geo["page_size"] * geo["d_v"] * geo["bytes_per_elem"]
    assert kpb + vpb == gd["page_bytes_k_plus_v"]
    assert -(-(2 ** 32) // gd["value_page_divisor"]) == gd["high_page"]
    assert gd["high_page"] + 1 == gd["num_pages"]
    assert gd["num_pages"] * (kpb + vpb) == gd["cache_bytes"]
    assert round(gd["cache_bytes"] / 1e9, 1) == gd["cache_bytes_approx_gb"]
    assert gd["high_page"] * kpb >= 2 ** 32 and gd["high_page"] * vpb >= 2 ** 32
    assert (gd["high_page"] - 1) * vpb < 2 ** 32


# ----------------------------------------------------------------------------- vectorized pages
def test_vectorized_gather_matches_the_pages_inverse_permutes():
    """The 5-D page layout as the pages state it: permuting a K cache
    [P, Hkv, D/16, ps, 16] by (0,3,1,2,4), and a V cache [P, Hkv, ps/16, Dv, 16]
    by (0,2,4,1,3), gives token-major pages [P, ps, Hkv, D]; the oracle's
    gather must read exactly those rows."""
    rng = np.random.default_rng(11)
    P, Hkv, ps, D, Dv, x = 5, 2, 32, 48, 32, 16
    k5 = rng.integers(0, 120, size=(P, Hkv, D // x, ps, x)).astype(np.uint8)
    v5 = rng.integers(0, 120, size=(P, Hkv, ps // x, Dv, x)).astype(np.uint8)
    kt = k5.transpose(0, 3, 1, 2, 4).reshape(P, ps, Hkv, D)
    vt = v5.transpose(0, 2, 4, 1, 3).reshape(P, ps, Hkv, Dv)
    block_row = [3, 0, 4]
    L = 77
    for g in range(Hkv):
        kg = oracle.gather_paged(k5, block_row, L, g, layout="vectorized", kind="k")
        vg = oracle.gather_paged(v5, block_row, L, g, layout="vectorized", kind="v")
        for j in range(L):
            p, sl = block_row[j // ps], j % ps
            assert np.array_equal(kg[j], oracle.decode_e4m3(kt[p, sl, g]))
            assert np.array_equal(vg[j], oracle.decode_e4m3(vt[p, sl, g]))


def test_vectorized_pages_give_the_head_major_result():
    """The same logical cache in both page layouts gives identical fp64
    attention (the layout only moves bytes)."""
    d = synth.make_paged([3, 40], [70, 40], 4, 2, 64, 32, page_size=32, seed=171, extra_pages=2)
    e = synth.to_vectorized(d)
    args = (d["cu_q"], d["seqlen_k"], d["block_table"], dict(causal=True), float(d["k_descale"]), float(d["v_descale"]))
    o1, l1 = oracle.attention_paged(f64(d["q"]), d["k_cache"].numpy(), d["v_cache"].numpy(), *args)
    o2, l2 = oracle.attention_paged(f64(e["q"]), e["k_cache"].numpy(), e["v_cache"].numpy(), *args, layout="vectorized")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ----------------------------------------------------------------------------- E4M3 queries
def test_fp8_query_codes_decode_to_the_golden_points_times_descale():
    """Q codes are read by the same OCP E4M3 rule as the caches, then scaled."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "e4m3_points.json")) as f:
        pts = [(int(c, 16), v) for c, v in json.load(f)["points"] if v != "nan"]
    codes = np.array([c for c, _ in pts], dtype=np.uint8).reshape(1, 1, -1)
    got = olay.paged_queries(codes, 0.375).reshape(-1)
    assert np.array_equal(got, np.array([v for _, v in pts]) * 0.375)
    with pytest.raises(ValueError):
        olay.paged_queries(codes)
    with pytest.raises(ValueError):
        olay.paged_queries(np.zeros((1, 1, 4)), 0.5)


def test_fp8_query_zero_codes_give_log_count_and_mean():
    """All-zero Q codes (any q_descale): every visible key has logit 0, so
    LSE = ln(visible count) and O = mean of the visible V rows."""
    lq, lk = [3, 1, 40], [9, 70, 40]
    d = synth.make_paged(lq, lk, 4, 2, 64, 32, page_size=16, seed=7, q_dtype="fp8")
    q = np.zeros(tuple(d["q"].shape), dtype=np.uint8)
    kd, vd = float(d["k_descale"]), float(d["v_descale"])
    o, lse = oracle.attention_paged(q, f64(d["k_cache"]), f64(d["v_cache"]), d["cu_q"], d["seqlen_k"],
                                    d["block_table"], dict(causal=True), kd, vd, q_descale=3.0)
    cu = d["cu_q"].tolist()
    vlog = d["v_logical"].double().numpy() if d["v_logical"].dtype != torch.uint8 else \
        oracle.decode_e4m3(d["v_logical"].numpy()) * vd
    ks = np.cumsum([0] + lk)
    for b in range(3):
        for i in range(lq[b]):
            n = i + lk[b] - lq[b] + 1
            for h in range(4):
                assert abs(lse[h, cu[b] + i] - math.log(n)) < 1e-12
                assert np.allclose(o[cu[b] + i, h], vlog[ks[b]:ks[b] + n, h // 2].mean(axis=0), atol=1e-12)


def test_fp8_query_descale_acts_as_a_logit_scale():
    """q_descale multiplies every logit: (q_descale 2c, scale s) equals
    (q_descale c, scale 2s), and differs from (q_descale c, scale s)."""
    d = synth.make_paged([5, 17], [30, 17], 4, 4, 64, 64, page_size=8, seed=11, q_dtype="fp8")
    args = (f64(d["q"]), f64(d["k_cache"]), f64(d["v_cache"]), d["cu_q"], d["seqlen_k"], d["block_table"])
    kd, vd, c = float(d["k_descale"]), float(d["v_descale"]), float(d["q_descale"])
    o1, l1 = oracle.attention_paged(*args, dict(causal=True, scale=0.1), kd, vd, q_descale=2 * c)
    o2, l2 = oracle.attention_paged(*args, dict(causal=True, scale=0.2), kd, vd, q_descale=c)
    o3, l3 = oracle.attention_paged(*args, dict(causal=True, scale=0.1), kd, vd, q_descale=c)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)
    assert not np.allclose(l1, l3, atol=1e-3)


# ----------------------------------------------------------------------------- E4M3 encoding, KV-cache write
def _golden_points():
    with open(os.path.join(os.path.dirname(__file__), "golden", "e4m3_points.json")) as f:
        return [(int(c, 16), v) for c, v in json.load(f)["points"]]


def test_e4m3_encode_golden_points():
    for c, v in _golden_points():
        if v == "nan":
            assert oracle.encode_e4m3(np.float32("nan")) & 0x7F == 0x7F
        else:
            assert int(oracle.encode_e4m3(np.float32(v))) == c, (hex(c), v)


def test_e4m3_encode_round_trips_every_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = oracle.decode_e4m3(codes).astype(np.float32)
    assert np.array_equal(oracle.encode_e4m3(vals), codes)


def test_e4m3_encode_ties_go_to_even_and_halves_split():
    """Midpoints between neighbouring codes go to the even code; a hair
    either side goes to the nearer one (brute force over the code table)."""
    for c in range(0, 0x7E):
        lo, hi = oracle.decode_e4m3(np.uint8(c)), oracle.decode_e4m3(np.uint8(c + 1))
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert int(oracle.encode_e4m3(mid)) == even
        assert int(oracle.encode_e4m3(np.nextafter(mid, np.float32(0)))) == c
        assert int(oracle.encode_e4m3(np.nextafter(mid, np.float32(1e9)))) == c + 1
        assert int(oracle.encode_e4m3(-mid)) == even | 0x80


def test_e4m3_encode_saturates():
    big = np.array([448.0, 464.0, 479.9, 1e6, np.inf], dtype=np.float32)
    assert np.all(oracle.encode_e4m3(big) == 0x7E)
    assert np.all(oracle.encode_e4m3(-big) == 0xFE)


def test_e4m3_encode_matches_torch_cast_in_range():
    x = torch.randn(200000, generator=torch.Generator().manual_seed(5)) * 60
    x = x.clamp(-448, 448)
    x[:1000] = x[:1000] * 1e-3            # subnormal range
    want = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_e4m3(x.numpy()), want)


def test_amax_descale_rule():
    assert oracle.amax_descale(np.array([0.0, 3.5, -896.0])) == np.float32(2.0)
    assert oracle.amax_descale(np.zeros(5)) == np.float32(2.0 ** -126)
    x = np.array([1.0, -0.3], dtype=np.float32)
    assert oracle.amax_descale(x) == np.float32(np.float32(1.0) / np.float32(448.0))


@pytest.mark.parametrize("layout", ["head_major", "vectorized"])
def test_kv_cache_write_places_and_quantises(layout):
    """Each mapped token lands in its slot with codes within half an E4M3
    step of x / descale; skipped and untouched slots keep their bytes; the
    vectorised cache is the head-major one under the pages' layout map."""
    g = np.random.default_rng(3)
    T, Hkv, Dqk, Dv, P, ps = 37, 2, 64, 32, 6, 16
    k = g.standard_normal((T, Hkv, Dqk)).astype(np.float32)
    v = g.standard_normal((T, Hkv, Dv)).astype(np.float32)
    slots = g.permutation(P * ps)[:T].astype(np.int64)
    slots[4], slots[9] = -1, P * ps + 3
    kc0 = np.full((P, Hkv, ps, Dqk), 0x7F, np.uint8)
    vc0 = np.full((P, Hkv, ps, Dv), 0x7F, np.uint8)
    kc, vc, kd, vd = oracle.kv_cache_write(k, v, slots, kc0, vc0, ps)
    assert kd == oracle.amax_descale(k) and vd == oracle.amax_descale(v)
    written = set()
    for t, sl in enumerate(slots):
        if t in (4, 9):
            continue
        p, s = divmod(int(sl), ps)
        written.add((p, s))
        for x, c, dsc in ((k[t], kc[p, :, s], kd), (v[t], vc[p, :, s], vd)):
            y = x / dsc
            back = oracle.decode_e4m3(c)
            step = np.exp2(np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6))) - 3)
            assert np.all(np.abs(back - y) <= step / 2 + 1e-6)
    for p in range(P):
        for s in range(ps):
            if (p, s) not in written:
                assert np.all(kc[p, :, s] == 0x7F) and np.all(vc[p, :, s] == 0x7F)
    if layout == "vectorized":
        kv0 = synth.to_vectorized(dict(k_cache=torch.from_numpy(kc0), v_cache=torch.from_numpy(vc0)))
        kcv, vcv, _, _ = oracle.kv_cache_write(k, v, slots, kv0["k_cache"].numpy(), kv0["v_cache"].numpy(), ps,
                                               layout="vectorized")
        ref = synth.to_vectorized(dict(k_cache=torch.from_numpy(kc), v_cache=torch.from_numpy(vc)))
        assert np.array_equal(kcv, ref["k_cache"].numpy()) and np.array_equal(vcv, ref["v_cache"].numpy())


def test_kv_cache_write_given_descale():
    k = np.array([[[1.0] * 16]], dtype=np.float32)
    v = np.array([[[-2.0] * 16]], dtype=np.float32)
    kc, vc, kd, vd = oracle.kv_cache_write(k, v, [3], np.zeros((1, 1, 4, 16), np.uint8),
                                           np.zeros((1, 1, 4, 16), np.uint8), 4, k_descale=0.5, v_descale=0.25)
    assert kd == np.float32(0.5) and np.all(kc[0, 0, 3] == 0x40)     # 2.0
    assert np.all(vc[0, 0, 3] == 0xD0)                               # -8.0
    assert np.all(kc[0, 0, :3] == 0)


# ----------------------------------------------------------------------------- backward
def _loss(q, k, v, do, mods):
    o, _ = oracle.attention_dense(q, k, v, mods)
    return float((o * do).sum())


@pytest.mark.parametrize("sq,skv,mods", [(5, 7, dict(causal=True)), (7, 5, dict(causal=True)),
                                         (6, 6, dict()), (6, 9, dict(window=(2, 1))), (8, 3, dict(causal=True))])
def test_backward_matches_finite_differences(sq, skv, mods):
    """Central differences of sum(dO * O) from the forward oracle, at every
    coordinate of q, k and v (tiny shapes, GQA 4/2 so dK and dV sum over a
    group; rows without a visible key included)."""
    g = np.random.default_rng(sq * 10 + skv)
    q = g.standard_normal((1, sq, 4, 3))
    k = g.standard_normal((1, skv, 2, 3))
    v = g.standard_normal((1, skv, 2, 2))
    do = g.standard_normal((1, sq, 4, 2))
    dq, dk, dv = oracle.attention_bwd_dense(q, k, v, do, mods)
    h = 1e-6
    for x, dx in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = _loss(q, k, v, do, mods)
            x[idx] = x0 - h
            lm = _loss(q, k, v, do, mods)
            x[idx] = x0
            assert abs((lp - lm) / (2 * h) - dx[idx]) < 1e-7, (idx, (lp - lm) / (2 * h), dx[idx])


def test_backward_matches_torch_autograd_fp64():
    """torch autograd through a plain fp64 softmax attention (library case),
    causal with more keys than queries (no empty rows), varlen driver."""
    g = torch.Generator().manual_seed(9)
    lq, lk = [5, 9], [8, 9]
    cu_q, cu_k = np.cumsum([0] + lq), np.cumsum([0] + lk)
    q = torch.randn(sum(lq), 2, 8, generator=g, dtype=torch.float64, requires_grad=True)
    k = torch.randn(sum(lk), 1, 8, generator=g, dtype=torch.float64, requires_grad=True)
    v = torch.randn(sum(lk), 1, 4, generator=g, dtype=torch.float64, requires_grad=True)
    do = torch.randn(sum(lq), 2, 4, generator=g, dtype=torch.float64)
    outs = []
    for b in range(2):
        qb, kb, vb = q[cu_q[b]:cu_q[b + 1]], k[cu_k[b]:cu_k[b + 1]], v[cu_k[b]:cu_k[b + 1]]
        s = torch.einsum("ihd,jd->hij", qb, kb[:, 0]) / math.sqrt(8)
        i = torch.arange(lq[b])[:, None] + lk[b] - lq[b]
        s = s.masked_fill(torch.arange(lk[b])[None, :] > i, float("-inf"))
        outs.append(torch.einsum("hij,jd->ihd", torch.softmax(s, dim=-1), vb[:, 0]))
    (torch.cat(outs) * do).sum().backward()
    dq, dk, dv = oracle.attention_bwd_varlen(q.detach().numpy(), k.detach().numpy(), v.detach().numpy(),
                                             do.numpy(), cu_q, cu_k, dict(causal=True))
    assert np.allclose(dq, q.grad.numpy(), atol=1e-12)
    assert np.allclose(dk, k.grad.numpy(), atol=1e-12)
    assert np.allclose(dv, v.grad.numpy(), atol=1e-12)


def test_backward_delta_is_rowsum_do_o():
    """Delta_i = sum_j P_ij dP_ij equals dO_i . O_i (the form the kernels use)."""
    g = np.random.default_rng(2)
    q, k, v, do = g.standard_normal((6, 4)), g.standard_normal((9, 4)), g.standard_normal((9, 3)), \
        g.standard_normal((6, 3))
    vis = oatt.visible(6, 9, causal=True)
    o, _ = oatt.attend(q, k, v, 0.5, vis)
    s = np.where(vis, 0.5 * q @ k.T, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.allclose((p * (do @ v.T)).sum(axis=1), (do * o).sum(axis=1), atol=1e-12)


# ----------------------------------------------------------------------------- row samplers
# varlen_rows / paged_rows give the expected rows of every full-size parity
# test; they must equal the same rows of the full drivers above (which the
# closed forms, brute force and library cases pin).  Picks are a seeded
# shuffle of every (sequence, q-head, row) triple, so consecutive picks jump
# between sequences and kv-head groups (paged_rows keeps one gathered
# (sequence, kv-head) at a time and must refresh it on every change).  The
# samplers compute each row alone, the drivers in blocks: agreement to fp64
# rounding (1e-12) with identical -inf rows.
def _all_picks(lq, Hq, seed):
    picks = [(b, h, i) for b, n in enumerate(lq) for h in range(Hq) for i in range(n)]
    order = np.random.default_rng(seed).permutation(len(picks))
    return [picks[k] for k in order]


def _check_rows(o_full, lse_full, cu_q, picks, o_r, l_r):
    assert len(picks) > 0
    for n, (b, h, i) in enumerate(picks):
        t = int(cu_q[b]) + i
        if np.isneginf(lse_full[h, t]):
            assert np.isneginf(l_r[n]) and np.all(o_r[n] == 0.0), (b, h, i)
        else:
            assert abs(l_r[n] - lse_full[h, t]) <= 1e-12, (b, h, i, l_r[n], lse_full[h, t])
            assert np.max(np.abs(o_r[n] - o_full[t, h])) <= 1e-12, (b, h, i)


def _row_mods(case, B, Hq, nq, nk, seed):
    if case == "causal":
        return dict(causal=True)
    if case == "noncausal":
        return {}
    if case == "window":
        return dict(window=(7, 2))
    if case == "causal_window":
        return dict(causal=True, window=(5, -1))
    if case == "alibi_softcap":
        return dict(alibi_slope=0.3, softcap=5.0)
    if case == "block_mask":
        bm = synth.bernoulli_block_mask(B * Hq, -(-nq // 8), -(-nk // 8), 0.5, seed=seed).numpy()
        return dict(block_mask=bm, mask_block=(8, 8), causal=True)
    raise ValueError(case)


@pytest.mark.parametrize("case", ["causal", "noncausal", "window", "causal_window", "alibi_softcap", "block_mask"])
def test_varlen_rows_equal_the_full_driver(case):
    """Cross lengths (Sq != Skv both ways), a zero-length sequence, GQA 6/2."""
    lq, lk = [17, 0, 40, 5, 33], [25, 0, 40, 9, 20]
    Hq, Hkv = 6, 2
    d = synth.make_varlen(lq, lk, Hq, Hkv, 16, 8, seed=501)
    mods = _row_mods(case, len(lq), Hq, max(lq), max(lk), seed=502)
    q, k, v = _np(d["q"]), _np(d["k"]), _np(d["v"])
    cu_q, cu_k = d["cu_q"].numpy(), d["cu_k"].numpy()
    o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, mods)
    picks = _all_picks(lq, Hq, seed=503)
    o_r, l_r = oracle.varlen_rows(q, k, v, cu_q, cu_k, picks, mods)
    _check_rows(o, lse, cu_q, picks, o_r, l_r)


@pytest.mark.parametrize("layout,kv,qdt", [("head_major", "fp8", "bf16"), ("head_major", "fp8", "fp8"),
                                            ("vectorized", "fp8", "bf16"), ("vectorized", "fp8", "fp8"),
                                            ("head_major", "bf16", "bf16")])
@pytest.mark.parametrize("case", ["causal", "causal_window", "alibi_softcap", "block_mask"])
def test_paged_rows_equal_the_full_driver(layout, kv, qdt, case):
    """Both page layouts, E4M3 and bf16 caches, E4M3 and bf16 queries (E4M3
    queries go with E4M3 caches), chunked-prefill lengths (Sq < Skv), GQA 4/2."""
    lq, lk = [3, 40, 1, 17], [70, 40, 33, 17]
    Hq, Hkv = 4, 2
    d = synth.make_paged(lq, lk, Hq, Hkv, 64, 32, page_size=16, seed=511, extra_pages=3,
                         kv_dtype=kv, q_dtype=qdt)
    if layout == "vectorized":
        d = synth.to_vectorized(d)
    mods = _row_mods(case, len(lq), Hq, max(lq), max(lk), seed=512)
    qd = float(d["q_descale"]) if qdt == "fp8" else None
    args = (f64(d["q"]), f64(d["k_cache"]), f64(d["v_cache"]), d["cu_q"].numpy(), d["seqlen_k"].numpy(),
            d["block_table"].numpy())
    kd, vd = float(d["k_descale"]), float(d["v_descale"])
    o, lse = oracle.attention_paged(*args, mods, kd, vd, layout=layout, q_descale=qd)
    assert not np.isnan(o).any()
    picks = _all_picks(lq, Hq, seed=513)
    o_r, l_r = oracle.paged_rows(*args, picks, mods, kd, vd, layout=layout, q_descale=qd)
    _check_rows(o, lse, d["cu_q"].numpy(), picks, o_r, l_r)


def test_row_samplers_catch_a_wrong_row():
    """The comparison above is sharp: sampling row i+1 in place of row i, or
    the neighbouring q-head, is far outside the 1e-12 agreement."""
    lq = [12, 20]
    d = synth.make_varlen(lq, lq, 4, 2, 16, 8, seed=521)
    q, k, v = _np(d["q"]), _np(d["k"]), _np(d["v"])
    cu = d["cu_q"].numpy()
    o, lse = oracle.attention_varlen(q, k, v, cu, cu, dict(causal=True))
    for shifted in ([(1, 3, 5)], [(1, 2, 6)]):
        o_r, l_r = oracle.varlen_rows(q, k, v, cu, cu, shifted, dict(causal=True))
        with pytest.raises(AssertionError):
            _check_rows(o, lse, cu, [(1, 3, 6)], o_r, l_r)
