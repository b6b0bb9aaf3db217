"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Small and ragged shapes are compared element by element; the full-size
workloads are compared on sampled rows that the oracle computes one by one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import TOL_LSE, TOL_O_BF16, TOL_O_FP8, compare, f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import attention_fa_fwd_03_amd as fa

DEV = "cuda"


def _nan_like(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def _dense_run(d, mods_kw, Dv):
    q, k, v = (d[x].to(DEV) for x in ("q", "k", "v"))
    B, Sq, Hq, _ = q.shape
    o = _nan_like((B, Sq, Hq, Dv), torch.bfloat16)
    lse = _nan_like((B, Hq, Sq), torch.float32)
    fa.fa_fwd_dense(q, k, v, o, lse, fa.Mods(**mods_kw))
    torch.cuda.synchronize()
    return o, lse


def _oracle_mods(mods_kw, block_mask=None):
    m = dict(mods_kw)
    if "block_mask" in m:
        m["block_mask"] = None if m["block_mask"] is None else m["block_mask"].cpu().numpy()
    if block_mask is not None:
        m["block_mask"] = block_mask
    if "mask_block" not in m:
        m["mask_block"] = (128, 128)
    return m


# ----------------------------------------------------------------------------- dense
def test_dense_small_config():
    """B=1, H=2, Sq=Skv=128, D=64, scale 1/sqrt(64), non-causal."""
    d = synth.make_dense(1, 128, 128, 2, 2, 64, 64, seed=synth.seed_for(1))
    o, lse = _dense_run(d, dict(scale=1 / 8), 64)
    o_ref, l_ref = oracle.attention_dense(f64(d["q"]), f64(d["k"]), f64(d["v"]), dict(scale=1 / 8))
    compare(o.permute(0, 2, 1, 3), lse, o_ref.transpose(0, 2, 1, 3), l_ref, TOL_O_BF16, what="dense cfg1")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Skv", [(128, 128), (200, 333), (333, 200), (1, 77), (64, 1), (257, 257), (5, 0)])
def test_dense_shapes(D, causal, Sq, Skv):
    d = synth.make_dense(2, Sq, Skv, 4, 2, D, D, seed=11 + Sq + 7 * Skv + D)
    o, lse = _dense_run(d, dict(causal=causal), D)
    o_ref, l_ref = oracle.attention_dense(f64(d["q"]), f64(d["k"]), f64(d["v"]), dict(causal=causal))
    compare(o.permute(0, 2, 1, 3), lse, o_ref.transpose(0, 2, 1, 3), l_ref, TOL_O_BF16,
            what=f"dense D{D} c{causal} {Sq}x{Skv}")


# ----------------------------------------------------------------------------- varlen
def _varlen_run(d, mods_kw, Dv):
    q, k, v = (d[x].to(DEV) for x in ("q", "k", "v"))
    cu_q, cu_k = d["cu_q"].to(DEV), d["cu_k"].to(DEV)
    Tq, Hq, _ = q.shape
    o = _nan_like((Tq, Hq, Dv), torch.bfloat16)
    lse = _nan_like((Hq, Tq), torch.float32)
    fa.fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, max(d["lengths_q"]), max(d["lengths_k"]), fa.Mods(**mods_kw))
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 4, 4), (128, 8, 2), (64, 3, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_ragged(D, Hq, Hkv, causal):
    lq = [5, 0, 130, 64, 1, 300, 0, 77]
    lk = [5, 0, 130, 64, 1, 300, 0, 77]
    d = synth.make_varlen(lq, lk, Hq, Hkv, D, D, seed=21 + D + Hq)
    o, lse = _varlen_run(d, dict(causal=causal), D)
    o_ref, l_ref = oracle.attention_varlen(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["cu_q"], d["cu_k"],
                                           dict(causal=causal))
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_BF16, what="varlen ragged")


def test_varlen_cross_lengths():
    """Query and key lengths differ per sequence (bottom-right causal alignment)."""
    lq = [3, 40, 200, 1, 0, 65]
    lk = [10, 40, 150, 300, 7, 0]
    d = synth.make_varlen(lq, lk, 4, 2, 128, 128, seed=31)
    for causal in (False, True):
        o, lse = _varlen_run(d, dict(causal=causal), 128)
        o_ref, l_ref = oracle.attention_varlen(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["cu_q"], d["cu_k"],
                                               dict(causal=causal))
        compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_BF16, what=f"cross c{causal}")


def test_varlen_packing_is_bitwise_invariant():
    """A sequence gives bit-identical O/LSE alone and packed at any offset."""
    lens = [77, 300, 129]
    d = synth.make_varlen(lens, lens, 4, 4, 128, 128, seed=41)
    o_all, l_all = _varlen_run(d, dict(causal=True), 128)
    cu = d["cu_q"].tolist()
    for b in range(3):
        sl = slice(cu[b], cu[b + 1])
        one = dict(q=d["q"][sl], k=d["k"][sl], v=d["v"][sl], cu_q=torch.tensor([0, lens[b]], dtype=torch.int32),
                   cu_k=torch.tensor([0, lens[b]], dtype=torch.int32), lengths_q=[lens[b]], lengths_k=[lens[b]])
        o1, l1 = _varlen_run(one, dict(causal=True), 128)
        assert torch.equal(o1, o_all[sl]) and torch.equal(l1, l_all[:, sl])


def test_varlen_full_size_sampled():
    """H=16, D=128, 8 sequences with lengths uniform in [0,4096] (one zero,
    several not multiples of 64), causal; sampled rows against the oracle."""
    lens = synth.varlen_lengths(synth.seed_for(2))
    d = synth.make_varlen(lens, lens, 16, 16, 128, 128, seed=synth.seed_for(2))
    o, lse = _varlen_run(d, dict(causal=True), 128)
    rng = np.random.default_rng(5)
    picks = []
    for b, L in enumerate(lens):
        if L == 0:
            continue
        rows = sorted({0, 1, 63, 64, L - 1, L // 2, *rng.integers(0, L, 4).tolist()} & set(range(L)))
        for h in (0, 7, 15):
            picks += [(b, h, i) for i in rows]
    o_ref, l_ref = oracle.varlen_rows(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["cu_q"], d["cu_k"], picks,
                                      dict(causal=True))
    cu = d["cu_q"].tolist()
    og = torch.stack([o[cu[b] + i, h] for b, h, i in picks])
    lg = torch.stack([lse[h, cu[b] + i] for b, h, i in picks])
    compare(og, lg, o_ref, l_ref, TOL_O_BF16, what="varlen full")
    # every row of the packed output was written and is finite
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


# ----------------------------------------------------------------------------- closed forms on the GPU
def test_q_zero_gives_log_visible_count():
    lens = [100, 257, 64]
    d = synth.make_varlen(lens, lens, 2, 2, 128, 128, seed=51)
    d["q"] = torch.zeros_like(d["q"])
    for mods in (dict(causal=True), dict(window=(37, 0)), dict()):
        o, lse = _varlen_run(d, mods, 128)
        cu = d["cu_q"].tolist()
        for b, L in enumerate(lens):
            i = np.arange(L)
            if mods.get("causal"):
                n = i + 1
            elif "window" in mods:
                n = np.minimum(i, 37) + 1
            else:
                n = np.full(L, L)
            got = lse[:, cu[b]:cu[b + 1]].double().cpu().numpy()
            assert np.max(np.abs(got - np.log(n)[None, :])) < TOL_LSE


def test_diagonal_window_is_exact():
    """window (0,0): each row sees only its own key, so O equals that V row
    exactly and LSE equals that single scaled logit."""
    lens = [70, 129]
    d = synth.make_varlen(lens, lens, 4, 2, 128, 128, seed=61)
    d["v"] = torch.randint(-8, 9, d["v"].shape).to(torch.bfloat16)
    o, lse = _varlen_run(d, dict(window=(0, 0)), 128)
    qf, kf = d["q"].double(), d["k"].double()
    for h in range(4):
        g = h // 2
        assert torch.equal(o[:, h].cpu(), d["v"][:, g])
        s = (qf[:, h] * kf[:, g]).sum(-1) / math.sqrt(128)
        assert torch.max(torch.abs(lse[h].double().cpu() - s)) < TOL_LSE


def test_peaked_queries_pair_k_with_v():
    """Q_i = alpha * K_sigma(i): each row's softmax concentrates on one key, so any
    K/V row-pairing or permutation mistake shows as a large O error."""
    L = 256
    d = synth.make_varlen([L], [L], 2, 2, 128, 128, seed=71)
    sigma = torch.randperm(L, generator=torch.Generator().manual_seed(7))
    d["q"] = synth.peaked_queries(d["k"][sigma], 1.5)
    o, lse = _varlen_run(d, dict(), 128)
    o_ref, l_ref = oracle.attention_varlen(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["cu_q"], d["cu_k"], dict())
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_BF16, what="peaked")
    # the peak really dominates: O is close to the selected V row
    assert torch.max(torch.abs(o[:, 0].float().cpu() - d["v"][sigma, 0].float())) < 0.5


# ----------------------------------------------------------------------------- paged
def _paged_run(d, mods_kw, Dv, workspace=True):
    q = d["q"].to(DEV)
    kc, vc = d["k_cache"].to(DEV), d["v_cache"].to(DEV)
    Tq, Hq, Dqk = q.shape
    P, Hkv, ps, _ = kc.shape
    B = len(d["lengths_k"])
    msq, msk = max(d["lengths_q"]), max(d["lengths_k"])
    o = _nan_like((Tq, Hq, Dv), torch.bfloat16)
    lse = _nan_like((Hq, Tq), torch.float32)
    fp8 = kc.dtype == torch.uint8
    ws = None
    if workspace:
        n = fa.fa_fwd_paged_workspace_size(B, Tq, msq, msk, Hq, Hkv, Dqk, Dv, ps,
                                           fa.FA_FP8_E4M3 if fp8 else fa.FA_BF16)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
    fa.fa_fwd_paged(q, kc, vc, o, lse, d["cu_q"].to(DEV), d["seqlen_k"].to(DEV), d["block_table"].to(DEV),
                    msq, msk, d["k_descale"].to(DEV), d["v_descale"].to(DEV), ws, fa.Mods(**mods_kw))
    torch.cuda.synchronize()
    return o, lse


def _paged_ref(d, mods_kw):
    return oracle.attention_paged(f64(d["q"]), f64(d["k_cache"]), f64(d["v_cache"]), d["cu_q"], d["seqlen_k"],
                                  d["block_table"], dict(mods_kw), float(d["k_descale"]), float(d["v_descale"]))


@pytest.mark.parametrize("ps", [64, 16, 128, 8, 1])
def test_paged_fp8_prefill_small(ps):
    lk = [70, 3, 128, 129, 600]
    lq = [70, 3, 128, 129, 600]
    d = synth.make_paged(lq, lk, 4, 4, 192, 128, page_size=ps, seed=81 + ps, extra_pages=3)
    o, lse = _paged_run(d, dict(causal=True), 128)
    o_ref, l_ref = _paged_ref(d, dict(causal=True))
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8, what=f"paged ps{ps}")


def test_paged_fp8_chunked_prefill_and_gqa():
    """Fewer queries than keys (bottom-right causal), GQA 2:1, D 128/128."""
    lk = [300, 64, 1000]
    lq = [40, 64, 100]
    d = synth.make_paged(lq, lk, 4, 2, 128, 128, page_size=64, seed=91)
    o, lse = _paged_run(d, dict(causal=True), 128)
    o_ref, l_ref = _paged_ref(d, dict(causal=True))
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8, what="chunked")


def _reshuffle(d, seed):
    """Same logical cache, different physical page placement."""
    P = d["k_cache"].shape[0]
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(seed))
    e = dict(d)
    e["k_cache"] = torch.empty_like(d["k_cache"])
    e["v_cache"] = torch.empty_like(d["v_cache"])
    e["k_cache"][perm] = d["k_cache"]
    e["v_cache"][perm] = d["v_cache"]
    e["block_table"] = perm.to(torch.int32)[d["block_table"].long()]
    return e


@pytest.mark.parametrize("ps", [64, 1])
@pytest.mark.parametrize("lq", [[200, 64, 1], [1, 1, 1]])
def test_paged_placement_is_bitwise_invariant(lq, ps):
    lk = [300, 64, 700]
    d = synth.make_paged(lq, lk, 8, 1 if lq[0] == 1 else 8, 192, 128, page_size=ps, seed=95, extra_pages=11)
    o1, l1 = _paged_run(d, dict(causal=True), 128)
    e = _reshuffle(d, 3)
    o2, l2 = _paged_run(e, dict(causal=True), 128)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_full_prefill_sampled():
    """Q [8192,16,192] bf16, FP8 K (192) / V (128) in pages of 64 with a
    shuffled block table, 4 sequences of 2048, causal; sampled rows."""
    L = [2048] * 4
    d = synth.make_paged(L, L, 16, 16, 192, 128, page_size=64, seed=synth.seed_for(3))
    o, lse = _paged_run(d, dict(causal=True), 128)
    rng = np.random.default_rng(3)
    picks = [(b, h, int(i)) for b in range(4) for h in (0, 9, 15) for i in {0, 1, 2047, 1024, *rng.integers(0, 2048, 3).tolist()}]
    o_ref, l_ref = oracle.paged_rows(f64(d["q"]), f64(d["k_cache"]), f64(d["v_cache"]), d["cu_q"], d["seqlen_k"],
                                     d["block_table"], picks, dict(causal=True),
                                     float(d["k_descale"]), float(d["v_descale"]))
    cu = d["cu_q"].tolist()
    og = torch.stack([o[cu[b] + i, h] for b, h, i in picks])
    lg = torch.stack([lse[h, cu[b] + i] for b, h, i in picks])
    compare(og, lg, o_ref, l_ref, TOL_O_FP8, what="paged full")


# ----------------------------------------------------------------------------- vectorised pages
def _paged_vec_run(d, mods_kw, Dv):
    """fa_fwd_paged_vec over the vectorised copy of a make_paged() cache."""
    e = synth.to_vectorized(d)
    q = d["q"].to(DEV)
    kc, vc = e["k_cache"].to(DEV), e["v_cache"].to(DEV)
    Tq, Hq, Dqk = q.shape
    P, Hkv, _, ps, _ = kc.shape
    B = len(d["lengths_k"])
    msq, msk = max(d["lengths_q"]), max(d["lengths_k"])
    o = _nan_like((Tq, Hq, Dv), torch.bfloat16)
    lse = _nan_like((Hq, Tq), torch.float32)
    n = fa.fa_fwd_paged_workspace_size(B, Tq, msq, msk, Hq, Hkv, Dqk, Dv, ps, fa.FA_FP8_E4M3)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
    fa.fa_fwd_paged_vec(q, kc, vc, o, lse, d["cu_q"].to(DEV), d["seqlen_k"].to(DEV), d["block_table"].to(DEV),
                        msq, msk, d["k_descale"].to(DEV), d["v_descale"].to(DEV), ws, fa.Mods(**mods_kw))
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("decode", [False, True])
@pytest.mark.parametrize("vec", [False, True])
@pytest.mark.parametrize("dv", [128, 192])
def test_paged_fp8_peaked_queries_pair_k_with_v(vec, dv, decode):
    """Paged FP8 prefill (or single-query decode) with each query equal to
    1.5 x the dequantised K row of one visible key: the softmax concentrates
    on that key, so any K/V row pairing mistake in the E4M3 staging or the
    transposed byte reads shows as a large O error (random queries spread P
    too thinly to expose it)."""
    L = [200, 77]
    lq = [1, 1] if decode else L
    Hq, Hkv = (16, 2) if decode else (4, 2)
    d = synth.make_paged(lq, L, Hq, Hkv, 192, dv, page_size=16 if vec else 64, seed=97)
    gen = torch.Generator().manual_seed(5)
    q = d["q"].clone()
    cu = d["cu_q"].tolist()
    picks = []
    for b, n in enumerate(L):
        rows = [oracle.gather_paged(f64(d["k_cache"]), d["block_table"][b].numpy(), n, g, float(d["k_descale"]))
                for g in range(Hkv)]
        for i in range(lq[b]):
            ip = i + n - lq[b]                                         # aligned position (bottom-right)
            j = int(torch.randint(0, ip + 1, (1,), generator=gen))    # a key row i sees (causal)
            picks.append((b, i, j))
            for h in range(Hq):
                q[cu[b] + i, h] = synth.peaked_queries(torch.from_numpy(rows[h // (Hq // Hkv)][j]), 1.5)
    d["q"] = q
    o, lse = (_paged_vec_run(d, dict(causal=True), dv) if vec else _paged_run(d, dict(causal=True), dv))
    o_ref, l_ref = _paged_ref(d, dict(causal=True))
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8,
            what=f"peaked vec={vec} dv={dv} decode={decode}")
    # the peak dominates: O of head 0 is close to the picked V row
    worst = 0.0
    for b, n in enumerate(L):
        vrows = oracle.gather_paged(f64(d["v_cache"]), d["block_table"][b].numpy(), n, 0, float(d["v_descale"]))
        for (bb, i, j) in picks:
            if bb == b:
                worst = max(worst, float(np.max(np.abs(o[cu[b] + i, 0].float().cpu().numpy() - vrows[j]))))
    assert worst < 0.5, worst


# (lengths_q, lengths_k, Hq, Hkv, Dqk, mods): prefill, chunked prefill with
# GQA, decode with one row block, decode with two row blocks and a window
VEC_CASES = {
    "prefill": ([70, 3, 128, 129, 600], [70, 3, 128, 129, 600], 4, 4, 192, dict(causal=True)),
    "chunked": ([40, 64, 100], [300, 64, 1000], 4, 2, 128, dict(causal=True)),
    "decode": ([1] * 8, [1, 31, 32, 33, 64, 1000, 3000, 257], 16, 2, 192, dict(causal=True)),
    "decode2rb": ([2, 1, 2, 2, 2, 2, 0, 2], [0, 1, 2, 33, 500, 2100, 64, 5000], 32, 2, 192,
                  dict(causal=True, window=(100, 0))),
}


@pytest.mark.parametrize("ps", [16, 32, 64, 1024])
@pytest.mark.parametrize("case", sorted(VEC_CASES))
def test_paged_vec_is_bitwise_head_major(case, ps):
    """The vectorised page format gives bitwise the head-major result for the
    same logical cache (unused pages and bytes past seqlen_k hold NaN codes
    in both: value bytes that share a load with live ones are cleared)."""
    lq, lk, Hq, Hkv, Dqk, mods_kw = VEC_CASES[case]
    d = synth.make_paged(lq, lk, Hq, Hkv, Dqk, 128, page_size=ps, seed=171 + ps, extra_pages=5)
    o1, l1 = _paged_run(d, mods_kw, 128)
    o2, l2 = _paged_vec_run(d, mods_kw, 128)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{case} ps{ps}"


@pytest.mark.parametrize("case,ps", [("decode", 16), ("prefill", 64), ("chunked", 1024)])
def test_paged_vec_matches_oracle(case, ps):
    """Oracle parity with the oracle reading the vectorised pages itself."""
    lq, lk, Hq, Hkv, Dqk, mods_kw = VEC_CASES[case]
    d = synth.make_paged(lq, lk, Hq, Hkv, Dqk, 128, page_size=ps, seed=191 + ps, extra_pages=2)
    o, lse = _paged_vec_run(d, mods_kw, 128)
    e = synth.to_vectorized(d)
    o_ref, l_ref = oracle.attention_paged(f64(d["q"]), f64(e["k_cache"]), f64(e["v_cache"]), d["cu_q"],
                                          d["seqlen_k"], d["block_table"], dict(mods_kw),
                                          float(d["k_descale"]), float(d["v_descale"]), layout="vectorized")
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8, what=f"vec {case} ps{ps}")


# ----------------------------------------------------------------------------- E4M3 queries
def _paged_q8_run(d, mods_kw, Dv, vec=False):
    """Paged call with E4M3 queries (fa_fwd_paged_ex), head-major or vectorised pages."""
    e = synth.to_vectorized(d) if vec else d
    q, qd = d["q"].to(DEV), d["q_descale"].to(DEV)
    kc, vc = e["k_cache"].to(DEV), e["v_cache"].to(DEV)
    Tq, Hq, Dqk = q.shape
    Hkv, ps = kc.shape[1], (kc.shape[3] if vec else kc.shape[2])
    B = len(d["lengths_k"])
    msq, msk = max(d["lengths_q"]), max(d["lengths_k"])
    o = _nan_like((Tq, Hq, Dv), torch.bfloat16)
    lse = _nan_like((Hq, Tq), torch.float32)
    n = fa.fa_fwd_paged_workspace_size(B, Tq, msq, msk, Hq, Hkv, Dqk, Dv, ps, fa.FA_FP8_E4M3)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
    fn = fa.fa_fwd_paged_vec if vec else fa.fa_fwd_paged
    fn(q, kc, vc, o, lse, d["cu_q"].to(DEV), d["seqlen_k"].to(DEV), d["block_table"].to(DEV), msq, msk,
       d["k_descale"].to(DEV), d["v_descale"].to(DEV), ws, fa.Mods(**mods_kw), q_descale=qd)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("case,ps", [("prefill", 64), ("chunked", 16), ("decode", 64), ("decode2rb", 32)])
def test_paged_fp8_queries_match_oracle(case, ps):
    """E4M3 queries with a per-tensor q descale (prefill converts them
    exactly to bf16; decode feeds the codes to the FP8 product as they are);
    head-major and vectorised pages give bitwise the same result."""
    lq, lk, Hq, Hkv, Dqk, mods_kw = VEC_CASES[case]
    d = synth.make_paged(lq, lk, Hq, Hkv, Dqk, 128, page_size=ps, seed=211 + ps, extra_pages=3, q_dtype="fp8")
    o, lse = _paged_q8_run(d, mods_kw, 128)
    o_ref, l_ref = oracle.attention_paged(f64(d["q"]), f64(d["k_cache"]), f64(d["v_cache"]), d["cu_q"],
                                          d["seqlen_k"], d["block_table"], dict(mods_kw), float(d["k_descale"]),
                                          float(d["v_descale"]), q_descale=float(d["q_descale"]))
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8, what=f"q8 {case} ps{ps}")
    o2, l2 = _paged_q8_run(d, mods_kw, 128, vec=True)
    assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_paged_fp8_queries_need_q_descale():
    d = synth.make_paged([1], [40], 16, 2, 192, 128, page_size=64, seed=5, q_dtype="fp8")
    with pytest.raises(TypeError):
        fa.fa_fwd_paged(d["q"].to(DEV), d["k_cache"].to(DEV), d["v_cache"].to(DEV),
                        torch.empty((1, 16, 128), dtype=torch.bfloat16, device=DEV),
                        torch.empty((16, 1), dtype=torch.float32, device=DEV), d["cu_q"].to(DEV),
                        d["seqlen_k"].to(DEV), d["block_table"].to(DEV), 1, 40, d["k_descale"].to(DEV),
                        d["v_descale"].to(DEV))


# ----------------------------------------------------------------------------- value width 192
# (lengths_q, lengths_k, Hq, Hkv, mods): Q/K and V/O width 192
V192_CASES = {
    "prefill": ([70, 3, 128, 129, 300], [70, 3, 128, 129, 300], 4, 4, dict(causal=True)),
    "chunked": ([40, 64, 100], [300, 64, 1000], 4, 2, dict(causal=True)),
    "decode": ([1] * 6, [1, 31, 33, 64, 1000, 3000], 16, 2, dict(causal=True)),
    "decode2rb": ([2, 1, 2, 0, 2], [0, 1, 33, 64, 2100], 32, 2, dict(causal=True, window=(100, 0))),
}


@pytest.mark.parametrize("ps", [64, 16])
@pytest.mark.parametrize("case", sorted(V192_CASES))
def test_paged_v192_matches_oracle(case, ps):
    """D_qk = D_v = 192 (the pages' V192 variant) over FP8 pages: oracle
    parity on head-major pages, bitwise equality on vectorised pages."""
    lq, lk, Hq, Hkv, mods_kw = V192_CASES[case]
    d = synth.make_paged(lq, lk, Hq, Hkv, 192, 192, page_size=ps, seed=231 + ps, extra_pages=3)
    o, lse = _paged_run(d, mods_kw, 192)
    o_ref, l_ref = _paged_ref(d, mods_kw)
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8, what=f"v192 {case} ps{ps}")
    o2, l2 = _paged_vec_run(d, mods_kw, 192)
    assert torch.equal(o, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("case", ["chunked", "decode2rb"])
def test_paged_v192_fp8_queries(case):
    lq, lk, Hq, Hkv, mods_kw = V192_CASES[case]
    d = synth.make_paged(lq, lk, Hq, Hkv, 192, 192, page_size=64, seed=241, extra_pages=2, q_dtype="fp8")
    o, lse = _paged_q8_run(d, mods_kw, 192, vec=True)
    o_ref, l_ref = oracle.attention_paged(f64(d["q"]), f64(d["k_cache"]), f64(d["v_cache"]), d["cu_q"],
                                          d["seqlen_k"], d["block_table"], dict(mods_kw), float(d["k_descale"]),
                                          float(d["v_descale"]), q_descale=float(d["q_descale"]))
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8, what=f"v192 q8 {case}")


# ----------------------------------------------------------------------------- FP8 KV-cache write
def _kv_rows(T, Hkv, Dqk, Dv, seed, special=False):
    g = torch.Generator().manual_seed(seed)
    k = (torch.randn((T, Hkv, Dqk), generator=g) * 3).to(torch.bfloat16)
    v = (torch.randn((T, Hkv, Dv), generator=g) * 0.5).to(torch.bfloat16)
    if special:
        # every E4M3 midpoint (ties), values near them, the subnormal range
        # and values past 448, all exact in bf16
        codes = torch.arange(0, 0x7E, dtype=torch.int64)
        lo = torch.from_numpy(oracle.decode_e4m3(codes.numpy().astype("uint8")))
        hi = torch.from_numpy(oracle.decode_e4m3((codes + 1).numpy().astype("uint8")))
        mids = ((lo + hi) / 2).to(torch.bfloat16)
        extra = torch.tensor([448.0, 460.0, 500.0, 1e4, -1e4, 2 ** -10, 3 * 2 ** -10, -(2 ** -8), 0.0, -0.0],
                             dtype=torch.bfloat16)
        vals = torch.cat([mids, -mids, extra])
        flat = k.view(-1)
        flat[: vals.numel()] = vals
    return k, v


@pytest.mark.parametrize("layout,ps", [("head_major", 64), ("head_major", 1), ("vectorized", 16),
                                       ("vectorized", 64)])
@pytest.mark.parametrize("given", [False, True])
def test_kv_cache_write_is_bitwise_the_oracle(layout, ps, given):
    """Codes and descales bitwise equal to the oracle: random rows, every
    E4M3 midpoint, subnormals and saturation (given descale 1 for K), with
    skipped and out-of-range slots; untouched bytes keep their NaN fill."""
    T, Hkv, Dqk, Dv, P = 300, 2, 192, 128, 24
    k, v = _kv_rows(T, Hkv, Dqk, Dv, seed=ps + 7, special=given)
    g = torch.Generator().manual_seed(ps)
    slots = torch.randperm(P * ps, generator=g)[:T].to(torch.int64)
    if P * ps < T:
        slots = torch.randint(0, P * ps, (T,), generator=g)
        slots = torch.unique(slots)
        slots = torch.cat([slots, torch.full((T - slots.numel(),), -1, dtype=torch.int64)])
    slots[5], slots[17] = -1, P * ps + 100
    if layout == "head_major":
        kc0 = torch.full((P, Hkv, ps, Dqk), 0x7F, dtype=torch.uint8)
        vc0 = torch.full((P, Hkv, ps, Dv), 0x7F, dtype=torch.uint8)
    else:
        kc0 = torch.full((P, Hkv, Dqk // 16, ps, 16), 0x7F, dtype=torch.uint8)
        vc0 = torch.full((P, Hkv, ps // 16, Dv, 16), 0x7F, dtype=torch.uint8)
    kd0, vd0 = (1.0, 0.02) if given else (None, None)
    kc_r, vc_r, kd_r, vd_r = oracle.kv_cache_write(k.float().numpy(), v.float().numpy(), slots.numpy(), kc0.numpy(),
                                                   vc0.numpy(), ps, layout, kd0, vd0)
    kc, vc = kc0.to(DEV), vc0.to(DEV)
    kd = torch.tensor([kd0 if given else float("nan")], dtype=torch.float32, device=DEV)
    vd = torch.tensor([vd0 if given else float("nan")], dtype=torch.float32, device=DEV)
    ws = torch.empty(max(fa.fa_kv_cache_write_fp8_workspace_size(T, Hkv, Dqk, Dv), 4), dtype=torch.uint8, device=DEV)
    fa.fa_kv_cache_write_fp8(k.to(DEV), v.to(DEV), slots.to(DEV), kc, vc, kd, vd, compute_scale=not given,
                             workspace=ws)
    torch.cuda.synchronize()
    assert np.float32(kd.item()) == np.float32(kd_r) and np.float32(vd.item()) == np.float32(vd_r)
    assert np.array_equal(kc.cpu().numpy(), kc_r), (kc.cpu().numpy() != kc_r).sum()
    assert np.array_equal(vc.cpu().numpy(), vc_r), (vc.cpu().numpy() != vc_r).sum()


def test_kv_cache_write_then_decode():
    """A cache filled by the writer serves the decode path: same result as
    the oracle attention over the oracle-written cache."""
    lk = [100, 1000, 37]
    B, Hq, Hkv, ps = 3, 16, 2, 64
    d = synth.make_paged([1] * B, lk, Hq, Hkv, 192, 128, page_size=ps, seed=251, extra_pages=4)
    T = sum(lk)
    k, v = _kv_rows(T, Hkv, 192, 128, seed=3)
    bt = d["block_table"]
    slots = torch.cat([bt[b, torch.arange(lk[b]) // ps].long() * ps + torch.arange(lk[b]) % ps for b in range(B)])
    kc = torch.full_like(d["k_cache"], 0x7F).to(DEV)
    vc = torch.full_like(d["v_cache"], 0x7F).to(DEV)
    kd = torch.empty(1, dtype=torch.float32, device=DEV)
    vd = torch.empty(1, dtype=torch.float32, device=DEV)
    ws = torch.empty(fa.fa_kv_cache_write_fp8_workspace_size(T, Hkv, 192, 128), dtype=torch.uint8, device=DEV)
    fa.fa_kv_cache_write_fp8(k.to(DEV), v.to(DEV), slots.to(DEV), kc, vc, kd, vd, workspace=ws)
    e = dict(d, k_cache=kc, v_cache=vc, k_descale=kd, v_descale=vd)
    o, lse = _paged_run(e, dict(causal=True), 128)
    kc_r, vc_r, kd_r, vd_r = oracle.kv_cache_write(k.float().numpy(), v.float().numpy(), slots.numpy(),
                                                   torch.full_like(d["k_cache"], 0x7F).numpy(),
                                                   torch.full_like(d["v_cache"], 0x7F).numpy(), ps)
    o_ref, l_ref = oracle.attention_paged(f64(d["q"]), kc_r, vc_r, d["cu_q"], d["seqlen_k"], d["block_table"],
                                          dict(causal=True), float(kd_r), float(vd_r))
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8, what="written cache")


# ----------------------------------------------------------------------------- decode
@pytest.mark.parametrize("Hq,Hkv,Dqk,sq", [(16, 2, 192, 1), (8, 8, 128, 1), (16, 2, 192, 4), (64, 8, 192, 1)])
def test_decode_small(Hq, Hkv, Dqk, sq):
    lk = [1, 31, 32, 33, 64, 1000, 3000, 257]
    lq = [min(sq, l) for l in lk]
    d = synth.make_paged(lq, lk, Hq, Hkv, Dqk, 128, page_size=64, seed=101 + Hq + sq, extra_pages=5)
    o, lse = _paged_run(d, dict(causal=True), 128)
    o_ref, l_ref = _paged_ref(d, dict(causal=True))
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8, what="decode")


@pytest.mark.parametrize("ps,Hq,Hkv,sq", [(16, 16, 2, 1), (8, 16, 2, 1), (1, 16, 2, 1), (8, 32, 2, 2)])
def test_decode_small_pages(ps, Hq, Hkv, sq):
    """Pages smaller than the 32-key decode tile: each lane looks up the page
    of its key row (bytes past seqlen_k and unused pages hold NaN)."""
    lk = [1, 31, 32, 33, 64, 300, 1000, 77]
    lq = [min(sq, l) for l in lk]
    d = synth.make_paged(lq, lk, Hq, Hkv, 192, 128, page_size=ps, seed=151 + ps + sq, extra_pages=9)
    o, lse = _paged_run(d, dict(causal=True), 128)
    o_ref, l_ref = _paged_ref(d, dict(causal=True))
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8, what=f"decode ps{ps}")


def test_decode_many_short_units():
    """Many short sequences (1..120 keys, two without keys, two without a
    query), GQA 16/8: about 7800 tiles over 3072 wavefronts, so a wavefront
    takes tiles from several (sequence, kv-head) units and units are cut
    across wavefronts."""
    g = np.random.default_rng(7)
    lk = g.integers(1, 121, 400).tolist()
    lk[3] = lk[10] = 0
    lq = [1] * 400
    lq[5] = lq[20] = 0
    d = synth.make_paged(lq, lk, 16, 8, 128, 128, page_size=32, seed=131, extra_pages=7)
    o, lse = _paged_run(d, dict(causal=True), 128)
    o_ref, l_ref = _paged_ref(d, dict(causal=True))
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8, what="decode short units")


@pytest.mark.parametrize("mods_kw", [dict(causal=True), dict(causal=True, window=(100, 0)), dict(window=(50, 3))])
def test_decode_two_row_blocks(mods_kw):
    """Two queries x 16 q-heads per kv-head = 32 rows per unit (two row
    blocks per wavefront), with empty and key-starved sequences."""
    lk = [0, 1, 2, 33, 500, 2100, 64, 5000]
    lq = [2, 1, 2, 2, 2, 2, 0, 2]
    d = synth.make_paged(lq, lk, 32, 2, 192, 128, page_size=64, seed=137, extra_pages=3)
    o, lse = _paged_run(d, mods_kw, 128)
    o_ref, l_ref = _paged_ref(d, mods_kw)
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8, what=f"decode 2rb {mods_kw}")


@pytest.mark.parametrize("lq", [[1, 1, 1, 1], [40, 64, 100, 33]])
def test_paged_pages_beyond_4gib(lq):
    """Page ids up to 2^19 (K cache 51.5 GB, V 34.4 GB: byte offsets above
    2^35) with the highest ids in use: decode (one query) and chunked
    prefill give bitwise the results of the same logical sequences in a
    compact cache, and those match the oracle."""
    num_pages = 524289
    need = num_pages * 8 * 64 * (192 + 128) + (4 << 30)
    if torch.cuda.mem_get_info()[0] < need:
        pytest.skip("needs %.1f GB of free device memory" % (need / 1e9))
    lk = [700, 64, 1000, 33]
    seed = synth.seed_for(4) + 7
    big = synth.make_paged(lq, lk, 64, 8, 192, 128, page_size=64, seed=seed, device=DEV,
                           min_pages=num_pages, place_high=6)
    assert int(big["block_table"].max()) == num_pages - 1
    o1, l1 = _paged_run(big, dict(causal=True), 128)
    del big
    torch.cuda.empty_cache()
    # same generator device as above, so the logical K/V and Q are the same values
    small = synth.make_paged(lq, lk, 64, 8, 192, 128, page_size=64, seed=seed, device=DEV, extra_pages=2)
    o2, l2 = _paged_run(small, dict(causal=True), 128)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, l_ref = _paged_ref({k: (v.cpu() if torch.is_tensor(v) else v) for k, v in small.items()}, dict(causal=True))
    compare(o2.permute(1, 0, 2), l2, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8, what="pages beyond 4 GiB")


def test_decode_requires_workspace():
    d = synth.make_paged([1, 1], [100, 50], 16, 2, 192, 128, page_size=64, seed=111)
    with pytest.raises(fa.FaError) as e:
        _paged_run(d, dict(), 128, workspace=False)
    assert e.value.code == -4


@pytest.mark.parametrize("variant", ["head_major", "vec", "vec_q8", "v192_q8"])
def test_decode_full_size_sampled(variant):
    """64 sequences, contexts uniform in [1024, 32768], GQA 64/8, D 192/128
    (192/192 for v192), pages of 64 with a shuffled block table, in the
    launch configuration the benchmark times; 6 sequences checked in full,
    the oracle reading the same page format and query type."""
    lk = synth.make_decode_lengths(synth.seed_for(4))
    lq = [1] * 64
    Dv = 192 if variant.startswith("v192") else 128
    q8 = variant.endswith("q8")
    vec = variant != "head_major"
    d = synth.make_paged(lq, lk, 64, 8, 192, Dv, page_size=64, seed=synth.seed_for(4), device=DEV,
                         q_dtype="fp8" if q8 else "bf16")
    if q8:
        o, lse = _paged_q8_run(d, dict(causal=True), Dv, vec=vec)
    elif vec:
        o, lse = _paged_vec_run(d, dict(causal=True), Dv)
    else:
        o, lse = _paged_run(d, dict(causal=True), Dv)
    e = synth.to_vectorized(d) if vec else d
    bsel = [0, 5, 17, 33, 50, 63]
    picks = [(b, h, 0) for b in bsel for h in range(64)]
    o_ref, l_ref = oracle.paged_rows(f64(d["q"]), f64(e["k_cache"]), f64(e["v_cache"]), d["cu_q"].cpu(),
                                     d["seqlen_k"].cpu(), d["block_table"].cpu(), picks, dict(causal=True),
                                     float(d["k_descale"]), float(d["v_descale"]),
                                     layout="vectorized" if vec else "head_major",
                                     q_descale=float(d["q_descale"]) if q8 else None)
    og = torch.stack([o[b, h] for b, h, _ in picks])
    lg = torch.stack([lse[h, b] for b, h, _ in picks])
    compare(og, lg, o_ref, l_ref, TOL_O_FP8, what=f"decode full {variant}")


# ----------------------------------------------------------------------------- flex
FLEX_CASES = {
    "alibi": dict(alibi_slope=0.0625),
    "softcap": dict(softcap=20.0),
    "window": dict(window=(256, 0)),
    "window_sym": dict(window=(16, 8)),
    "alibi_softcap_causal": dict(alibi_slope=0.25, softcap=5.0, causal=True),
}


@pytest.mark.parametrize("case", sorted(FLEX_CASES))
def test_flex_mods_small(case):
    d = synth.make_dense(2, 300, 300, 2, 2, 128, 128, seed=121)
    mods = FLEX_CASES[case]
    o, lse = _dense_run(d, mods, 128)
    o_ref, l_ref = oracle.attention_dense(f64(d["q"]), f64(d["k"]), f64(d["v"]), dict(mods))
    compare(o.permute(0, 2, 1, 3), lse, o_ref.transpose(0, 2, 1, 3), l_ref, TOL_O_BF16, what=case)


@pytest.mark.parametrize("kind", ["bernoulli", "block_causal", "bernoulli_causal"])
def test_flex_block_mask_small(kind):
    B, H, S = 2, 2, 640
    nb = math.ceil(S / 128)
    if kind.startswith("bernoulli"):
        bm = synth.bernoulli_block_mask(B * H, nb, nb, 0.5, seed=131)
        bm[0, 1, :] = 0          # a fully masked query block
    else:
        bm = synth.block_causal_mask(B * H, nb, nb)
    d = synth.make_dense(B, S, S, H, H, 128, 128, seed=132)
    mods = dict(block_mask=bm.to(DEV), mask_block=(128, 128), causal=kind.endswith("causal") and kind != "block_causal")
    o, lse = _dense_run(d, mods, 128)
    o_ref, l_ref = oracle.attention_dense(f64(d["q"]), f64(d["k"]), f64(d["v"]), _oracle_mods(mods))
    compare(o.permute(0, 2, 1, 3), lse, o_ref.transpose(0, 2, 1, 3), l_ref, TOL_O_BF16, what=kind)


@pytest.mark.parametrize("case", ["alibi", "softcap", "window", "bernoulli", "block_causal"])
def test_flex_full_size_sampled(case):
    """B=2, H=16, S=8192, D=128 (non-causal unless stated); sampled rows."""
    B, H, S = 2, 16, 8192
    d = synth.make_dense(B, S, S, H, H, 128, 128, seed=synth.seed_for(5))
    if case == "bernoulli":
        mods = dict(block_mask=synth.bernoulli_block_mask(B * H, 64, 64, 0.5, seed=synth.seed_for(5, 3)).to(DEV))
    elif case == "block_causal":
        mods = dict(block_mask=synth.block_causal_mask(B * H, 64, 64).to(DEV))
    else:
        mods = dict(FLEX_CASES[case])
    o, lse = _dense_run(d, mods, 128)
    rng = np.random.default_rng(9)
    rows = sorted({0, 1, 127, 128, 4095, 8191, *rng.integers(0, S, 4).tolist()})
    picks = [(b, h, i) for b in range(B) for h in (0, 11) for i in rows]
    qv = f64(d["q"]).reshape(B * S, H, 128)
    kv = f64(d["k"]).reshape(B * S, H, 128)
    vv = f64(d["v"]).reshape(B * S, H, 128)
    cu = np.array([0, S, 2 * S])
    o_ref, l_ref = oracle.varlen_rows(qv, kv, vv, cu, cu, picks, _oracle_mods(mods))
    og = torch.stack([o[b, i, h] for b, h, i in picks])
    lg = torch.stack([lse[b, h, i] for b, h, i in picks])
    compare(og, lg, o_ref, l_ref, TOL_O_BF16, what=f"flex full {case}")
