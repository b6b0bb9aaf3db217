"""GPU parity of exported paths beyond the main parity file: bf16 page caches
(prefill, chunked prefill and single-query rows, page sizes 1 to 64, with
and without score mods), score mods at D = 64, windows on the FP8 paged
prefill, score mods and block masks on FP8 paged caches (prefill and
decode, every head-dim pair, both page formats, E4M3 queries), and bf16
queries far from unit scale against FP8 caches (the per-row power-of-two
split of the queries).  Every call goes through the C
ABI; every result is compared with the fp64 oracle on the same inputs.
"""
import math

import pytest
import torch

import oracle
import synth
from tests.helpers import TOL_O_BF16, TOL_O_FP8, compare, f64
from tests.test_gpu_parity import (FLEX_CASES, VEC_CASES, _dense_run, _oracle_mods, _paged_q8_run, _paged_ref,
                                   _paged_run, _paged_vec_run, _varlen_run)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import attention_fa_fwd_03_amd as fa

DEV = "cuda"


def _cmp_packed(o, lse, o_ref, l_ref, tol, what):
    compare(o.permute(1, 0, 2), lse, o_ref.transpose(1, 0, 2), l_ref, tol, what=what)


# ----------------------------------------------------------------------------- bf16 pages
BF16_PAGED_LQ = {"prefill": [70, 3, 128, 129, 300], "chunked": [40, 3, 1, 64, 100], "decode": [1, 1, 1, 1, 1]}


@pytest.mark.parametrize("case", sorted(BF16_PAGED_LQ))
@pytest.mark.parametrize("ps", [1, 16, 64])
@pytest.mark.parametrize("D", [64, 128])
def test_bf16_paged_matches_oracle(D, ps, case):
    """bf16 caches in head-major pages (NaN in unused pages and past
    seqlen_k), GQA 4/2, causal."""
    lk = [70, 3, 128, 129, 300]
    d = synth.make_paged(BF16_PAGED_LQ[case], lk, 4, 2, D, D, page_size=ps, seed=601 + D + ps, kv_dtype="bf16",
                         extra_pages=3)
    o, lse = _paged_run(d, dict(causal=True), D)
    o_ref, l_ref = _paged_ref(d, dict(causal=True))
    _cmp_packed(o, lse, o_ref, l_ref, TOL_O_BF16, f"bf16 paged D{D} ps{ps} {case}")


@pytest.mark.parametrize("case", ["alibi", "softcap", "window_sym", "alibi_softcap_causal", "block_mask"])
def test_bf16_paged_mods(case):
    """Score mods and a block mask on bf16 pages (pages of 16, chunked rows)."""
    lq, lk = [300, 40, 200], [300, 64, 500]
    B, Hq = len(lq), 4
    d = synth.make_paged(lq, lk, Hq, 4, 128, 128, page_size=16, seed=611, kv_dtype="bf16", extra_pages=2)
    if case == "block_mask":
        bm = synth.bernoulli_block_mask(B * Hq, math.ceil(max(lq) / 128), math.ceil(max(lk) / 128), 0.5, seed=612)
        bm[1, 0, :] = 0    # a fully masked query block
        mods = dict(block_mask=bm.to(DEV), mask_block=(128, 128))
    else:
        mods = dict(FLEX_CASES[case])
    o, lse = _paged_run(d, mods, 128)
    o_ref, l_ref = _paged_ref(d, _oracle_mods(mods))
    _cmp_packed(o, lse, o_ref, l_ref, TOL_O_BF16, f"bf16 paged {case}")


# ----------------------------------------------------------------------------- mods at D = 64
@pytest.mark.parametrize("case", sorted(FLEX_CASES))
@pytest.mark.parametrize("layout", ["dense", "varlen"])
def test_flex_mods_d64(case, layout):
    mods = FLEX_CASES[case]
    if layout == "dense":
        d = synth.make_dense(2, 300, 300, 2, 2, 64, 64, seed=621)
        o, lse = _dense_run(d, mods, 64)
        o_ref, l_ref = oracle.attention_dense(f64(d["q"]), f64(d["k"]), f64(d["v"]), dict(mods))
        compare(o.permute(0, 2, 1, 3), lse, o_ref.transpose(0, 2, 1, 3), l_ref, TOL_O_BF16, what=f"d64 {case}")
    else:
        lq, lk = [5, 0, 130, 64, 300], [40, 0, 130, 64, 333]
        d = synth.make_varlen(lq, lk, 4, 2, 64, 64, seed=622)
        o, lse = _varlen_run(d, mods, 64)
        o_ref, l_ref = oracle.attention_varlen(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["cu_q"], d["cu_k"],
                                               dict(mods))
        _cmp_packed(o, lse, o_ref, l_ref, TOL_O_BF16, f"d64 varlen {case}")


def test_flex_block_mask_d64():
    B, H, S = 2, 2, 640
    nb = math.ceil(S / 128)
    bm = synth.bernoulli_block_mask(B * H, nb, nb, 0.5, seed=631)
    d = synth.make_dense(B, S, S, H, H, 64, 64, seed=632)
    mods = dict(block_mask=bm.to(DEV), mask_block=(128, 128), causal=True)
    o, lse = _dense_run(d, mods, 64)
    o_ref, l_ref = oracle.attention_dense(f64(d["q"]), f64(d["k"]), f64(d["v"]), _oracle_mods(mods))
    compare(o.permute(0, 2, 1, 3), lse, o_ref.transpose(0, 2, 1, 3), l_ref, TOL_O_BF16, what="d64 block mask")


# ----------------------------------------------------------------------------- FP8 paged prefill windows
@pytest.mark.parametrize("window", [(100, 0), (50, 3), (0, 0)])
@pytest.mark.parametrize("vec", [False, True])
def test_paged_fp8_prefill_window(window, vec):
    """Sliding windows on the FP8 paged prefill (rows enough for the prefill
    kernel), both page formats, D 192/128."""
    lq, lk = [300, 40, 200], [300, 64, 700]
    d = synth.make_paged(lq, lk, 4, 4, 192, 128, page_size=64, seed=641, extra_pages=2)
    mods = dict(causal=True, window=window)
    o, lse = _paged_vec_run(d, mods, 128) if vec else _paged_run(d, mods, 128)
    o_ref, l_ref = _paged_ref(d, mods)
    _cmp_packed(o, lse, o_ref, l_ref, TOL_O_FP8, f"fp8 window {window} vec={vec}")


# ----------------------------------------------------------------------------- query range
def _scaled_queries(d, how):
    """bf16 queries far from N(0,1) and the softmax scale that keeps the
    logits where they were: every element times 40 or 1e-3, or one element
    per row times 200 (a row whose maximum dwarfs the rest)."""
    q = d["q"].float()
    base = 1.0 / math.sqrt(q.shape[-1])
    if how == "mixed":
        q[..., 7] *= 200.0
        return q.to(torch.bfloat16), base / 20.0
    return (q * how).to(torch.bfloat16), base / how


@pytest.mark.parametrize("how", [40.0, 1e-3, "mixed"])
@pytest.mark.parametrize("vec", [False, True])
@pytest.mark.parametrize("path", ["prefill", "decode"])
def test_fp8_cache_bf16_query_range(path, vec, how):
    """The E4M3 split of bf16 queries takes a power-of-two scale per row, so
    queries whose magnitudes would overflow (x40: |16 q| > 448) or sink into
    E4M3 subnormals (x1e-3) with a fixed scale stay within the FP8
    tolerance, on the paged prefill and on the decode."""
    if path == "prefill":
        lq, lk, Hq, Hkv = [200, 77], [200, 300], 4, 4
    else:
        lq, lk, Hq, Hkv = [1, 1, 1], [300, 64, 700], 8, 2
    d = synth.make_paged(lq, lk, Hq, Hkv, 192, 128, page_size=64, seed=651, extra_pages=2)
    d["q"], scale = _scaled_queries(d, how)
    mods = dict(causal=True, scale=scale)
    o, lse = _paged_vec_run(d, mods, 128) if vec else _paged_run(d, mods, 128)
    o_ref, l_ref = _paged_ref(d, mods)
    _cmp_packed(o, lse, o_ref, l_ref, TOL_O_FP8, f"query range {how} {path} vec={vec}")


# ----------------------------------------------------------------------------- soft-cap saturation
@pytest.mark.parametrize("qscale", [30.0, 500.0])
@pytest.mark.parametrize("D", [64, 128])
def test_softcap_saturation(D, qscale):
    """Soft-cap where tanh saturates: queries scaled so that |logit| / cap
    reaches ~10 (x30) or ~100 (x500), past the point where the kernel's
    2^(2u log2 e) overflows to +inf or underflows to 0; the capped logits
    must come out at +-cap, alone and with ALiBi and a causal mask."""
    d = synth.make_dense(1, 300, 300, 2, 2, D, D, seed=661 + D)
    d["q"] = (d["q"].float() * qscale).to(torch.bfloat16)
    for mods in (dict(softcap=5.0), dict(softcap=5.0, alibi_slope=0.25, causal=True)):
        o, lse = _dense_run(d, mods, D)
        o_ref, l_ref = oracle.attention_dense(f64(d["q"]), f64(d["k"]), f64(d["v"]), dict(mods))
        compare(o.permute(0, 2, 1, 3), lse, o_ref.transpose(0, 2, 1, 3), l_ref, TOL_O_BF16,
                what=f"softcap saturation D{D} x{qscale} {sorted(mods)}")


# ----------------------------------------------------------------------------- launch stream
def test_calls_follow_the_current_stream():
    """The binding launches on torch's current stream (read as a raw handle)
    or on an explicit stream: queued behind a slow producer of Q on a side
    stream (default priority), the result is the oracle's only if the
    attention kernel ran after the producer on that same stream."""
    d = synth.make_dense(1, 256, 256, 2, 2, 128, 128, seed=671)
    k, v = d["k"].to(DEV), d["v"].to(DEV)
    o_ref, l_ref = oracle.attention_dense(f64(d["q"]), f64(d["k"]), f64(d["v"]), {})
    side = torch.cuda.Stream()
    for how in ("current", "explicit"):
        q = torch.zeros_like(d["q"], device=DEV)
        o = torch.full((1, 256, 2, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((1, 2, 256), float("nan"), dtype=torch.float32, device=DEV)
        big = torch.randn(4096, 4096, device=DEV)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            for _ in range(8):          # keep the side stream busy before Q is written
                big = big @ big / 64.0
            q.copy_(d["q"].to(DEV, non_blocking=True))
            if how == "current":
                fa.fa_fwd_dense(q, k, v, o, lse)
        if how == "explicit":
            fa.fa_fwd_dense(q, k, v, o, lse, stream=side)
        side.synchronize()
        compare(o.permute(0, 2, 1, 3), lse, o_ref.transpose(0, 2, 1, 3), l_ref, TOL_O_BF16, what=f"stream {how}")


# ----------------------------------------------------------------------------- seeded sweep
# ----------------------------------------------------------------------------- FP8 pages with score mods
FP8_MODS = {
    "alibi_causal": dict(causal=True, alibi_slope=0.0625),
    "softcap": dict(softcap=20.0),
    "alibi_softcap_causal": dict(causal=True, alibi_slope=0.0625, softcap=20.0),
    "softcap_window": dict(window=(90, 5), softcap=15.0),
    "bmask_causal": dict(causal=True, bmask=True),
    "bmask_alibi": dict(alibi_slope=0.125, bmask=True),
}


def _fp8_mods(name, d, seed):
    """The named mods for make_paged() data d; a block mask of 128 x 64
    tiles (active with probability 0.5) where asked."""
    m = dict(FP8_MODS[name])
    if m.pop("bmask", False):
        Hq = d["q"].shape[1]
        B = len(d["lengths_k"])
        nqb = max(1, math.ceil(max(d["lengths_q"]) / 128))
        nkb = max(1, math.ceil(max(d["lengths_k"]) / 64))
        m["block_mask"] = synth.bernoulli_block_mask(B * Hq, nqb, nkb, 0.5, seed=seed).to(DEV)
        m["mask_block"] = (128, 64)
    return m


def _fp8_ref(d, m, q8=False):
    kw = dict(q_descale=float(d["q_descale"])) if q8 else {}
    return oracle.attention_paged(f64(d["q"]), f64(d["k_cache"]), f64(d["v_cache"]), d["cu_q"], d["seqlen_k"],
                                  d["block_table"], _oracle_mods(m), float(d["k_descale"]), float(d["v_descale"]),
                                  **kw)


@pytest.mark.parametrize("name", sorted(FP8_MODS))
@pytest.mark.parametrize("shape", sorted(VEC_CASES))
def test_paged_fp8_score_mods(shape, name):
    """ALiBi, soft-cap, windows and block masks on FP8 head-major pages: the
    prefill kernel's mods variant (prefill, chunked) and the decode kernel's
    (one and two row blocks), against the oracle on the dequantised cache."""
    lq, lk, Hq, Hkv, Dqk, _ = VEC_CASES[shape]
    d = synth.make_paged(lq, lk, Hq, Hkv, Dqk, 128, page_size=64, seed=261 + len(name), extra_pages=3)
    m = _fp8_mods(name, d, seed=271)
    o, lse = _paged_run(d, m, 128)
    o_ref, l_ref = _fp8_ref(d, m)
    _cmp_packed(o, lse, o_ref, l_ref, TOL_O_FP8, f"fp8 mods {shape} {name}")


@pytest.mark.parametrize("name", ["alibi_softcap_causal", "bmask_causal"])
@pytest.mark.parametrize("shape", sorted(VEC_CASES))
def test_paged_fp8_score_mods_variants(shape, name):
    """The same mods through every other instantiation: vectorised pages
    (bitwise the head-major result), E4M3 queries (oracle, and bitwise
    across page formats), and D_qk = D_v = 192 (oracle, and vectorised)."""
    lq, lk, Hq, Hkv, Dqk, _ = VEC_CASES[shape]
    d = synth.make_paged(lq, lk, Hq, Hkv, Dqk, 128, page_size=16, seed=281, extra_pages=3)
    m = _fp8_mods(name, d, seed=283)
    o, lse = _paged_run(d, m, 128)
    o2, l2 = _paged_vec_run(d, m, 128)
    assert torch.equal(o, o2) and torch.equal(lse, l2), f"vec {shape} {name}"
    d8 = synth.make_paged(lq, lk, Hq, Hkv, Dqk, 128, page_size=16, seed=285, extra_pages=3, q_dtype="fp8")
    o, lse = _paged_q8_run(d8, m, 128)
    o_ref, l_ref = _fp8_ref(d8, m, q8=True)
    _cmp_packed(o, lse, o_ref, l_ref, TOL_O_FP8, f"q8 mods {shape} {name}")
    o2, l2 = _paged_q8_run(d8, m, 128, vec=True)
    assert torch.equal(o, o2) and torch.equal(lse, l2), f"q8 vec {shape} {name}"
    d9 = synth.make_paged(lq, lk, Hq, Hkv, 192, 192, page_size=16, seed=287, extra_pages=3)
    o, lse = _paged_run(d9, m, 192)
    o_ref, l_ref = _fp8_ref(d9, m)
    _cmp_packed(o, lse, o_ref, l_ref, TOL_O_FP8, f"v192 mods {shape} {name}")
    o2, l2 = _paged_vec_run(d9, m, 192)
    assert torch.equal(o, o2) and torch.equal(lse, l2), f"v192 vec {shape} {name}"


def _paged_sweep_case(i):
    """Seeded paged call: lengths (prefill, chunked or decode rows), page size,
    head dims, GQA, query type, page format, mods and block mask, all drawn
    from the exported paged surface."""
    g = torch.Generator().manual_seed(9000 + i)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=g))
    B = ri(1, 5)
    shape = ("prefill", "chunked", "decode")[ri(0, 2)]
    lk = [ri(0, 700) for _ in range(B)]
    if shape == "prefill":
        lq = list(lk)
    elif shape == "chunked":
        lq = [min(n, ri(0, 150)) for n in lk]
    else:
        lq = [ri(0, 2) if n > 0 else 0 for n in lk]
    Dqk, Dv = ((192, 128), (128, 128), (192, 192))[ri(0, 2)]
    Hkv = ri(1, 2)
    Hq = Hkv * (1, 2, 8)[ri(0, 2)]
    vec = ri(0, 1) == 1
    ps = (16, 64, 256)[ri(0, 2)] if vec else (1, 8, 16, 64, 256)[ri(0, 4)]
    q8 = ri(0, 2) == 0
    kind = ri(0, 6)
    mods = [dict(causal=True), dict(), dict(window=(ri(0, 200), ri(0, 20))), dict(causal=True, alibi_slope=0.0625),
            dict(softcap=15.0), dict(causal=True, softcap=30.0, alibi_slope=0.03), dict(causal=True, bmask=True)][kind]
    return lq, lk, Hq, Hkv, Dqk, Dv, ps, vec, q8, mods


@pytest.mark.parametrize("i", range(24))
def test_seeded_paged_sweep(i):
    """FP8 caches over the whole paged surface against the oracle on the
    dequantised cache (NaN-poisoned unused pages and page tails)."""
    lq, lk, Hq, Hkv, Dqk, Dv, ps, vec, q8, mods = _paged_sweep_case(i)
    if sum(lq) == 0:
        lq[0] = 1 if lk[0] > 0 else 0
    d = synth.make_paged(lq, lk, Hq, Hkv, Dqk, Dv, page_size=ps, seed=9100 + i, extra_pages=3,
                         q_dtype="fp8" if q8 else "bf16")
    m = dict(mods)
    if m.pop("bmask", False):
        nqb = max(1, math.ceil(max(lq) / 128))
        nkb = max(1, math.ceil(max(lk) / 64))
        m["block_mask"] = synth.bernoulli_block_mask(len(lk) * Hq, nqb, nkb, 0.6, seed=9200 + i).to(DEV)
        m["mask_block"] = (128, 64)
    what = f"paged sweep {i}: lq {lq} lk {lk} Hq {Hq} Hkv {Hkv} D {Dqk}/{Dv} ps {ps} vec {vec} q8 {q8} {mods}"
    if q8:
        o, lse = _paged_q8_run(d, m, Dv, vec=vec)
    elif vec:
        o, lse = _paged_vec_run(d, m, Dv)
    else:
        o, lse = _paged_run(d, m, Dv)
    o_ref, l_ref = _fp8_ref(d, m, q8=q8)
    _cmp_packed(o, lse, o_ref, l_ref, TOL_O_FP8, what)


def _sweep_case(i):
    """Case i of the sweep: seeded lengths (zero, short, tile-straddling),
    head dims, GQA ratio and mods, chosen by a generator of its own."""
    g = torch.Generator().manual_seed(7000 + i)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=g))
    B = ri(1, 4)
    cross = ri(0, 1) == 1
    lq = [ri(0, 260) for _ in range(B)]
    lk = [ri(0, 300) if cross else n for n in lq]
    if B > 1 and ri(0, 2) == 0:
        z = ri(0, B - 1)
        lq[z] = 0
        if not cross:
            lk[z] = 0
    D = (64, 128)[ri(0, 1)]
    Hkv = ri(1, 2)
    Hq = Hkv * (1, 2, 4)[ri(0, 2)]
    mods = {}
    if ri(0, 1):
        mods["causal"] = True
    kind = ri(0, 4)
    if kind == 1:
        mods["window"] = (ri(0, 80), ri(0, 40))
    elif kind == 2:
        mods["alibi_slope"] = 0.05 * ri(1, 6)
    elif kind == 3:
        mods["softcap"] = float(ri(2, 30))
    elif kind == 4:
        mods["alibi_slope"], mods["softcap"] = 0.1, 8.0
    return lq, lk, Hq, Hkv, D, mods


@pytest.mark.parametrize("i", range(24))
def test_seeded_varlen_sweep(i):
    """24 seeded small varlen problems across lengths, head dims, GQA and
    mods, each against the oracle."""
    lq, lk, Hq, Hkv, D, mods = _sweep_case(i)
    d = synth.make_varlen(lq, lk, Hq, Hkv, D, D, seed=7100 + i)
    o, lse = _varlen_run(d, mods, D)
    o_ref, l_ref = oracle.attention_varlen(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["cu_q"], d["cu_k"], dict(mods))
    _cmp_packed(o, lse, o_ref, l_ref, TOL_O_BF16, f"sweep {i}: lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} D={D} {mods}")


@pytest.mark.parametrize("vec", [False, True])
@pytest.mark.parametrize("small,big", [(16, 64), (32, 128)])
def test_paged_fp8_prefill_page_size_is_bitwise_invariant(small, big, vec):
    """Pages of fewer than 64 keys take per-row page lookups, pages of 64 or
    more one buffer descriptor per tile (two kernel variants): the same
    logical cache (same seed, so the same E4M3 bytes, queries and descales)
    in either page size gives the same bytes of O and LSE.  Lengths leave
    ragged tails; one query chunk is shorter than its keys."""
    lq, lk = [200, 64, 1, 130], [200, 300, 65, 130]
    runs = []
    for ps in (small, big):
        d = synth.make_paged(lq, lk, 8, 2, 192, 128, page_size=ps, seed=463, extra_pages=4)
        runs.append((_paged_vec_run if vec else _paged_run)(d, dict(causal=True), 128))
    (o1, l1), (o2, l2) = runs
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"pages {small} vs {big} vec={vec}"
