"""fa_fwd_paged_noalloc (no workspace argument; decode scratch in the
library's static device array) against fa_fwd_paged with a caller
workspace: two calls in a row, the second smaller, each bitwise equal to
the workspace path and within the FP8 tolerance of the fp64 oracle."""
import pytest
import torch

import oracle
import synth
from tests.helpers import TOL_O_FP8, compare, f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _call(fa, d, Hq, Dqk, Dv, noalloc):
    q = d["q"].to(DEV)
    kc, vc = d["k_cache"].to(DEV), d["v_cache"].to(DEV)
    Tq = q.shape[0]
    B = len(d["lengths_k"])
    msq, msk = max(d["lengths_q"]), max(d["lengths_k"])
    o = torch.full((Tq, Hq, Dv), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((Hq, Tq), float("nan"), dtype=torch.float32, device=DEV)
    args = (q, kc, vc, o, lse, d["cu_q"].to(DEV), d["seqlen_k"].to(DEV), d["block_table"].to(DEV), msq, msk,
            d["k_descale"].to(DEV), d["v_descale"].to(DEV))
    if noalloc:
        fa.fa_fwd_paged_noalloc(*args, mods=fa.Mods(causal=True))
    else:
        n = fa.fa_fwd_paged_workspace_size(B, Tq, msq, msk, Hq, kc.shape[1], Dqk, Dv, kc.shape[2], fa.FA_FP8_E4M3)
        assert n > 0     # the decode path, the one that uses scratch
        ws = torch.empty(n, dtype=torch.uint8, device=DEV)
        fa.fa_fwd_paged(*args, ws, fa.Mods(causal=True))
    torch.cuda.synchronize()
    return o, lse


def test_noalloc_matches_the_workspace_path_twice():
    import attention_fa_fwd_03_amd as fa
    cases = [
        # larger call first: 16 sequences, contexts up to 8192, GQA 64/8, D 192/128
        ([1] * 16, synth.make_decode_lengths(777, n=16, lo=1024, hi=8192), 64, 8, 192, 128, 64),
        # then a smaller one: the array keeps the first call's bytes
        ([1, 1, 1], [300, 64, 700], 8, 2, 192, 128, 64),
    ]
    for n, (lq, lk, Hq, Hkv, Dqk, Dv, ps) in enumerate(cases):
        d = synth.make_paged(lq, lk, Hq, Hkv, Dqk, Dv, page_size=ps, seed=7001 + n, extra_pages=2)
        o1, l1 = _call(fa, d, Hq, Dqk, Dv, noalloc=True)
        o2, l2 = _call(fa, d, Hq, Dqk, Dv, noalloc=False)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"call {n}: outputs differ"
        if n == 1:
            o_ref, l_ref = oracle.attention_paged(f64(d["q"]), f64(d["k_cache"]), f64(d["v_cache"]), d["cu_q"],
                                                  d["seqlen_k"], d["block_table"], dict(causal=True),
                                                  float(d["k_descale"]), float(d["v_descale"]))
            compare(o1.permute(1, 0, 2), l1, o_ref.transpose(1, 0, 2), l_ref, TOL_O_FP8, what="noalloc")
