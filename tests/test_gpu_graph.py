"""Calls captured in a HIP graph (torch.cuda.CUDAGraph) replay the eager
results: the varlen prefill, the paged FP8 decode (with a caller workspace
and through fa_fwd_paged_noalloc, whose scratch is the library's static
array) and the varlen backward.  The library allocates nothing, copies
nothing between host and device and never synchronises inside a call, so
each call is a plain sequence of kernel launches on the caller's stream.

Each graph is replayed several times with eager work between the replays:
the outputs are refilled with NaN (every element must be rewritten), and
the inputs are switched between two seeded sets in place, so every replay
must equal, bitwise, the eager call on the inputs it sees at that moment."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _replays(graph, fill, switch, outs, expect):
    """Replay `graph` for the input sets in `expect` order, refilling the
    outputs with NaN and switching inputs eagerly before each replay."""
    for which in (0, 1, 0, 1):
        switch(which)
        fill()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("first", "second", "third", "fourth", "fifth"), outs, expect[which]):
            assert torch.equal(got, ref), f"replay on input set {which}: output {name} differs from the eager call"


def test_graph_varlen_prefill():
    import attention_fa_fwd_03_amd as fa
    lq = [300, 0, 1000, 517, 64]
    Hq, Hkv, D = 8, 2, 128
    sets = [synth.make_varlen(lq, lq, Hq, Hkv, D, D, seed=8101 + i) for i in range(2)]
    q, k, v = (sets[0][x].to(DEV).clone() for x in ("q", "k", "v"))
    cu = sets[0]["cu_q"].to(DEV)
    Tq = q.shape[0]
    o = torch.empty((Tq, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=DEV)
    mods = fa.Mods(causal=True)

    def switch(i):
        for t, x in ((q, "q"), (k, "k"), (v, "v")):
            t.copy_(sets[i][x].to(DEV))

    def fill():
        o.fill_(float("nan"))
        lse.fill_(float("nan"))

    expect = []
    for i in range(2):
        switch(i)
        fill()
        fa.fa_fwd_varlen(q, k, v, o, lse, cu, cu, max(lq), max(lq), mods)
        torch.cuda.synchronize()
        expect.append((o.clone(), lse.clone()))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_fwd_varlen(q, k, v, o, lse, cu, cu, max(lq), max(lq), mods)
    _replays(g, fill, switch, (o, lse), expect)


@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_paged_decode(noalloc):
    import attention_fa_fwd_03_amd as fa
    lk = [700, 64, 1500, 1, 333, 1024]
    lq = [1] * len(lk)
    Hq, Hkv, Dqk, Dv, ps = 64, 8, 192, 128, 64
    # unpoisoned caches: set 1's bytes are read through set 0's block table,
    # so every page both sets name must hold finite codes
    sets = [synth.make_paged(lq, lk, Hq, Hkv, Dqk, Dv, page_size=ps, seed=8201 + i, extra_pages=2, poison=False)
            for i in range(2)]
    q, kc, vc = (sets[0][x].to(DEV).clone() for x in ("q", "k_cache", "v_cache"))
    kd, vd = sets[0]["k_descale"].to(DEV).clone(), sets[0]["v_descale"].to(DEV).clone()
    cu, sk, bt = (sets[0][x].to(DEV) for x in ("cu_q", "seqlen_k", "block_table"))
    Tq, B = q.shape[0], len(lk)
    o = torch.empty((Tq, Hq, Dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=DEV)
    mods = fa.Mods(causal=True)
    ws = None
    if not noalloc:
        n = fa.fa_fwd_paged_workspace_size(B, Tq, 1, max(lk), Hq, Hkv, Dqk, Dv, ps, fa.FA_FP8_E4M3)
        assert n > 0
        ws = torch.empty(n, dtype=torch.uint8, device=DEV)

    def call():
        args = (q, kc, vc, o, lse, cu, sk, bt, 1, max(lk), kd, vd)
        if noalloc:
            fa.fa_fwd_paged_noalloc(*args, mods=mods)
        else:
            fa.fa_fwd_paged(*args, ws, mods)

    def switch(i):
        for t, x in ((q, "q"), (kc, "k_cache"), (vc, "v_cache"), (kd, "k_descale"), (vd, "v_descale")):
            t.copy_(sets[i][x].to(DEV))

    def fill():
        o.fill_(float("nan"))
        lse.fill_(float("nan"))

    expect = []
    for i in range(2):
        switch(i)
        fill()
        call()
        torch.cuda.synchronize()
        expect.append((o.clone(), lse.clone()))
        assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    _replays(g, fill, switch, (o, lse), expect)


def test_graph_varlen_backward():
    import attention_fa_fwd_03_amd as fa
    lq = [257, 0, 640, 99]
    Hq, Hkv, D = 4, 2, 128
    sets = []
    for i in range(2):
        d = synth.make_varlen(lq, lq, Hq, Hkv, D, D, seed=8301 + i)
        d["do"] = synth.randn_bf16(tuple(d["q"].shape), 8351 + i)
        sets.append(d)
    q, k, v, do = (sets[0][x].to(DEV).clone() for x in ("q", "k", "v", "do"))
    cu = sets[0]["cu_q"].to(DEV)
    Tq, Tk = q.shape[0], k.shape[0]
    mods = fa.Mods(causal=True)
    # the forward's O and LSE of each set are inputs of the backward
    fwd = []
    for i in range(2):
        qi, ki, vi = (sets[i][x].to(DEV) for x in ("q", "k", "v"))
        oi = torch.empty((Tq, Hq, D), dtype=torch.bfloat16, device=DEV)
        li = torch.empty((Hq, Tq), dtype=torch.float32, device=DEV)
        fa.fa_fwd_varlen(qi, ki, vi, oi, li, cu, cu, max(lq), max(lq), mods)
        fwd.append((oi, li))
    o, lse = fwd[0][0].clone(), fwd[0][1].clone()
    dq = torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_size(Tq, Hq), dtype=torch.uint8, device=DEV)

    def call():
        fa.fa_bwd_varlen(q, k, v, o, do, lse, dq, dk, dv, cu, cu, max(lq), max(lq), mods, workspace=ws)

    def switch(i):
        for t, x in ((q, "q"), (k, "k"), (v, "v"), (do, "do")):
            t.copy_(sets[i][x].to(DEV))
        o.copy_(fwd[i][0])
        lse.copy_(fwd[i][1])

    def fill():
        for t in (dq, dk, dv):
            t.fill_(float("nan"))

    expect = []
    for i in range(2):
        switch(i)
        fill()
        call()
        torch.cuda.synchronize()
        expect.append((dq.clone(), dk.clone(), dv.clone()))
    assert not torch.isnan(expect[0][0]).any()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    _replays(g, fill, switch, (dq, dk, dv), expect)
