#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

Default workload: packed varlen causal prefill, H=16, D=128, bf16, 8
sequences with lengths uniform in [0, 4096] (one zero-length, several not
multiples of 64).  One step = one fa_fwd_varlen call over that batch (the
whole hot path: work enumeration, K/V addressing and staging, Q.K^T, masks,
online softmax, P.V, epilogue with O and LSE).  Inputs are resident in HBM
before timing starts.

The default line also carries the metric's second half and the other
workloads, each timed the same way (HIP events on the launch stream plus the
host clock):
  "decode":    the paged FP8 decode (64 sequences, contexts U[1024, 32768],
               GQA 64/8, D 192/128, pages of 64): HBM GB/s, roofline and
               the oracle's CPU baseline;
  "secondary": the paged FP8 prefill (4 x 2048, D 192/128) and the five
               flex workloads (B2 H16 S8192 D128: ALiBi, soft-cap, window
               (256, 0), Bernoulli block mask, block-causal);
  "latency":   per-call cost of the dense 1x128x2x64 forward (GPU time,
               wall time, host cost of the binding and of the C call).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--only]
                  [--flex alibi|softcap|window|bernoulli|block_causal|none|causal] [--page-size P]
                  [--layout head_major|vec] [--q-dtype bf16|fp8] [--dv 128|192]
                  [--no-cpu-baseline]
                  [--copy-calibration]
  python bench.py --config N --traffic-from FETCH_CSV WRITE_CSV

--config selects another workload for investigation (1 dense D64, 3 paged
FP8 prefill, 4 paged FP8 decode, 5 flex, 6 FP8 KV-cache write of the decode
cache, 7 backward pass of config 2's batch); the default line is config 2
(--only leaves out its decode, secondary and latency entries).  --layout vec
runs configs 3 and 4 on the vectorised 5-D page format (fa_fwd_paged_vec)
instead of head-major pages; --q-dtype fp8 gives them E4M3 queries with a
per-tensor descale (fa_fwd_paged_ex); --dv 192 runs them with value/output
width 192.
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s + fraction of MFMA peak; paged-decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
COPY_BYTES = 256 << 20        # calibration copy for the HBM byte counters
# dominant kernel of each kind, matched as a substring of the kernel name
# (the bf16 prefill is fa_prefill_bf16_kernel, the FP8-cache one fa_prefill_kernel)
DOMINANT = {"prefill": "fa_prefill_bf16_kernel", "prefill_fp8": "fa_prefill_kernel", "decode": "fa_decode_kernel",
            "kvwrite": "fa_kv_write_kernel", "backward": "fa_bwd_dkdv"}
KERNEL_SOURCES = {
    "prefill": ["attention_fa_fwd_03_amd/csrc/fa_prefill_bf16.hip", "attention_fa_fwd_03_amd/csrc/fa_prefill_common.h",
                "attention_fa_fwd_03_amd/csrc/fa_device.h", "attention_fa_fwd_03_amd/csrc/fa_kernels.h"],
    "prefill_fp8": ["attention_fa_fwd_03_amd/csrc/fa_prefill.hip", "attention_fa_fwd_03_amd/csrc/fa_prefill_common.h",
                    "attention_fa_fwd_03_amd/csrc/fa_device.h", "attention_fa_fwd_03_amd/csrc/fa_kernels.h"],
    "decode": ["attention_fa_fwd_03_amd/csrc/fa_decode.hip", "attention_fa_fwd_03_amd/csrc/fa_device.h",
               "attention_fa_fwd_03_amd/csrc/fa_kernels.h"],
    "kvwrite": ["attention_fa_fwd_03_amd/csrc/fa_kvcache.hip", "attention_fa_fwd_03_amd/csrc/fa_device.h",
                "attention_fa_fwd_03_amd/csrc/fa_kernels.h"],
    "backward": ["attention_fa_fwd_03_amd/csrc/fa_backward.hip", "attention_fa_fwd_03_amd/csrc/fa_prefill_common.h",
                 "attention_fa_fwd_03_amd/csrc/fa_device.h", "attention_fa_fwd_03_amd/csrc/fa_kernels.h"],
}


def kernel_sha(kind: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_key: str, kind: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    the kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    e = tab.get(workload_key)
    if not e or e.get("kernel_sha") != kernel_sha(kind):
        return None
    return e["hbm_bytes_per_launch"]


def traffic_from_counters(fetch_csv: str, write_csv: str, key: str, kind: str) -> dict:
    """Turn two rocprofv3 --pmc CSVs (FETCH_SIZE run, WRITE_SIZE run; both
    with --copy-calibration) into HBM bytes per launch of the dominant kernel
    and record them in profiles/traffic.json under `key`.

    Each counter is scaled by what it reads for the calibration copy
    (COPY_BYTES read and COPY_BYTES written by the runtime's copy kernel), so
    the result does not depend on the counters' unit."""
    import csv

    def per_dispatch(path, counter):
        vals, copies = [], []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                if DOMINANT[kind] in r["Kernel_Name"]:
                    vals.append(v)
                elif "rocclr" in r["Kernel_Name"] and "copy" in r["Kernel_Name"].lower():
                    copies.append(v)
        if not vals or not copies:
            raise SystemExit(f"{path}: no {counter} rows for {DOMINANT[kind]} and the calibration copy")
        return sum(vals) / len(vals), max(copies), len(vals)

    fetch, copy_fetch, n_f = per_dispatch(fetch_csv, "FETCH_SIZE")
    write, copy_write, n_w = per_dispatch(write_csv, "WRITE_SIZE")
    sf, sw = COPY_BYTES / copy_fetch, COPY_BYTES / copy_write
    entry = dict(kernel=DOMINANT[kind], kernel_sha=kernel_sha(kind), dispatches=[n_f, n_w],
                 fetch_size_per_dispatch=round(fetch, 1), write_size_per_dispatch=round(write, 1),
                 copy_fetch_size=round(copy_fetch, 1), copy_write_size=round(copy_write, 1),
                 bytes_per_fetch_unit=round(sf, 3), bytes_per_write_unit=round(sw, 3),
                 hbm_bytes_per_launch=round(fetch * sf + write * sw))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    tab = {}
    if os.path.exists(path):
        with open(path) as f:
            tab = json.load(f)
    tab[key] = entry
    with open(path, "w") as f:
        json.dump(tab, f, indent=1, sort_keys=True)
        f.write("\n")
    return entry


def build_workload(cfg: int, flex: str, torch, synth, fa, page_size: int = 64, layout: str = "head_major",
                   q_dtype: str = "bf16", dv: int = 128):
    """Returns (name, run_fn, work dict, oracle sample fn)."""
    dev = "cuda"
    if cfg == 1:
        d = synth.make_dense(1, 128, 128, 2, 2, 64, 64, seed=synth.seed_for(1), device=dev)
        o = torch.empty(1, 128, 2, 64, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(1, 2, 128, dtype=torch.float32, device=dev)
        mods = fa.Mods(scale=1 / 8)
        flops = 1 * 2 * 128 * 128 * (2 * 64 + 2 * 64)
        run = lambda: fa.fa_fwd_dense(d["q"], d["k"], d["v"], o, lse, mods)
        name = "dense non-causal B1 H2 S128 D64 bf16"
        return name, run, dict(flops=flops, kind="prefill", bound="mfma"), {"B": 1, "H": 2, "S": 128, "D": 64}, None
    if cfg == 2:
        lens = synth.varlen_lengths(synth.seed_for(2))
        d = synth.make_varlen(lens, lens, 16, 16, 128, 128, seed=synth.seed_for(2), device=dev)
        T = sum(lens)
        o = torch.empty(T, 16, 128, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(16, T, dtype=torch.float32, device=dev)
        mods = fa.Mods(causal=True)
        flops = sum(16 * L * (L + 1) // 2 * (2 * 128 + 2 * 128) for L in lens)
        run = lambda: fa.fa_fwd_varlen(d["q"], d["k"], d["v"], o, lse, d["cu_q"], d["cu_k"], max(lens), max(lens), mods)
        name = "varlen causal prefill H16 D128 bf16, 8 seqs U[0,4096]"

        def sample():
            import oracle
            qh, kh, vh = (d[x].float().cpu().double().numpy() for x in ("q", "k", "v"))
            cu = d["cu_q"].cpu().numpy()
            dt, reps = _timed_reps(lambda: oracle.attention_varlen(qh, kh, vh, cu, cu, dict(causal=True),
                                                                   workers=_cores()))
            return dict(seconds=dt, work=flops * reps,
                        sample=f"the whole batch (all 8 sequences, all 16 heads), {reps} passes")
        return name, run, dict(flops=flops, kind="prefill", bound="mfma"), \
            {"seqlens": lens, "total_tokens": T, "H": 16, "D": 128, "causal": True}, sample
    if cfg == 3:
        L = [2048] * 4
        d = synth.make_paged(L, L, 16, 16, 192, dv, page_size=64, seed=synth.seed_for(3), device=dev,
                             q_dtype=q_dtype)
        if layout == "vec":
            d = synth.to_vectorized(d)
        fn = fa.fa_fwd_paged_vec if layout == "vec" else fa.fa_fwd_paged
        o = torch.empty(8192, 16, dv, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(16, 8192, dtype=torch.float32, device=dev)
        mods = fa.Mods(causal=True)
        flops = 64 * 2048 * 2049 // 2 * (2 * 192 + 2 * dv)
        run = lambda: fn(d["q"], d["k_cache"], d["v_cache"], o, lse, d["cu_q"], d["seqlen_k"],
                         d["block_table"], 2048, 2048, d["k_descale"], d["v_descale"], None, mods,
                         q_descale=d["q_descale"])
        name = f"paged FP8 causal prefill 4x2048 H16 Dqk192 Dv{dv} page64" + (" vectorised" if layout == "vec" else "") \
            + (" fp8-q" if q_dtype == "fp8" else "")
        return name, run, dict(flops=flops, kind="prefill_fp8", bound="mfma"), \
            {"B": 4, "S": 2048, "H": 16, "d_qk": 192, "d_v": dv, "page_size": 64, "layout": layout,
             "q_dtype": q_dtype}, None
    if cfg == 4:
        lk = synth.make_decode_lengths(synth.seed_for(4))
        lq = [1] * 64
        ps = page_size
        d = synth.make_paged(lq, lk, 64, 8, 192, dv, page_size=ps, seed=synth.seed_for(4), device=dev,
                             q_dtype=q_dtype)
        if layout == "vec":
            d = synth.to_vectorized(d)
            torch.cuda.empty_cache()
        fn = fa.fa_fwd_paged_vec if layout == "vec" else fa.fa_fwd_paged
        o = torch.empty(64, 64, dv, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(64, 64, dtype=torch.float32, device=dev)
        n = fa.fa_fwd_paged_workspace_size(64, 64, 1, max(lk), 64, 8, 192, dv, ps)
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
        mods = fa.Mods(causal=True)
        kv_bytes = sum(lk) * 8 * (192 + dv)
        io_bytes = 64 * 64 * 192 * (1 if q_dtype == "fp8" else 2) + 64 * 64 * dv * 2 + 64 * 64 * 4 + sum(math.ceil(x / ps) for x in lk) * 4
        flops = sum(lk) * 64 * (2 * 192 + 2 * dv)
        run = lambda: fn(d["q"], d["k_cache"], d["v_cache"], o, lse, d["cu_q"], d["seqlen_k"],
                         d["block_table"], 1, max(lk), d["k_descale"], d["v_descale"], ws, mods,
                         q_descale=d["q_descale"])
        name = f"paged FP8 decode 64 seqs ctx U[1024,32768] GQA 64/8 Dqk192 Dv{dv} page{ps}" + \
            (" vectorised" if layout == "vec" else "") + (" fp8-q" if q_dtype == "fp8" else "")

        def sample():
            import oracle
            n_seq = 8   # the first 8 sequences; only their pages are copied to the host
            bt = d["block_table"][:n_seq]
            npg = [math.ceil(x / ps) for x in lk[:n_seq]]
            ids = torch.cat([bt[b, :npg[b]] for b in range(n_seq)]).long()
            kc = d["k_cache"].index_select(0, ids).cpu().numpy()
            vc = d["v_cache"].index_select(0, ids).cpu().numpy()
            cbt = torch.zeros(n_seq, max(npg), dtype=torch.int64)
            pos = 0
            for b in range(n_seq):
                cbt[b, :npg[b]] = torch.arange(pos, pos + npg[b])
                pos += npg[b]
            qh = d["q"][:n_seq].cpu().numpy() if q_dtype == "fp8" else d["q"][:n_seq].float().cpu().double().numpy()
            qd = float(d["q_descale"]) if q_dtype == "fp8" else None
            cu = torch.arange(n_seq + 1).numpy()
            kd, vd = float(d["k_descale"]), float(d["v_descale"])
            dt, reps = _timed_reps(lambda: oracle.attention_paged(qh, kc, vc, cu, lk[:n_seq], cbt.numpy(),
                                                                  dict(causal=True), kd, vd, workers=_cores(),
                                                                  layout="vectorized" if layout == "vec"
                                                                  else "head_major", q_descale=qd))
            sbytes = sum(lk[:n_seq]) * 8 * (192 + dv)
            return dict(seconds=dt, work=sbytes * reps,
                        sample=f"sequences 0-{n_seq - 1} ({sum(lk[:n_seq])} cached tokens, all heads), {reps} passes")
        return name, run, dict(flops=flops, bytes=kv_bytes + io_bytes, kind="decode", bound="hbm"), \
            {"B": 64, "ctx_total": sum(lk), "Hq": 64, "Hkv": 8, "d_v": dv, "page_size": ps, "layout": layout,
             "q_dtype": q_dtype}, sample
    if cfg == 5:
        B, H, S, D = 2, 16, 8192, 128
        d = synth.make_dense(B, S, S, H, H, D, D, seed=synth.seed_for(5), device=dev)
        o = torch.empty(B, S, H, D, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(B, H, S, dtype=torch.float32, device=dev)
        bound = "mfma"
        if flex == "alibi":
            mods, pairs = fa.Mods(alibi_slope=0.0625), S * S
        elif flex == "softcap":
            mods, pairs = fa.Mods(softcap=20.0), S * S
        elif flex == "window":
            mods, pairs = fa.Mods(window=(256, 0)), sum(min(i, 256) + 1 for i in range(S))
            bound = "hbm"
        elif flex == "none":
            mods, pairs = fa.Mods(), S * S
        elif flex == "causal":
            mods, pairs = fa.Mods(causal=True), S * (S + 1) // 2
        elif flex == "bernoulli":
            bm = synth.bernoulli_block_mask(B * H, 64, 64, 0.5, seed=synth.seed_for(5, 3)).to(dev)
            mods, pairs = fa.Mods(block_mask=bm), None
            act = int(bm.sum())
        else:
            bm = synth.block_causal_mask(B * H, 64, 64).to(dev)
            mods, pairs = fa.Mods(block_mask=bm), None
            act = int(bm.sum())
        if pairs is None:
            flops = act * 128 * 128 * (2 * D + 2 * D)
        else:
            flops = B * H * pairs * (2 * D + 2 * D)
        byts = 4 * B * S * H * D * 2 + B * H * S * 4
        run = lambda: fa.fa_fwd_dense(d["q"], d["k"], d["v"], o, lse, mods)
        name = f"flex {flex} B2 H16 S8192 D128 bf16"
        return name, run, dict(flops=flops, bytes=byts, kind="prefill", bound=bound), \
            {"B": B, "H": H, "S": S, "D": D, "mod": flex}, None
    if cfg == 7:
        # backward of the default batch: the forward runs once beforehand for
        # O and LSE; a step is one fa_bwd_varlen call (dQ with Delta, then dK/dV)
        lens = synth.varlen_lengths(synth.seed_for(2))
        d = synth.make_varlen(lens, lens, 16, 16, 128, 128, seed=synth.seed_for(2), device=dev)
        T = sum(lens)
        o = torch.empty(T, 16, 128, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(16, T, dtype=torch.float32, device=dev)
        mods = fa.Mods(causal=True)
        fa.fa_fwd_varlen(d["q"], d["k"], d["v"], o, lse, d["cu_q"], d["cu_k"], max(lens), max(lens), mods)
        dout = synth.randn_bf16((T, 16, 128), synth.seed_for(7), device=dev)
        dq, dk, dvv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
        ws = torch.empty(fa.fa_bwd_workspace_size(T, 16), dtype=torch.uint8, device=dev)
        # algorithmic: the five products of the backward (S, dP, dV, dK, dQ),
        # 2.5 times the forward's two, over the visible pairs
        flops = sum(16 * L * (L + 1) // 2 * 5 * 2 * 128 for L in lens)
        run = lambda: fa.fa_bwd_varlen(d["q"], d["k"], d["v"], o, dout, lse, dq, dk, dvv, d["cu_q"], d["cu_k"],
                                       max(lens), max(lens), mods, workspace=ws)
        name = "varlen causal backward H16 D128 bf16, 8 seqs U[0,4096]"
        return name, run, dict(flops=flops, kind="backward", bound="mfma"), \
            {"seqlens": lens, "total_tokens": T, "H": 16, "D": 128, "causal": True}, None
    if cfg == 6:
        # every token of the decode cache (64 sequences, contexts U[1024, 32768],
        # 8 kv-heads, 192/128) quantised from bf16 with per-tensor amax
        # descales and written into pages of page_size (shuffled)
        lk = synth.make_decode_lengths(synth.seed_for(4))
        T, Hkv, ps = sum(lk), 8, page_size
        g = torch.Generator(device=dev).manual_seed(synth.seed_for(6))
        k = torch.randn((T, Hkv, 192), generator=g, device=dev).to(torch.bfloat16)
        v = torch.randn((T, Hkv, dv), generator=g, device=dev).to(torch.bfloat16)
        P = (T + ps - 1) // ps
        slots = torch.randperm(P, generator=g, device=dev).repeat_interleave(ps)[:T] * ps + \
            torch.arange(T, device=dev) % ps
        if layout == "vec":
            kc = torch.empty((P, Hkv, 12, ps, 16), dtype=torch.uint8, device=dev)
            vc = torch.empty((P, Hkv, ps // 16, dv, 16), dtype=torch.uint8, device=dev)
        else:
            kc = torch.empty((P, Hkv, ps, 192), dtype=torch.uint8, device=dev)
            vc = torch.empty((P, Hkv, ps, dv), dtype=torch.uint8, device=dev)
        kd = torch.empty(1, dtype=torch.float32, device=dev)
        vd = torch.empty(1, dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_kv_cache_write_fp8_workspace_size(T, Hkv, 192, dv), dtype=torch.uint8, device=dev)
        run = lambda: fa.fa_kv_cache_write_fp8(k, v, slots, kc, vc, kd, vd, workspace=ws)
        # the per-tensor maximum must see every row before any code is
        # written: two reads of the bf16 rows, one write of the codes
        byts = 2 * T * Hkv * (192 + dv) * 2 + T * Hkv * (192 + dv) + T * 8
        name = f"FP8 KV-cache write {T} tokens Hkv8 D192/{dv} page{ps} amax descales" + \
            (" vectorised" if layout == "vec" else "")
        return name, run, dict(flops=0, bytes=byts, kind="kvwrite", bound="hbm"), \
            {"T": T, "Hkv": Hkv, "d_qk": 192, "d_v": dv, "page_size": ps, "layout": layout}, None
    raise SystemExit(f"unknown config {cfg}")


def _timed_reps(fn, min_seconds: float = 10.0, max_reps: int = 30):
    """Run the oracle sample until it has taken at least min_seconds (a
    bounded sample of about 10 s of CPU work).  Returns (seconds, passes)."""
    t0 = time.perf_counter()
    reps = 0
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        fn()
        reps += 1
    return time.perf_counter() - t0, reps


def _affinity() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _cores() -> int:
    """Oracle worker threads: the affinity cores, at most 16 (a host's CPU
    share for one GPU)."""
    return max(1, min(_affinity(), 16))


def _key(cfg, flex="alibi", page_size=64, layout="head_major", q_dtype="bf16", dv=128):
    key = f"config{cfg}" + (f"_{flex}" if cfg == 5 else "")
    if cfg == 4 and page_size != 64:
        key += f"_ps{page_size}"
    if cfg == 6:
        key += f"_ps{page_size}" + ("_vec" if layout == "vec" else "") + (f"_dv{dv}" if dv != 128 else "")
    if cfg in (3, 4) and layout == "vec":
        key += "_vec"
    if cfg in (3, 4) and q_dtype == "fp8":
        key += "_q8"
    if cfg in (3, 4) and dv != 128:
        key += f"_dv{dv}"
    return key


def measure(torch, synth, fa, cfg, flex="alibi", steps=30, warmup=10, page_size=64, layout="head_major",
            q_dtype="bf16", dv=128, cpu=True):
    """One workload: W untimed steps, then K steps timed by the host clock
    and by HIP events on the launch stream (torch's current stream, where
    the binding enqueues).  Returns a dict with value/unit/roofline/config
    and, for workloads that have one and when asked, the oracle's cpu_baseline."""
    name, run, work, cfg_extra, sample = build_workload(cfg, flex, torch, synth, fa, page_size, layout, q_dtype, dv)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_s = ev0.elapsed_time(ev1) * 1e-3 / steps
    tflops = work["flops"] * steps / wall / 1e12
    if work["bound"] == "hbm":
        value, unit = work["bytes"] * steps / wall / 1e9, "GB/s"
        achieved = work["bytes"] / per_launch_s / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 2), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4))
    else:
        value, unit = tflops, "TFLOP/s"
        achieved = work["flops"] / per_launch_s / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 4))
    roof["traffic"] = measured_traffic(_key(cfg, flex, page_size, layout, q_dtype, dv), work["kind"])
    roof["kernel_ms"] = round(per_launch_s * 1e3, 4)
    out = dict(value=round(value, 3), unit=unit, ms_per_step=round(wall * 1e3 / steps, 4),
               config={"workload": name, **cfg_extra}, roofline=roof, cpu_baseline=None,
               dtype=("fp8-qkv/bf16" if q_dtype == "fp8" else "fp8-kv/bf16") if cfg in (3, 4)
               else ("bf16->fp8" if cfg == 6 else "bf16"))
    if work["bound"] == "hbm" and work["flops"]:
        out["config"]["tflops"] = round(tflops, 3)
    if sample is not None and cpu:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            r = sample()
        cval = r["work"] / r["seconds"] / (1e9 if work["bound"] == "hbm" else 1e12)
        out["cpu_baseline"] = dict(value=round(cval, 6), unit=unit, cores=_cores(), cores_available=_affinity(),
                                   kind="oracle", sample=r["sample"], seconds=round(r["seconds"], 2))
    return out


def call_latency(torch, synth, fa, calls=2000):
    """Per-call cost of the dense 1x128x2x64 forward (launch-bound: 8.4 MFLOP):
    GPU time of one launch (HIP events over many back-to-back launches),
    wall time per call with the queue kept busy, wall time of one call
    waited on, and the host side split into the Python binding's
    marshalling and the C call (validation and kernel launch), timed by
    calling the C entry point through ctypes with prepared arguments."""
    import ctypes
    from attention_fa_fwd_03_amd import binding as B
    d = synth.make_dense(1, 128, 128, 2, 2, 64, 64, seed=synth.seed_for(1), device="cuda")
    o = torch.empty(1, 128, 2, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, 2, 128, dtype=torch.float32, device="cuda")
    mods = fa.Mods(scale=1 / 8)
    run = lambda: fa.fa_fwd_dense(d["q"], d["k"], d["v"], o, lse, mods)
    for _ in range(50):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(calls):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_busy = (time.perf_counter() - t0) / calls
    gpu = ev0.elapsed_time(ev1) * 1e-3 / calls
    # one call waited on, repeatedly
    n1 = 200
    t0 = time.perf_counter()
    for _ in range(n1):
        run()
        torch.cuda.synchronize()
    wall_sync = (time.perf_counter() - t0) / n1
    # the C entry point alone (validation + launch), arguments prepared once
    cmods = mods.to_c()
    cm = ctypes.byref(cmods)
    sp = ctypes.c_void_p(stream.cuda_stream)
    args = (d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), o.data_ptr(), lse.data_ptr(),
            1, 128, 128, 2, 2, 64, 64, cm, sp)
    t0 = time.perf_counter()
    for _ in range(calls):
        B.lib.fa_fwd_dense(*args)
    c_call = (time.perf_counter() - t0) / calls
    torch.cuda.synchronize()
    # an empty ctypes call into the library: the foreign-call floor
    t0 = time.perf_counter()
    for _ in range(calls):
        B.lib.fa_abi_version()
    ffi = (time.perf_counter() - t0) / calls
    us = lambda x: round(x * 1e6, 2)
    return dict(workload="dense non-causal B1 H2 S128 D64 bf16 (launch-bound)", unit="us per call",
                gpu_us=us(gpu), wall_us_queued=us(wall_busy), wall_us_synchronised=us(wall_sync),
                host_us_binding=us(max(wall_busy - c_call, 0.0)), host_us_c_call=us(c_call),
                host_us_ctypes_floor=us(ffi), calls=calls)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--flex", default="alibi")
    ap.add_argument("--page-size", type=int, default=64, help="decode config: cache page size (power of two)")
    ap.add_argument("--layout", choices=["head_major", "vec"], default="head_major",
                    help="paged configs: head-major or vectorised 5-D pages")
    ap.add_argument("--q-dtype", choices=["bf16", "fp8"], default="bf16",
                    help="paged configs: bf16 or E4M3 queries")
    ap.add_argument("--dv", type=int, choices=[128, 192], default=128, help="paged configs: value/output width")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true",
                    help="default config only: leave out the decode, secondary and latency entries")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 256 MiB device copy first (reference for HBM byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="record HBM bytes per launch from two rocprofv3 --pmc counter CSVs and exit")
    args = ap.parse_args()
    key = _key(args.config, args.flex, args.page_size, args.layout, args.q_dtype, args.dv)
    if args.traffic_from:
        kind = {3: "prefill_fp8", 4: "decode", 6: "kvwrite", 7: "backward"}.get(args.config, "prefill")
        print(json.dumps({key: traffic_from_counters(args.traffic_from[0], args.traffic_from[1], key, kind)}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(sequences and heads are independent units that would shard across GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import attention_fa_fwd_03_amd as fa

    torch.cuda.init()
    if args.copy_calibration:
        # reference for the HBM byte counters: one device-to-device copy of
        # COPY_BYTES through the HIP runtime's own copy kernel
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                       ctypes.c_void_p]
        a = torch.zeros(COPY_BYTES, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        rc = hip.hipMemcpyAsync(b.data_ptr(), a.data_ptr(), COPY_BYTES, 3,
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        if rc != 0:
            raise SystemExit(f"hipMemcpyAsync failed: {rc}")
        del a, b

    cpu = not args.no_cpu_baseline
    m = measure(torch, synth, fa, args.config, args.flex, args.steps, args.warmup, args.page_size, args.layout,
                args.q_dtype, args.dv, cpu=cpu)
    line = {
        "metric": METRIC,
        "value": m["value"],
        "unit": m["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m["dtype"],
        "data": "synthetic",
        "config": m["config"],
        "roofline": m["roofline"],
        "cpu_baseline": m["cpu_baseline"],
    }
    if args.config == 2 and not args.only:
        # the metric's second half: the paged FP8 decode's HBM GB/s (config 4),
        # timed the same way, with its own oracle baseline
        torch.cuda.empty_cache()
        dm = measure(torch, synth, fa, 4, steps=args.steps, warmup=args.warmup, cpu=cpu)
        line["decode"] = {"metric": "paged-decode HBM GB/s", **dm}
        torch.cuda.empty_cache()
        sec = []
        k2, w2 = min(args.steps, 20), min(args.warmup, 5)
        for cfg, flex in [(3, None), (5, "alibi"), (5, "softcap"), (5, "window"), (5, "bernoulli"),
                          (5, "block_causal")]:
            sm = measure(torch, synth, fa, cfg, flex or "alibi", k2, w2, cpu=False)
            sec.append({"workload": sm["config"]["workload"], "value": sm["value"], "unit": sm["unit"],
                        "dtype": sm["dtype"], "roofline": {k: sm["roofline"][k] for k in
                                                           ("bound", "achieved", "peak", "unit", "frac",
                                                            "traffic", "kernel_ms")}})
            torch.cuda.empty_cache()
        line["secondary"] = sec
        line["latency"] = call_latency(torch, synth, fa)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
