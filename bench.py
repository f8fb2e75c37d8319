#!/usr/bin/env python3
"""Benchmark of the paged GQA decode path on one MI355X.

One step = one astr_paged_decode call (split kernel + combine kernel) over one
batch of the decode microbench shape: B=32 requests, 1 query token each,
Hq=32, Hkv=8, head_dim=128, bf16, seq_len ~ U{200..2000}, a 2^17-slot pool
addressed through a random-permutation req_to_token (page size 1).

Caches are kept cold: the timed steps rotate over --sets independent input
sets (pools, tables, queries), so the bytes one step touches are gone from
the 256 MB Infinity Cache by the time that set comes round again.  Inputs
are resident in HBM before the timed region starts.

Prints one JSON line (stdout).  `value` is algorithmic HBM bytes of the whole
call (K + V + Q + O + index arrays + lse) per second, in GB/s.  `roofline`
is for the dominant kernel (the split kernel), timed live with HIP events that
the kernel's own dispatch stamps at its start and end (hipExtLaunchKernel).  `cpu_baseline`
times the fp64 CPU oracle on the same workload.  `prefill` reports the ragged
prefill kernel (B=8, prefix U{0..2048}, q_len U{1..512}) against the bf16
MFMA peak.  `append` times a decode step that first appends each request's new
token to the pools: the standalone append kernel followed by decode, against
the fused append + decode call.  `graph` times a 32-layer decode step made of
per-layer calls against the same step captured once and replayed as a graph.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "paged GQA decode µs/call + achieved HBM GB/s (% peak), B=32 seq 200-2000"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, AMD published peak
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, AMD published peak
ROOT = os.path.dirname(os.path.abspath(__file__))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_flops(inp):
    """4 * D * Hq per visible (query row, key) pair; causally masked pairs are not counted."""
    _, Hq, D = inp["q"].shape
    kv, qo = inp["kv_indptr"], inp["qo_indptr"]
    pairs = 0
    for b in range(len(kv) - 1):
        L = int(kv[b + 1] - kv[b])
        qb = int(qo[b + 1] - qo[b])
        c = L - qb
        pairs += qb * c + qb * (qb + 1) // 2
    return 4 * D * Hq * pairs


def cpu_baseline(inp, budget_s):
    import oracle
    from paged_gqa_decode_astr_amd import profiling
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        runs, t0 = 0, time.perf_counter()
        while True:
            out = oracle.paged_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                         inp["req_to_token_stride"], inp["kv_indptr"], inp["sm_scale"])
            runs += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    per = el / runs
    return out, {"value": profiling.decode_bytes(inp) / per / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                 "sample": f"fp64 NumPy oracle over one full decode_b32 batch (set 0, {B_str(inp)}), "
                           f"{runs} run(s) in {el:.1f} s, {per * 1e3:.1f} ms/call, BLAS limited to 1 thread; "
                           f"host has {len(os.sched_getaffinity(0))} cores"}


def graph_leg(args, dev, layers_per_step=32, batches=(1, 4, 8, 16, 32), steps=20):
    """Whole-step graph against eager calls: a decode step of `layers_per_step` layers (each with its own
    pools, queries and outputs; seq_len ~ U{200..2000}, Hq 32 / Hkv 8, D 128) run as per-layer
    astr_paged_decode calls from Python, and as one captured astr_decode_graph replayed per step."""
    import torch
    from paged_gqa_decode_astr_amd import _lib, tensors
    from paged_gqa_decode_astr_amd.workloads import build_paged_inputs

    res = []
    s = torch.cuda.Stream()
    for B in batches:
        log(f"[bench] graph leg B={B}")
        seq = np.random.default_rng(B).integers(200, 2001, size=B)
        inp = build_paged_inputs(seq, 32, 8, 128, 1 << 16, seed=7000 + B)
        layers = []
        for _ in range(layers_per_step):
            d = tensors.to_device(inp, dev)
            d["o"] = torch.empty(B, 32, 128, dtype=torch.bfloat16, device=dev)
            d["lse"] = torch.empty(B, 32, dtype=torch.float32, device=dev)
            layers.append(d)
        a0, keep = _lib.make_args(layers[0]["q"], layers[0]["k_pool"], layers[0]["v_pool"], layers[0]["req_to_token"],
                                  layers[0]["kv_indptr"], layers[0]["kv_indptr_host"], layers[0]["o"], sm_scale=1.0,
                                  req_to_token_stride=layers[0]["req_to_token_stride"])
        ns = _lib.astr_plan_decode(a0, 0).num_splits
        ws = tensors.decode_workspace(B, 32, 128, dev, max_splits=ns)
        s.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()

        def eager_step():
            for d in layers:
                tensors.run_decode(d, o=d["o"], lse=d["lse"], workspace=ws, num_splits=ns, stream=s)

        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            eager_step()
        torch.cuda.synchronize()
        t0.record(s)
        for _ in range(steps):
            eager_step()
        t1.record(s)
        torch.cuda.synchronize()
        eager_us = t0.elapsed_time(t1) / steps * 1e3
        g = _lib.DecodeGraph(layers, ws, num_splits=ns, stream=s)
        for _ in range(3):
            g.launch()
        torch.cuda.synchronize()
        t0.record(s)
        for _ in range(steps):
            g.launch()
        t1.record(s)
        torch.cuda.synchronize()
        graph_us = t0.elapsed_time(t1) / steps * 1e3
        g.close()
        res.append({"batch": B, "eager_us_per_step": round(eager_us, 1), "graph_us_per_step": round(graph_us, 1),
                    "speedup": round(eager_us / graph_us, 2)})
        del layers, ws
        torch.cuda.synchronize()
    return {"workload": f"decode step of {layers_per_step} layers, each its own pools; seq_len ~ U{{200..2000}}, "
                        "Hq 32 / Hkv 8, D 128; eager = per-layer astr_paged_decode calls from Python, graph = one "
                        "astr_decode_graph launch per step", "steps": steps, "by_batch": res}


def B_str(inp):
    return f"B={inp['q'].shape[0]}, {int(inp['kv_indptr'][-1])} keys"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4, help="independent input sets rotated to keep caches cold")
    ap.add_argument("--config", default="decode_b32", help="decode workload (tiny, decode_b32, long_b1, long_b4, ragged_b256)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle time budget (0 = skip)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-append", action="store_true", help="skip the KV append + decode leg")
    ap.add_argument("--no-graph", action="store_true", help="skip the whole-step graph leg")
    ap.add_argument("--no-warm", action="store_true", help="skip the warm-cache reference leg")
    ap.add_argument("--probe", action="store_true", help="also measure torch copy / row-gather bandwidth ceilings")
    ap.add_argument("--num-splits", type=int, default=0, help="decode work groups per kv head (0 = library plan)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (this path has no "
              "multi-GPU mode)", file=sys.stderr)
        return 2

    import torch
    from paged_gqa_decode_astr_amd import _lib, profiling, tensors
    from paged_gqa_decode_astr_amd.hip_events import HipEvent
    from paged_gqa_decode_astr_amd.workloads import CONFIGS, make_inputs

    _lib.load_library()
    dev = "cuda"
    cfg = CONFIGS[args.config]
    log(f"[bench] building {args.sets} input sets of {args.config}")
    sets = tensors.decode_sets(args.config, args.sets, dev, num_splits=args.num_splits)
    torch.cuda.synchronize()

    def step(k, events=None):
        tensors.decode_step(sets, k, num_splits=args.num_splits, timing_events=events)

    log(f"[bench] warmup {args.warmup}")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        step(k)
    stop.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    ms_per_step = ms_total / args.steps
    total_bytes = sum(profiling.decode_bytes(sets[k % len(sets)][0]) for k in range(args.steps))
    value = total_bytes / (ms_total * 1e-3) / 1e9

    # Per-kernel durations: start/end stamps taken by each kernel's own dispatch (hipExtLaunchKernel).
    log("[bench] per-kernel event timing")
    evs = [[HipEvent() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(k, evs[k])
    torch.cuda.synchronize()
    split_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    comb_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    split_bytes = sum(profiling.split_kernel_bytes(sets[k % len(sets)][0]) for k in range(args.steps))
    achieved = split_bytes / (split_ms.sum() * 1e-3) / 1e9
    plan = _lib.astr_plan_decode(_lib.make_args(
        sets[0][1]["q"], sets[0][1]["k_pool"], sets[0][1]["v_pool"], sets[0][1]["req_to_token"],
        sets[0][1]["kv_indptr"], sets[0][1]["kv_indptr_host"], sets[0][1]["o"], sm_scale=1.0,
        req_to_token_stride=sets[0][1]["req_to_token_stride"], num_splits=args.num_splits)[0], 0)

    B, Hq, D = sets[0][0]["q"].shape
    G = Hq // cfg.num_kv_heads
    kernel_name = f"decode_split_kernel<{D},{G}>"
    traffic = profiling.read_traffic(args.config)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.config}: {cfg.description}; B={B} Hq={Hq} Hkv={cfg.num_kv_heads} D={D}, "
                               f"pool 2^{int(math.log2(cfg.num_slots))} slots, page_size 1",
                   "batch": B, "cache": f"cold: {args.sets} rotating input sets",
                   "num_splits": plan.num_splits},
        "us_per_call": round(ms_per_step * 1e3, 2),
        "pct_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "kernels_us": {"split": round(float(split_ms.mean()) * 1e3, 2), "combine": round(float(comb_ms.mean()) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": kernel_name,
                     "bytes_per_launch": int(split_bytes / args.steps),
                     "us_per_launch": round(float(split_ms.mean()) * 1e3, 2)},
    }

    # Warm: the same input set every call, so K/V can stay in the 256 MB
    # Infinity Cache and the L2s (a reference point; the value above is cold).
    if not args.no_warm:
        log("[bench] warm leg (one input set)")
        for _ in range(args.warmup):
            step(0)
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            step(0)
        stop.record()
        torch.cuda.synchronize()
        warm_ms = start.elapsed_time(stop) / args.steps
        out["warm"] = {"us_per_call": round(warm_ms * 1e3, 2),
                       "GBs": round(profiling.decode_bytes(sets[0][0]) / (warm_ms * 1e-3) / 1e9, 1),
                       "note": "set 0 every call (caches warm); not the headline value"}

    if not args.no_append:
        log("[bench] append leg: KV append + decode, separate vs fused")
        asets = tensors.decode_sets(args.config, args.sets, dev, num_splits=args.num_splits, new_tokens=True)
        torch.cuda.synchronize()

        def sep(k, ev_app=None):
            _, d = asets[k % len(asets)]
            tensors.run_append(d, timing_events=ev_app)
            tensors.run_decode(d, o=d["o"], lse=d["lse"], workspace=d["ws"], num_splits=args.num_splits)

        def fused(k):
            _, d = asets[k % len(asets)]
            tensors.run_decode_append(d, o=d["o"], lse=d["lse"], workspace=d["ws"], num_splits=args.num_splits)

        legs = {}
        for name, fn in (("separate", sep), ("fused", fused)):
            for k in range(args.warmup):
                fn(k)
            torch.cuda.synchronize()
            start.record()
            for k in range(args.steps):
                fn(k)
            stop.record()
            torch.cuda.synchronize()
            legs[name] = start.elapsed_time(stop) / args.steps * 1e3
        aev = [[HipEvent() for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            sep(k, aev[k])
        torch.cuda.synchronize()
        app_us = float(np.mean([e[0].elapsed_time(e[1]) for e in aev])) * 1e3
        abytes = profiling.append_bytes(asets[0][0])
        out["append"] = {
            "workload": f"{args.config} with each request's last token appended first",
            "us_per_call_separate": round(legs["separate"], 2), "us_per_call_fused": round(legs["fused"], 2),
            "append_kernel_us": round(app_us, 2), "append_bytes": abytes,
            "append_kernel_GBs": round(abytes / (app_us * 1e-6) / 1e9, 1),
            "note": "separate = astr_kv_append then astr_paged_decode; fused = astr_paged_decode_append "
                    "(same output bits); append_kernel_us from dispatch-stamped events of the standalone kernel"}
        del asets

    if not args.no_graph:
        out["graph"] = graph_leg(args, dev)

    if not args.no_prefill:
        log("[bench] prefill leg")
        pin = make_inputs("prefill_b8", 0)
        pd = tensors.to_device(pin, dev)
        po = torch.empty_like(pd["q"])
        plse = torch.empty(pd["q"].shape[0], pd["q"].shape[1], dtype=torch.float32, device=dev)
        pws = tensors.prefill_workspace(pd)          # zeroed once; every call leaves its counters at zero
        psteps = max(10, args.steps // 4)
        fl = prefill_flops(pin)

        def prefill_us(ws):
            for _ in range(5):
                tensors.run_prefill(pd, o=po, lse=plse, workspace=ws)
            torch.cuda.synchronize()
            pev = [[HipEvent() for _ in range(2)] for _ in range(psteps)]
            for k in range(psteps):
                tensors.run_prefill(pd, o=po, lse=plse, timing_events=pev[k], workspace=ws)
            torch.cuda.synchronize()
            return float(np.mean([e[0].elapsed_time(e[1]) for e in pev])) * 1e3

        p_us = prefill_us(pws)
        whole_us = prefill_us(None)
        tf = fl / (p_us * 1e-6) / 1e12
        pa, pkeep = _lib.make_args(pd["q"], pd["k_pool"], pd["v_pool"], pd["req_to_token"], pd["kv_indptr"],
                                   pd["kv_indptr_host"], po, sm_scale=pd["sm_scale"],
                                   req_to_token_stride=pd["req_to_token_stride"], qo_indptr=pd["qo_indptr"],
                                   qo_indptr_host=pd["qo_indptr_host"])
        pplan = _lib.astr_plan_prefill(pa, 0)
        out["prefill"] = {"workload": f"prefill_b8: {CONFIGS['prefill_b8'].description}",
                          "us_per_call": round(p_us, 2), "flops": fl,
                          "plan": {"work_groups": pplan.num_items, "split_tile_heads": pplan.split_tiles,
                                   "chunk_key_tiles": pplan.chunk_tiles, "workspace_bytes": pplan.workspace_bytes},
                          "whole_tiles_us_per_call": round(whole_us, 2),
                          "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                                       "kernel": f"prefill_kernel<{D},{G}>"}}
        del pws, pkeep
        # Long cached prefix with few new tokens (2 requests, 20000 keys, 64 new tokens each): few query
        # tiles with ~313 key tiles each, where the plan splits the key ranges over the idle CUs.
        from paged_gqa_decode_astr_amd.workloads import build_paged_inputs
        lin = build_paged_inputs(np.array([20000, 20000]), 32, 8, 128, 1 << 16, seed=5100, q_lens=np.array([64, 64]))
        ld = tensors.to_device(lin, dev)
        lo = torch.empty_like(ld["q"])
        lws = tensors.prefill_workspace(ld)

        def long_us(ws):
            for _ in range(3):
                tensors.run_prefill(ld, o=lo, workspace=ws)
            torch.cuda.synchronize()
            ev = [[HipEvent() for _ in range(2)] for _ in range(psteps)]
            for k in range(psteps):
                tensors.run_prefill(ld, o=lo, timing_events=ev[k], workspace=ws)
            torch.cuda.synchronize()
            return float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3

        lsplit, lwhole = long_us(lws), long_us(None)
        lfl = prefill_flops(lin)
        out["prefill_long_prefix"] = {
            "workload": "2 requests, seq_len 20000, q_len 64, Hq 32 / Hkv 8, D 128 (long cached prefix)",
            "us_per_call_split": round(lsplit, 2), "us_per_call_whole_tiles": round(lwhole, 2),
            "TFLOPs_split": round(lfl / (lsplit * 1e-6) / 1e12, 1)}
        del ld, lws

    if args.probe:
        log("[bench] probes")
        n = 1 << 29
        a = torch.empty(n, dtype=torch.int16, device=dev)
        bb = torch.empty_like(a)
        for _ in range(3):
            bb.copy_(a)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(20):
            bb.copy_(a)
        t1.record()
        torch.cuda.synchronize()
        copy_gbs = 20 * 2 * a.numel() * 2 / (t0.elapsed_time(t1) * 1e-3) / 1e9
        inp0, d0 = sets[0]
        N = int(inp0["kv_indptr"][-1])
        slots = torch.from_numpy(inp0["req_to_token"][inp0["req_to_token"] >= 0].astype(np.int64)).to(dev)
        kf = d0["k_pool"].view(d0["k_pool"].shape[0], -1)
        vf = d0["v_pool"].view(d0["v_pool"].shape[0], -1)
        gk = torch.index_select(kf, 0, slots)
        gv = torch.index_select(vf, 0, slots)
        torch.cuda.synchronize()
        t0.record()
        for k in range(20):
            _, dk = sets[k % len(sets)]
            torch.index_select(dk["k_pool"].view(dk["k_pool"].shape[0], -1), 0, slots, out=gk)
            torch.index_select(dk["v_pool"].view(dk["v_pool"].shape[0], -1), 0, slots, out=gv)
        t1.record()
        torch.cuda.synchronize()
        gather_gbs = 20 * 2 * (2 * N * kf.shape[1] * 2) / (t0.elapsed_time(t1) * 1e-3) / 1e9
        out["probes"] = {"torch_copy_GBs": round(copy_gbs, 1),
                         "torch_row_gather_GBs": round(gather_gbs, 1),
                         "note": "copy: read+write bytes of a 1 GiB device copy; gather: index_select of the same "
                                 "2 KiB K and V slot rows (read + write counted)"}

    if args.cpu_seconds > 0:
        log("[bench] cpu oracle baseline")
        inp0, d0 = sets[0]
        step(0)
        torch.cuda.synchronize()
        (ref_o, ref_lse), cpu = cpu_baseline(inp0, args.cpu_seconds)
        got = tensors.bf16_to_f64(d0["o"])
        cpu["parity_max_abs"] = float(np.abs(got - ref_o).max())
        out["cpu_baseline"] = cpu

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
