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
the kernel's own dispatch stamps at its start and end (hipExtLaunchKernel).
Further sections:
  configs      the other decode workloads (tiny, long_b1, long_b4, ragged_b256),
               each cold, same fields as the headline;
  masked       decode_b32 with a 2-D boolean mask (the masked kernel variant);
  warm         decode_b32 on one input set every call (caches warm; reference);
  append       KV append + decode, separate kernels against the fused call;
  graph        a 32-layer decode step: per-layer GPU time and host issue time of
               eager calls, against one captured graph launch per step;
  prefill      the ragged prefill kernel (B=8, prefix U{0..2048}, q_len
               U{1..512}) against the bf16 MFMA peak, and a long-prefix case;
  cpu_baseline the fp64 CPU oracle on decode_b32, all host cores and 1 thread.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

METRIC = "paged GQA decode µs/call + achieved HBM GB/s (% peak), B=32 seq 200-2000"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, AMD published peak
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, AMD published peak
ROOT = os.path.dirname(os.path.abspath(__file__))
# Input sets per decode workload for cold timing: the bytes one call touches,
# times the sets, stay above twice the 256 MB Infinity Cache.
COLD_SETS = {"tiny": 4, "decode_b32": 4, "long_b1": 4, "long_b4": 2, "ragged_b256": 1}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def oracle_leg(inp, budget_s, threads):
    """Repeated full-batch calls of the fp64 oracle for about budget_s seconds (BLAS limited to
    `threads` threads, None = no limit).  Returns (last output, seconds per call, runs)."""
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=threads):
        runs, t0 = 0, time.perf_counter()
        while True:
            out = oracle.paged_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                         inp["req_to_token_stride"], inp["kv_indptr"], inp["sm_scale"])
            runs += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    return out, el / runs, runs


def cpu_baseline(inp, budget_s):
    """The oracle on the host's cores (BLAS at its default thread count), and on one thread."""
    from threadpoolctl import threadpool_info
    from paged_gqa_decode_astr_amd import profiling
    cores = len(os.sched_getaffinity(0))
    blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
    blas_threads = max(blas) if blas else 1
    out, per_all, runs_all = oracle_leg(inp, budget_s / 2, None)
    _, per_one, runs_one = oracle_leg(inp, budget_s / 2, 1)
    nbytes = profiling.decode_bytes(inp)
    return out, {"value": nbytes / per_all / 1e9, "unit": "GB/s", "cores": cores, "blas_threads": blas_threads,
                 "kind": "oracle", "ms_per_call": round(per_all * 1e3, 1),
                 "one_thread": {"value": round(nbytes / per_one / 1e9, 3), "unit": "GB/s",
                                "ms_per_call": round(per_one * 1e3, 1), "runs": runs_one},
                 "sample": f"fp64 NumPy oracle over one full decode_b32 batch (set 0, {B_str(inp)}), repeated for "
                           f"~{budget_s / 2:.0f} s per leg: {runs_all} run(s) with BLAS at {blas_threads} threads on "
                           f"{cores} cores, {runs_one} run(s) with BLAS at 1 thread"}


def timed_decode(torch, sets, steps, warmup, num_splits=0, mask=None):
    """Cold timing of one decode workload: `steps` calls rotating over `sets`, timed between stream
    events (whole call), then again with dispatch-stamped events for the split and combine kernels."""
    from paged_gqa_decode_astr_amd import profiling, tensors
    from paged_gqa_decode_astr_amd.hip_events import HipEvent

    def call(k, events=None):
        _, d = sets[k % len(sets)]
        tensors.run_decode(d, o=d["o"], lse=d["lse"], workspace=d["ws"], num_splits=num_splits,
                           timing_events=events, mask=None if mask is None else mask[k % len(sets)])

    for k in range(warmup):
        call(k)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(steps):
        call(k)
    stop.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    evs = [[HipEvent() for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        call(k, evs[k])
    torch.cuda.synchronize()
    split_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    comb_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    extra = [0 if mask is None else int(sets[k % len(sets)][0]["kv_indptr"][-1]) for k in range(steps)]
    call_bytes = sum(profiling.decode_bytes(sets[k % len(sets)][0]) + extra[k] for k in range(steps))
    split_bytes = sum(profiling.split_kernel_bytes(sets[k % len(sets)][0]) + extra[k] for k in range(steps))
    gbs = call_bytes / (ms_total * 1e-3) / 1e9
    achieved = split_bytes / (split_ms.sum() * 1e-3) / 1e9
    return {"us_per_call": round(ms_total / steps * 1e3, 2), "GBs": round(gbs, 1),
            "pct_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
            "split_us": round(float(split_ms.mean()) * 1e3, 2), "combine_us": round(float(comb_ms.mean()) * 1e3, 2),
            "split_GBs": round(achieved, 1), "split_frac": round(achieved / PEAK_HBM_GBS, 4),
            "bytes_per_call": int(call_bytes / steps), "split_bytes_per_launch": int(split_bytes / steps)}


def graph_leg(args, dev, layers_per_step=32, batches=(1, 4, 8, 16, 32), steps=20, passes=5):
    """Whole-step graph against eager calls: a decode step of `layers_per_step` layers (each with its own
    pools, queries and outputs; seq_len ~ U{200..2000}, Hq 32 / Hkv 8, D 128) run as per-layer
    astr_paged_decode calls from Python, and as one captured astr_decode_graph replayed per step.
    Each figure is the median over `passes` passes of `steps` steps: the GPU time per step (stream
    events) and, for eager calls, the host time to issue one step's calls."""
    import torch
    from paged_gqa_decode_astr_amd import _lib, tensors
    from paged_gqa_decode_astr_amd.workloads import build_paged_inputs

    res = []
    s = torch.cuda.Stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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

        def timed(fn):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            gpu, host = [], []
            for _ in range(passes):
                t0.record(s)
                h0 = time.perf_counter()
                for _ in range(steps):
                    fn()
                host.append((time.perf_counter() - h0) / steps * 1e6)
                t1.record(s)
                torch.cuda.synchronize()
                gpu.append(t0.elapsed_time(t1) / steps * 1e3)
            return statistics.median(gpu), statistics.median(host)

        eager_us, eager_host_us = timed(eager_step)
        g = _lib.DecodeGraph(layers, ws, num_splits=ns, stream=s)
        graph_us, graph_host_us = timed(g.launch)
        g.close()
        res.append({"batch": B, "eager_us_per_step": round(eager_us, 1),
                    "eager_us_per_layer": round(eager_us / layers_per_step, 2),
                    "eager_host_issue_us_per_layer": round(eager_host_us / layers_per_step, 2),
                    "graph_us_per_step": round(graph_us, 1), "graph_host_issue_us_per_step": round(graph_host_us, 1),
                    "speedup": round(eager_us / graph_us, 2)})
        del layers, ws, keep
        torch.cuda.synchronize()
    return {"workload": f"decode step of {layers_per_step} layers, each its own pools; seq_len ~ U{{200..2000}}, "
                        "Hq 32 / Hkv 8, D 128; eager = per-layer astr_paged_decode calls from Python, graph = one "
                        "astr_decode_graph launch per step",
            "timing": f"median over {passes} passes of {steps} steps; GPU time from stream events, host issue "
                      "time from the host clock around the issuing loop",
            "by_batch": res}


def B_str(inp):
    return f"B={inp['q'].shape[0]}, {int(inp['kv_indptr'][-1])} keys"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4, help="independent input sets rotated to keep caches cold")
    ap.add_argument("--config", default="decode_b32", help="decode workload (tiny, decode_b32, long_b1, long_b4, ragged_b256)")
    ap.add_argument("--cpu-seconds", type=float, default=16.0, help="CPU oracle time budget, both legs (0 = skip)")
    ap.add_argument("--no-configs", action="store_true", help="skip the other decode workloads")
    ap.add_argument("--no-masked", action="store_true", help="skip the masked decode leg")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-append", action="store_true", help="skip the KV append + decode leg")
    ap.add_argument("--no-graph", action="store_true", help="skip the whole-step graph leg")
    ap.add_argument("--no-warm", action="store_true", help="skip the warm-cache reference leg")
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

    log(f"[bench] timing {args.steps} steps (+{args.warmup} warm-up)")
    head = timed_decode(torch, sets, args.steps, args.warmup, args.num_splits)
    plan = _lib.astr_plan_decode(_lib.make_args(
        sets[0][1]["q"], sets[0][1]["k_pool"], sets[0][1]["v_pool"], sets[0][1]["req_to_token"],
        sets[0][1]["kv_indptr"], sets[0][1]["kv_indptr_host"], sets[0][1]["o"], sm_scale=1.0,
        req_to_token_stride=sets[0][1]["req_to_token_stride"], num_splits=args.num_splits)[0], 0)

    B, Hq, D = sets[0][0]["q"].shape
    G = Hq // cfg.num_kv_heads
    kernel_name = f"decode_split_kernel<{D},{G}>"
    traffic = profiling.read_traffic(args.config)
    out = {
        "metric": METRIC, "value": head["GBs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(head["us_per_call"] / 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.config}: {cfg.description}; B={B} Hq={Hq} Hkv={cfg.num_kv_heads} D={D}, "
                               f"pool 2^{int(math.log2(cfg.num_slots))} slots, page_size 1",
                   "batch": B, "cache": f"cold: {args.sets} rotating input sets",
                   "num_splits": plan.num_splits},
        "us_per_call": head["us_per_call"],
        "pct_peak_hbm": head["pct_peak_hbm"],
        "kernels_us": {"split": head["split_us"], "combine": head["combine_us"]},
        "roofline": {"bound": "hbm", "achieved": head["split_GBs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": head["split_frac"], "traffic": traffic, "kernel": kernel_name,
                     "bytes_per_launch": head["split_bytes_per_launch"], "us_per_launch": head["split_us"]},
    }

    if not args.no_masked:
        log("[bench] masked decode leg")
        masks = []
        for t, (inp, _) in enumerate(sets):
            Lmax = int(np.diff(inp["kv_indptr"]).max())
            rng = np.random.default_rng(900 + t)
            m = (rng.random((B, (Lmax + 3) // 4 * 4)) < 0.9).astype(np.uint8)
            m[:, 0] = 1
            masks.append(torch.from_numpy(m).to(dev))
        mres = timed_decode(torch, sets, args.steps, args.warmup, args.num_splits, mask=masks)
        out["masked"] = dict(mres, workload=f"{args.config} with a 2-D [B, kv_len] uint8 mask, 90% of keys visible "
                                              "(bytes include one mask byte per key)",
                             kernel=f"decode_split_kernel<{D},{G},*,*,MASK>")
        del masks

    # Warm: the same input set every call, so K/V can stay in the 256 MB
    # Infinity Cache and the L2s (a reference point; the value above is cold).
    if not args.no_warm:
        log("[bench] warm leg (one input set)")
        wres = timed_decode(torch, sets[:1], args.steps, args.warmup, args.num_splits)
        out["warm"] = {"us_per_call": wres["us_per_call"], "GBs": wres["GBs"], "split_us": wres["split_us"],
                       "note": "set 0 every call (caches warm); not the headline value"}

    if not args.no_append:
        log("[bench] append leg: KV append + decode, separate vs fused")
        asets = tensors.decode_sets(args.config, args.sets, dev, num_splits=args.num_splits, new_tokens=True)
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

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
        fl = profiling.prefill_flops(pin)

        def prefill_us(d, o, ws, lse=None):
            for _ in range(5):
                tensors.run_prefill(d, o=o, lse=lse, workspace=ws)
            torch.cuda.synchronize()
            pev = [[HipEvent() for _ in range(2)] for _ in range(psteps)]
            for k in range(psteps):
                tensors.run_prefill(d, o=o, lse=lse, timing_events=pev[k], workspace=ws)
            torch.cuda.synchronize()
            return float(np.mean([e[0].elapsed_time(e[1]) for e in pev])) * 1e3

        p_us = prefill_us(pd, po, pws, plse)
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
                          "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                                       "kernel": f"prefill_kernel<{D},{G}>"}}
        del pws, pkeep, pd
        # Long cached prefix with few new tokens (2 requests, 20000 keys, 64 new tokens each): few query
        # tiles with ~313 key tiles each, where the plan splits the key ranges over the idle CUs.
        from paged_gqa_decode_astr_amd.workloads import build_paged_inputs
        lin = build_paged_inputs(np.array([20000, 20000]), 32, 8, 128, 1 << 16, seed=5100, q_lens=np.array([64, 64]))
        ld = tensors.to_device(lin, dev)
        lo = torch.empty_like(ld["q"])
        lws = tensors.prefill_workspace(ld)
        lsplit, lwhole = prefill_us(ld, lo, lws), prefill_us(ld, lo, None)
        lfl = profiling.prefill_flops(lin)
        out["prefill_long_prefix"] = {
            "workload": "2 requests, seq_len 20000, q_len 64, Hq 32 / Hkv 8, D 128 (long cached prefix)",
            "us_per_call_split": round(lsplit, 2), "us_per_call_whole_tiles": round(lwhole, 2),
            "TFLOPs_split": round(lfl / (lsplit * 1e-6) / 1e12, 1)}
        del ld, lws

    if args.cpu_seconds > 0:
        log("[bench] cpu oracle baseline")
        inp0, d0 = sets[0]
        tensors.run_decode(d0, o=d0["o"], lse=d0["lse"], workspace=d0["ws"], num_splits=args.num_splits)
        torch.cuda.synchronize()
        (ref_o, ref_lse), cpu = cpu_baseline(inp0, args.cpu_seconds)
        got = tensors.bf16_to_f64(d0["o"])
        cpu["parity_max_abs"] = float(np.abs(got - ref_o).max())
        out["cpu_baseline"] = cpu

    if not args.no_configs and args.config == "decode_b32":
        del sets
        torch.cuda.empty_cache()
        out["configs"] = {}
        for c in ("tiny", "long_b1", "long_b4", "ragged_b256"):
            n = COLD_SETS[c]
            log(f"[bench] config {c} ({n} set(s))")
            csets = tensors.decode_sets(c, n, dev, num_splits=args.num_splits)
            torch.cuda.synchronize()
            cres = timed_decode(torch, csets, min(args.steps, 50), min(args.warmup, 10), args.num_splits)
            cres["workload"] = f"{c}: {CONFIGS[c].description}"
            cres["cache"] = f"cold: {n} input set(s), {cres['bytes_per_call'] * n / 1e6:.0f} MB touched per rotation"
            out["configs"][c] = cres
            del csets
            torch.cuda.empty_cache()

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
