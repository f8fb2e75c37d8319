"""rocprofv3 measurements of the decode kernels.

Subcommands:

  workload  the program that is profiled: warm-up and timed decode calls over
            rotating seeded input sets, then a plain copy kernel of known size
            (y = -x over 1 GiB of fp32) used to calibrate the HBM counters.
  pmc       runs `workload` under two rocprofv3 --pmc passes (FETCH_SIZE, then
            WRITE_SIZE), scales the split kernel's per-dispatch counts by what
            the same counters read for the copy kernel, and writes
            profiles/decode_split_<config>_pmc.{json,md}.
  prefill-workload
            the profiled prefill program: warm-up and timed prefill calls on
            one seeded prefill_b8 input set.
  prefill-pmc
            runs `prefill-workload` under rocprofv3 --pmc passes of shader
            counters (matrix-core busy cycles and bf16 MFMA operations, VALU and
            LDS activity, wave occupancy) and writes
            profiles/prefill_kernel_<config>_pmc.{json,md}.
  trace     runs a decode workload's bench.py leg (or, for a prefill
            workload, prefill-workload) under rocprofv3 --kernel-trace --stats
            and writes profiles/decode_<config>_kernel_trace.md (or
            profiles/prefill_<config>_kernel_trace.md).
  prefill-phases
            loads the phase-stamp build of the library (build --stamps), runs
            one prefill call of <config> (default prefill_b8) with its plan and
            writes the per-wavefront cycles of each tile-loop phase to
            profiles/prefill_kernel_<config>_phases.{json,md}.
  decode-timeline
            loads the same build, runs --calls cold decode calls of <config>
            and writes the split work groups' timeline (start, kv_indptr
            staged, first tile, end; by kv head, XCD and piece count) to
            profiles/decode_split_<config>_timeline.{json,md}.

`pmc` and `trace` never touch the GPU themselves (rocprofv3 starts the
profiled program as a child process); `prefill-phases` and `decode-timeline`
run the kernels in this process.  Algorithmic byte counts live here too,
so that bench.py and the summaries use one definition.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import shlex
import statistics
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
# Files whose contents decide what the split kernel reads: a stored counter
# summary is used only while they are unchanged.
TRAFFIC_SOURCES = ("paged_gqa_decode_astr_amd/csrc/decode.hip", "paged_gqa_decode_astr_amd/csrc/api.cpp")
COPY_ELEMS = 1 << 28          # fp32 elements of the calibration copy (1 GiB read + 1 GiB written)
COPY_REPS = 4


# ----------------------------------------------------------------------------- algorithmic bytes

def decode_bytes(inp, with_lse=True):
    """Algorithmic HBM bytes of one decode call, each byte counted once: K and V rows of every
    (key, kv head), q and o, req_to_token entries, kv_indptr and lse."""
    B, Hq, D = inp["q"].shape
    Hkv = inp["num_kv_heads"]
    N = int(inp["kv_indptr"][-1])
    kv = N * Hkv * D * 2 * 2
    qo = 2 * B * Hq * D * 2
    idx = N * 4 + (B + 1) * 4
    return kv + qo + idx + (B * Hq * 4 if with_lse else 0)


def split_kernel_bytes(inp):
    """Bytes the split kernel must read: K + V + q + req_to_token entries + kv_indptr."""
    B, Hq, D = inp["q"].shape
    Hkv = inp["num_kv_heads"]
    N = int(inp["kv_indptr"][-1])
    return N * Hkv * D * 2 * 2 + B * Hq * D * 2 + N * 4 + (B + 1) * 4


def append_bytes(inp):
    """Algorithmic HBM bytes of appending one new token per request: its K and V rows read once and
    written once (every kv head), plus its slot id."""
    B = inp["q"].shape[0]
    Hkv, D = inp["num_kv_heads"], inp["head_dim"]
    return B * Hkv * D * 2 * 2 * 2 + B * 4


PREFILL_SOURCES = ("paged_gqa_decode_astr_amd/csrc/prefill.hip", "paged_gqa_decode_astr_amd/csrc/api.cpp")


def sources_digest_of(path):
    return hashlib.sha256(open(os.path.join(ROOT, path), "rb").read()).hexdigest()


def sources_digest():
    return {p: sources_digest_of(p) for p in TRAFFIC_SOURCES}


def read_traffic(config):
    """HBM bytes per split-kernel launch from the stored counter summary, or None when there is
    none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, f"decode_split_{config}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("sources") != sources_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- profiled program

def _workload(args):
    import torch

    from . import _lib, tensors
    _lib.load_library()
    sets = tensors.decode_sets(args.config, args.sets, "cuda", num_splits=args.num_splits)
    torch.cuda.synchronize()
    for k in range(args.warmup + args.calls):
        tensors.decode_step(sets, k, num_splits=args.num_splits)
    torch.cuda.synchronize()
    x = torch.ones(COPY_ELEMS, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(COPY_REPS):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(f"[workload] {args.config}: {args.warmup}+{args.calls} decode calls over {args.sets} sets, "
          f"{COPY_REPS} copies of {COPY_ELEMS * 4} bytes", flush=True)
    return 0


def _workload_cmd(args):
    return [sys.executable, "-m", "paged_gqa_decode_astr_amd.profiling", "workload", "--config", args.config,
            "--sets", str(args.sets), "--warmup", str(args.warmup), "--calls", str(args.calls),
            "--num-splits", str(args.num_splits)]


def _run_profiler(cmd, log_path, timeout_s):
    """rocprofv3 as a child process (from /tmp, TMPDIR=/tmp); SIGKILL after timeout_s."""
    env = dict(os.environ, TMPDIR="/tmp", PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    full = ["timeout", "-s", "KILL", str(timeout_s)] + cmd
    print("[profile] " + " ".join(shlex.quote(c) for c in full), flush=True)
    with open(log_path, "w") as log:
        rc = subprocess.run(full, cwd="/tmp", env=env, stdout=log, stderr=subprocess.STDOUT).returncode
    if rc != 0:
        with open(log_path) as fh:
            tail = fh.read()[-2000:]
        raise SystemExit(f"profiler run failed (rc={rc}); log tail:\n{tail}")


def _counter_rows(raw_dir):
    files = glob.glob(os.path.join(raw_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {raw_dir}")
    per = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = int(r["Dispatch_Id"])
                ent = per.setdefault(key, {"name": r["Kernel_Name"], "values": {}})
                ent["values"][r["Counter_Name"]] = ent["values"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def _per_dispatch(rows, counter, match, last=None):
    vals = [r["values"][counter] for r in rows if match in r["name"] and counter in r["values"]]
    if last is not None:
        vals = vals[-last:]
    if not vals:
        names = sorted({r["name"][:80] for r in rows})
        raise SystemExit(f"no dispatch of a kernel matching {match!r} with {counter}; kernels seen: {names}")
    return vals


def _pmc(args):
    from .workloads import make_inputs
    raw = os.path.abspath(args.raw)
    os.makedirs(raw, exist_ok=True)
    wl = _workload_cmd(args)
    measured = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        out = os.path.join(raw, counter)
        cmd = ["rocprofv3", "--pmc", counter, "--output-format", "csv", "-d", out, "-o", "run", "--"] + wl
        _run_profiler(cmd, os.path.join(raw, f"{counter}.log"), args.timeout)
        rows = _counter_rows(out)
        split = _per_dispatch(rows, counter, "decode_split_kernel", last=args.calls)
        copy = _per_dispatch(rows, counter, "neg", last=COPY_REPS)
        measured[counter] = {"split_kib": split, "copy_kib": copy}

    copy_bytes = COPY_ELEMS * 4
    f_read = copy_bytes / (statistics.median(measured["FETCH_SIZE"]["copy_kib"]) * 1024)
    f_write = copy_bytes / (statistics.median(measured["WRITE_SIZE"]["copy_kib"]) * 1024)
    fetch = statistics.mean(measured["FETCH_SIZE"]["split_kib"]) * 1024 * f_read
    write = statistics.mean(measured["WRITE_SIZE"]["split_kib"]) * 1024 * f_write
    # Dispatch i of the measured calls used set (warmup + i) mod sets.
    per_set = [split_kernel_bytes(make_inputs(args.config, t)) for t in range(args.sets)]
    algo = statistics.mean(per_set[(args.warmup + i) % args.sets] for i in range(args.calls))
    pass_cmd = ("cd /tmp && TMPDIR=/tmp timeout -s KILL {t} rocprofv3 --pmc {c} --output-format csv -d <raw>/{c} "
                "-o run -- " + " ".join(shlex.quote(c) for c in wl))
    rec = {
        "kernel": "decode_split_kernel",
        "workload": args.config,
        "command": "python3 -m paged_gqa_decode_astr_amd.profiling pmc " + " ".join(
            f"--{k.replace('_', '-')} {v}" for k, v in [("config", args.config), ("sets", args.sets),
                                                       ("warmup", args.warmup), ("calls", args.calls),
                                                       ("num_splits", args.num_splits)]),
        "passes": [pass_cmd.format(t=args.timeout, c=c) for c in ("FETCH_SIZE", "WRITE_SIZE")],
        "sources": sources_digest(),
        "dispatches": args.calls,
        "split_fetch_kib_mean": statistics.mean(measured["FETCH_SIZE"]["split_kib"]),
        "split_write_kib_mean": statistics.mean(measured["WRITE_SIZE"]["split_kib"]),
        "copy_bytes_each_way": copy_bytes,
        "copy_fetch_kib_median": statistics.median(measured["FETCH_SIZE"]["copy_kib"]),
        "copy_write_kib_median": statistics.median(measured["WRITE_SIZE"]["copy_kib"]),
        "read_scale": f_read,
        "write_scale": f_write,
        "hbm_read_bytes_per_launch": fetch,
        "hbm_write_bytes_per_launch": write,
        "hbm_bytes_per_launch": fetch + write,
        "algorithmic_bytes_per_launch": algo,
        "traffic_over_algorithmic": (fetch + write) / algo,
    }
    os.makedirs(PROFILES, exist_ok=True)
    base = os.path.join(PROFILES, f"decode_split_{args.config}_pmc")
    with open(base + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    with open(base + ".md", "w") as fh:
        fh.write(f"# decode_split_kernel HBM traffic, workload {args.config}\n\n")
        fh.write(f"Command: `{rec['command']}`\n\nPasses (each its own rocprofv3 run):\n\n")
        for c in rec["passes"]:
            fh.write(f"- `{c}`\n")
        fh.write("\n| quantity | value |\n|---|---|\n")
        for k in ("dispatches", "split_fetch_kib_mean", "split_write_kib_mean", "copy_bytes_each_way",
                  "copy_fetch_kib_median", "copy_write_kib_median", "read_scale", "write_scale",
                  "hbm_read_bytes_per_launch", "hbm_write_bytes_per_launch", "hbm_bytes_per_launch",
                  "algorithmic_bytes_per_launch", "traffic_over_algorithmic"):
            v = rec[k]
            fh.write(f"| {k} | {v:.6g} |\n" if isinstance(v, float) else f"| {k} | {v} |\n")
        fh.write("\nCounters are FETCH_SIZE / WRITE_SIZE in KiB per dispatch, summed over instances; the scales "
                 "make the copy kernel (y = -x over 1 GiB of fp32) read and write exactly its size.\n")
    print(json.dumps(rec), flush=True)
    return 0


# Shader-counter passes for the prefill kernel.  One rocprofv3 run per pass: a
# run holds at most 8 SQ counters and 2 GRBM counters.
PREFILL_PASSES = (
    ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA", "SQ_BUSY_CU_CYCLES",
     "SQ_WAVE_CYCLES", "SQ_WAVES", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_COEXEC_CYCLES", "GRBM_GUI_ACTIVE"),
    ("SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_LDS", "SQ_INSTS_LDS",
     "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_CYCLES", "GRBM_GUI_ACTIVE"),
)
MI355X_SIMDS = 256 * 4
MI355X_XCDS = 8
MI355X_CLOCK_GHZ = 2.4


def _prefill_workload(args):
    import torch

    from . import _lib, tensors
    from .workloads import make_inputs
    _lib.load_library()
    inp = make_inputs(args.config, 0)
    d = tensors.to_device(inp, "cuda")
    o = torch.empty_like(d["q"])
    lse = torch.empty(d["q"].shape[0], d["q"].shape[1], dtype=torch.float32, device="cuda")
    ws = tensors.prefill_workspace(d)   # zeroed once; every call leaves its counters at zero
    torch.cuda.synchronize()
    for _ in range(args.warmup + args.calls):
        tensors.run_prefill(d, o=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    print(f"[prefill-workload] {args.config}: {args.warmup}+{args.calls} prefill calls", flush=True)
    return 0


def prefill_flops(inp):
    """Algorithmic FLOPs of one prefill call: 4 * D * Hq per causally visible (query row, key) pair."""
    _, Hq, D = inp["q"].shape
    kv, qo = inp["kv_indptr"], inp["qo_indptr"]
    pairs = 0
    for b in range(len(kv) - 1):
        L = int(kv[b + 1] - kv[b])
        qb = int(qo[b + 1] - qo[b])
        pairs += qb * (L - qb) + qb * (qb + 1) // 2
    return 4 * D * Hq * pairs


def _prefill_pmc(args):
    from .workloads import make_inputs
    raw = os.path.abspath(args.raw)
    os.makedirs(raw, exist_ok=True)
    wl = [sys.executable, "-m", "paged_gqa_decode_astr_amd.profiling", "prefill-workload", "--config", args.config,
          "--warmup", str(args.warmup), "--calls", str(args.calls)]
    vals = {}
    passes = []
    for i, counters in enumerate(PREFILL_PASSES):
        out = os.path.join(raw, f"prefill_pass{i}")
        cmd = ["rocprofv3", "--pmc", *counters, "--output-format", "csv", "-d", out, "-o", "run", "--"] + wl
        passes.append("cd /tmp && TMPDIR=/tmp timeout -s KILL {t} ".format(t=args.timeout) +
                      " ".join(shlex.quote(c) for c in cmd).replace(out, f"<raw>/prefill_pass{i}"))
        if not args.summarize_only:
            _run_profiler(cmd, os.path.join(raw, f"prefill_pass{i}.log"), args.timeout)
        rows = _counter_rows(out)
        for c in counters:
            key = c if c != "GRBM_GUI_ACTIVE" else f"GRBM_GUI_ACTIVE_pass{i}"
            vals[key] = statistics.mean(_per_dispatch(rows, c, "prefill_kernel", last=args.calls))
    inp = make_inputs(args.config, 0)
    algo = prefill_flops(inp)
    # GRBM_GUI_ACTIVE comes summed over the 8 XCDs (one GRBM each): per-XCD cycles of the dispatch.
    gui = vals["GRBM_GUI_ACTIVE_pass0"] / MI355X_XCDS
    gui1 = vals["GRBM_GUI_ACTIVE_pass1"] / MI355X_XCDS
    mfma_flops = vals["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    derived = {
        "dispatch_us (GUI active cycles per XCD / 2.4 GHz)": gui / (MI355X_CLOCK_GHZ * 1e3),
        "mfma_util_pct (MFMA busy cycles / (GUI active cycles x 1024 SIMDs))":
            100 * vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * MI355X_SIMDS),
        "mfma_bf16_flops_per_dispatch": mfma_flops,
        "mfma_busy_cycles_per_mfma": vals["SQ_VALU_MFMA_BUSY_CYCLES"] / max(1.0, vals["SQ_INSTS_MFMA"]),
        "algorithmic_flops_per_dispatch (causally visible pairs)": algo,
        "mfma_flops_over_algorithmic": mfma_flops / algo,
        "valu_busy_pct (VALU active quad-cycles x 4 / (GUI cycles x 1024 SIMDs))":
            100 * vals["SQ_ACTIVE_INST_VALU"] * 4 / (gui * MI355X_SIMDS),
        "lds_active_pct (LDS active quad-cycles x 4 / (GUI cycles x 256 CUs))":
            100 * vals["SQ_ACTIVE_INST_LDS"] * 4 / (gui1 * 256),
        "lds_bank_conflict_cycles_over_lds_active": vals["SQ_LDS_BANK_CONFLICT"] / max(1.0, vals["SQ_LDS_IDX_ACTIVE"]),
        "mean_resident_waves_per_cu (wave quad-cycles x 4 / (GUI cycles x 256))":
            vals["SQ_WAVE_CYCLES"] * 4 / (gui * 256),
        "mfma_valu_coexec_over_mfma_busy": vals["SQ_VALU_MFMA_COEXEC_CYCLES"] / max(1.0, vals["SQ_VALU_MFMA_BUSY_CYCLES"]),
    }
    rec = {
        "kernel": "prefill_kernel", "workload": args.config,
        "command": f"python3 -m paged_gqa_decode_astr_amd.profiling prefill-pmc --config {args.config} "
                   f"--warmup {args.warmup} --calls {args.calls}",
        "passes": passes, "sources": {p: sources_digest_of(p) for p in PREFILL_SOURCES},
        "dispatches": args.calls, "counters_mean_per_dispatch": vals, "derived": derived,
    }
    os.makedirs(PROFILES, exist_ok=True)
    base = args.out or os.path.join(PROFILES, f"prefill_kernel_{args.config}_pmc")
    with open(base + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    with open(base + ".md", "w") as fh:
        fh.write(f"# prefill_kernel shader counters, workload {args.config}\n\n")
        fh.write(f"Command: `{rec['command']}`\n\nPasses (each its own rocprofv3 run):\n\n")
        for c in passes:
            fh.write(f"- `{c}`\n")
        fh.write("\n| counter (mean per dispatch, summed over instances) | value |\n|---|---|\n")
        for k, v in vals.items():
            fh.write(f"| {k} | {v:.6g} |\n")
        fh.write("\n| derived | value |\n|---|---|\n")
        for k, v in derived.items():
            fh.write(f"| {k} | {v:.4g} |\n")
        fh.write("\nGRBM_GUI_ACTIVE counts GPU-active cycles of a dispatch, summed over the 8 XCDs; MI355X has 256 CUs "
                 "of 4 SIMDs (SIMD-cycle figures divide by 1024 SIMDs, CU figures by 256 CUs). "
                 "SQ_INSTS_VALU_MFMA_MOPS_BF16 counts bf16 MFMA math operations / 512.\n")
    print(json.dumps(rec), flush=True)
    return 0


def _trace(args, bench_args):
    """Kernel trace of one workload: a decode workload through bench.py (its headline leg only, unless
    bench arguments are given), a prefill workload through prefill-workload."""
    raw = os.path.abspath(args.raw)
    os.makedirs(raw, exist_ok=True)
    prefill = args.config.startswith("prefill")
    if prefill:
        prog = ["-m", "paged_gqa_decode_astr_amd.profiling", "prefill-workload", "--config", args.config,
                "--warmup", str(args.warmup), "--calls", str(args.calls)]
        path = os.path.join(PROFILES, f"prefill_{args.config}_kernel_trace.md")
        title = f"# Kernel trace of the prefill workload {args.config}\n\n"
    else:
        if not bench_args:
            # The headline leg only (plus, at decode_b32, its masked variant, a kernel of its own):
            # bench.py's other legs launch the same kernels at other shapes, which would enter
            # the kernels' averages.
            bench_args = ["--config", args.config, "--cpu-seconds", "0", "--no-graph", "--no-append", "--no-warm",
                          "--no-configs", "--no-prefill"] + ([] if args.config == "decode_b32" else ["--no-masked"])
        prog = [os.path.join(ROOT, "bench.py")] + bench_args
        path = os.path.join(PROFILES, f"decode_{args.config}_kernel_trace.md")
        title = f"# Kernel trace of the decode benchmark, workload {args.config}\n\n"
    cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", raw, "-o", "run", "--",
           sys.executable] + prog
    _run_profiler(cmd, os.path.join(raw, "trace.log"), args.timeout)
    stats = glob.glob(os.path.join(raw, "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {raw}")
    with open(stats[0]) as fh:
        rows = list(csv.DictReader(fh))
    bench = None
    with open(os.path.join(raw, "trace.log")) as fh:
        for line in fh:
            if line.startswith("{") and '"metric"' in line:
                bench = json.loads(line)
    shown = " ".join(shlex.quote(c) for c in ["python3"] + [os.path.relpath(c, ROOT) if c.startswith(ROOT) else c
                                                             for c in prog])
    os.makedirs(PROFILES, exist_ok=True)
    with open(path, "w") as fh:
        fh.write(title)
        fh.write("Command: `cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats --output-format csv "
                 f"-d <raw> -o run -- {shown}`\n\n")
        fh.write("| kernel | calls | average (us) | min (us) | max (us) | share of GPU time (%) |\n|---|---|---|---|---|---|\n")
        for r in rows[: args.top]:
            fh.write(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |\n")
        if bench is not None:
            fh.write(f"\nbench.py under the profiler: whole call {bench['us_per_call']} us.  (Its dispatch-stamped "
                     "event timings are not quoted here: the profiler's per-dispatch work lands inside them.)\n")
    print(open(path).read(), flush=True)
    return 0


# ----------------------------------------------------------------------------- stamped builds

STAMP_WGS = 4096   # work groups whose stamps the kernels keep (kStampWgs in prefill.hip / decode.hip)


def _stamps_lib():
    import ctypes

    from . import _lib, build
    if not os.path.exists(build.STAMPS_LIB):
        raise SystemExit(f"{build.STAMPS_LIB} is missing: python -m paged_gqa_decode_astr_amd.build --stamps")
    lib = _lib.load_library(build.STAMPS_LIB)
    for name in ("astr_debug_prefill_stamps", "astr_debug_decode_stamps"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
        clear = getattr(lib, name + "_clear")
        clear.restype = ctypes.c_int
        clear.argtypes = []
    return lib


def _write_summary(stem, rec, lines):
    os.makedirs(PROFILES, exist_ok=True)
    with open(stem + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
    with open(stem + ".md", "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(json.dumps(rec), flush=True)


def _prefill_phases(args):
    import numpy as np
    import torch

    from . import tensors
    from .workloads import make_inputs
    lib = _stamps_lib()
    inp = make_inputs(args.config, 0)
    d = tensors.to_device(inp, "cuda")
    o = torch.empty_like(d["q"])
    ws = tensors.prefill_workspace(d)            # the library's own plan (None: whole tiles)
    for _ in range(args.warmup):
        tensors.run_prefill(d, o=o, workspace=ws)
    torch.cuda.synchronize()
    assert lib.astr_debug_prefill_stamps_clear() == 0
    torch.cuda.synchronize()
    tensors.run_prefill(d, o=o, workspace=ws)
    torch.cuda.synchronize()
    buf = np.zeros((STAMP_WGS, 8, 6), dtype=np.uint64)
    assert lib.astr_debug_prefill_stamps(buf.ctypes.data, buf.nbytes) == 0
    tiles = buf[:, :, 5].astype(np.float64)
    wg_tiles = tiles.max(axis=1)
    used = wg_tiles > 0
    waves = tiles > 0
    per_tile = buf[:, :, :5].astype(np.float64) / np.maximum(tiles, 1)[:, :, None]
    names = ["gather_issue", "s_and_softmax", "pv", "gather_wait", "barrier"]
    top = used & (wg_tiles >= np.percentile(wg_tiles[used], 90))
    sel_top = waves & top[:, None]

    def means(mask):
        return {n: round(float(per_tile[..., i][mask].mean()), 1) for i, n in enumerate(names)}
    rec = {"kernel": "prefill_kernel", "workload": args.config,
           "command": f"python3 -m paged_gqa_decode_astr_amd.profiling prefill-phases --config {args.config} "
                      f"--warmup {args.warmup}",
           "sources": {pth: sources_digest_of(pth) for pth in PREFILL_SOURCES},
           "work_groups": int(used.sum()), "max_key_tiles": int(wg_tiles.max()),
           "cycles_per_tile_all": means(waves), "cycles_per_tile_longest_10pct": means(sel_top)}
    rec["cycles_per_tile_all"]["total"] = round(sum(rec["cycles_per_tile_all"].values()), 1)
    rec["cycles_per_tile_longest_10pct"]["total"] = round(sum(rec["cycles_per_tile_longest_10pct"].values()), 1)
    lines = [f"# prefill_kernel phase cycles per 64-key tile, workload {args.config}", "",
             f"Command: `{rec['command']}` (after `python -m paged_gqa_decode_astr_amd.build --stamps`).", "",
             "The phase-stamp build of the library (`ASTR_PHASE_STAMPS=1`; the shipped kernels have none of "
             "this code) adds up, per wavefront, the shader-clock cycles (`s_memtime`) of each phase of every "
             "key tile: issuing the next tile's gather, S = K Q^T with mask and softmax, P.V, waiting for the "
             "gather, the barrier. One call with the library's plan "
             f"({rec['work_groups']} work groups, up to {rec['max_key_tiles']} key tiles each).", "",
             "| phase | cycles per tile, all wavefronts | cycles per tile, the 10 % of work groups with the most tiles |",
             "|---|---|---|"]
    for n in names + ["total"]:
        lines.append(f"| {n} | {rec['cycles_per_tile_all'][n]} | {rec['cycles_per_tile_longest_10pct'][n]} |")
    _write_summary(os.path.join(PROFILES, f"prefill_kernel_{args.config}_phases"), rec, lines)
    return 0


def _decode_timeline(args):
    import numpy as np
    import torch

    from . import _lib, tensors
    lib = _stamps_lib()
    sets = tensors.decode_sets(args.config, args.sets, "cuda", num_splits=args.num_splits)
    torch.cuda.synchronize()
    d0 = sets[0][1]
    pargs, keep = _lib.make_args(d0["q"], d0["k_pool"], d0["v_pool"], d0["req_to_token"], d0["kv_indptr"],
                                 d0["kv_indptr_host"], d0["o"], sm_scale=1.0,
                                 req_to_token_stride=d0["req_to_token_stride"], num_splits=args.num_splits)
    plan = _lib.astr_plan_decode(pargs, 0)
    del keep
    gx = plan.grid_x
    for k in range(args.warmup):
        tensors.decode_step(sets, k, num_splits=args.num_splits)
    torch.cuda.synchronize()
    stats = []
    by_head, by_xcd, by_pieces = {}, {}, {}
    for k in range(args.warmup, args.warmup + args.calls):
        assert lib.astr_debug_decode_stamps_clear() == 0
        torch.cuda.synchronize()
        tensors.decode_step(sets, k, num_splits=args.num_splits)
        torch.cuda.synchronize()
        buf = np.zeros((STAMP_WGS, 8), dtype=np.uint64)
        assert lib.astr_debug_decode_stamps(buf.ctypes.data, buf.nbytes) == 0
        ids = np.nonzero(buf[:, 7])[0]
        r = buf[ids].astype(np.float64)
        t0 = r[:, 0].min()
        start, staged, first, end = ((r[:, i] - t0) / 100.0 for i in range(4))   # 100 MHz clock -> us
        loop = end - first
        stats.append({"wgs": len(ids), "span": end.max(), "start_p50": np.median(start), "start_max": start.max(),
                      "staged": np.median(staged - start), "setup": np.median(first - staged),
                      "loop": np.percentile(loop, [10, 50, 90, 100]), "end": np.percentile(end, [10, 50, 90, 100])})
        for key, dct in ((ids // gx, by_head), ((r[:, 5].astype(np.int64) & 0xF), by_xcd), (r[:, 6].astype(np.int64), by_pieces)):
            for v in np.unique(key):
                dct.setdefault(int(v), []).extend(loop[key == v].tolist())

    def med(key):
        return round(float(np.median([s_[key] for s_ in stats])), 2)

    def medv(key):
        return [round(float(x), 2) for x in np.median(np.array([s_[key] for s_ in stats]), axis=0)]
    rec = {"kernel": "decode_split_kernel", "workload": args.config,
           "command": f"python3 -m paged_gqa_decode_astr_amd.profiling decode-timeline --config {args.config} "
                      f"--sets {args.sets} --warmup {args.warmup} --calls {args.calls}",
           "sources": sources_digest(), "work_groups": int(stats[0]["wgs"]), "grid_x": gx, "calls": args.calls,
           "span_us": med("span"), "start_us_p50": med("start_p50"), "start_us_max": med("start_max"),
           "kv_indptr_staged_us": med("staged"), "setup_to_first_tile_us": med("setup"),
           "loop_us_p10_p50_p90_max": medv("loop"), "end_us_p10_p50_p90_max": medv("end"),
           "loop_us_by_kv_head": {h: round(float(np.mean(v)), 2) for h, v in sorted(by_head.items())},
           "loop_us_by_xcd": {x: round(float(np.mean(v)), 2) for x, v in sorted(by_xcd.items())},
           "loop_us_by_pieces": {n: round(float(np.mean(v)), 2) for n, v in sorted(by_pieces.items())}}
    lines = [f"# decode_split_kernel work-group timeline, workload {args.config}", "",
             f"Command: `{rec['command']}` (after `python -m paged_gqa_decode_astr_amd.build --stamps`).", "",
             "The timeline-stamp build of the library (`ASTR_PHASE_STAMPS=1`; the shipped kernels have none of "
             "this code) records, per split work group, the 100 MHz clock (`s_memrealtime`) at its start, once "
             "kv_indptr is staged, when its first tile's loads are issued and at its end, with its XCD and piece "
             f"count. Cold calls rotating over {args.sets} input sets; medians over {args.calls} calls; times in "
             f"µs from the first work group's start. {rec['work_groups']} work groups "
             f"(grid {gx} × kv heads, dispatched head by head).", "",
             "| quantity | value |", "|---|---|",
             f"| last work group ends (µs) | {rec['span_us']} |",
             f"| work-group starts: median / last (µs) | {rec['start_us_p50']} / {rec['start_us_max']} |",
             f"| kv_indptr staged after start (median µs) | {rec['kv_indptr_staged_us']} |",
             f"| staged to first tile issued (median µs) | {rec['setup_to_first_tile_us']} |",
             f"| tile loop p10 / p50 / p90 / max (µs) | {' / '.join(map(str, rec['loop_us_p10_p50_p90_max']))} |",
             f"| work-group ends p10 / p50 / p90 / max (µs) | {' / '.join(map(str, rec['end_us_p10_p50_p90_max']))} |",
             "", "Mean tile-loop time (µs):", "",
             "| kv head | " + " | ".join(str(h) for h in rec["loop_us_by_kv_head"]) + " |",
             "|---|" + "---|" * len(rec["loop_us_by_kv_head"]),
             "| loop | " + " | ".join(str(v) for v in rec["loop_us_by_kv_head"].values()) + " |", "",
             "| XCD | " + " | ".join(str(x) for x in rec["loop_us_by_xcd"]) + " |",
             "|---|" + "---|" * len(rec["loop_us_by_xcd"]),
             "| loop | " + " | ".join(str(v) for v in rec["loop_us_by_xcd"].values()) + " |", "",
             "| pieces | " + " | ".join(str(n) for n in rec["loop_us_by_pieces"]) + " |",
             "|---|" + "---|" * len(rec["loop_us_by_pieces"]),
             "| loop | " + " | ".join(str(v) for v in rec["loop_us_by_pieces"].values()) + " |"]
    _write_summary(os.path.join(PROFILES, f"decode_split_{args.config}_timeline"), rec, lines)
    return 0


def main(argv=None):
    argv = list(sys.argv[1:] if argv is None else argv)
    bench_args = []
    if "--" in argv:
        i = argv.index("--")
        argv, bench_args = argv[:i], argv[i + 1:]
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("mode", choices=["workload", "pmc", "prefill-workload", "prefill-pmc", "trace", "prefill-phases",
                                     "decode-timeline"])
    ap.add_argument("--config", default="decode_b32")
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--calls", type=int, default=40)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--raw", default="gpurun_out/prof", help="directory for rocprofv3's raw output")
    ap.add_argument("--timeout", type=int, default=240, help="seconds before a profiler run is killed")
    ap.add_argument("--top", type=int, default=8, help="kernels listed in the trace summary")
    ap.add_argument("--summarize-only", action="store_true",
                    help="prefill-pmc: write the summary from the raw output already under --raw (no profiler run)")
    ap.add_argument("--out", default=None, help="prefill-pmc: summary file stem (default profiles/prefill_kernel_<config>_pmc)")
    args = ap.parse_args(argv)
    if args.mode == "workload":
        return _workload(args)
    if args.mode == "pmc":
        return _pmc(args)
    if args.mode == "prefill-workload":
        return _prefill_workload(args)
    if args.mode == "prefill-pmc":
        if args.config == "decode_b32":
            args.config = "prefill_b8"
        return _prefill_pmc(args)
    if args.mode == "prefill-phases":
        if args.config == "decode_b32":
            args.config = "prefill_b8"
        return _prefill_phases(args)
    if args.mode == "decode-timeline":
        return _decode_timeline(args)
    return _trace(args, bench_args)


if __name__ == "__main__":
    sys.exit(main())
