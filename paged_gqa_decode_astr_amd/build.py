"""Build libastr_attn.so in-tree with hipcc for gfx950.

Usage: python -m paged_gqa_decode_astr_amd.build [--jobs N] [--probes]

--probes also builds the standalone measurement programs under probes/ (not
part of the library; the gather-ceiling probe behind the decode roofline).

Every HIP source is compiled with packed-fp32 instructions disabled; the host
C++ ABI layer is compiled by the same driver.  Objects go to _build/, the
shared library next to this file.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libastr_attn.so")
# The same sources built with ASTR_PHASE_STAMPS=1: phase and timeline stamps in
# the prefill and decode kernels, read by `profiling prefill-phases` and
# `profiling decode-timeline`.  Never loaded by the tests or the benchmark.
STAMPS_LIB = os.path.join(PKG, "libastr_attn_stamps.so")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffp-contract=fast", "-munsafe-fp-atomics"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, extra=(), objdir: str = OBJDIR) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + list(extra)
    if src.endswith(".hip"):
        cmd += HIP_FLAGS + ["-c", src, "-o", obj]
    else:
        cmd += ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int | None = None, extra=(), verbose: bool = False, lib: str = LIB, objdir: str = OBJDIR) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, len(srcs))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, objdir), srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    _check_no_missing_kernels(tmp)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build_stamps(jobs: int | None = None, verbose: bool = False) -> str:
    """The phase/timeline-stamp build of the library (a separate file, objects under _build/stamps)."""
    return build(jobs, extra=("-DASTR_PHASE_STAMPS=1",), verbose=verbose, lib=STAMPS_LIB,
                 objdir=os.path.join(OBJDIR, "stamps"))


def _check_no_missing_kernels(lib: str) -> None:
    """The link succeeds even when the host pass of a source left a kernel's
    launch stub out (the symbol stays undefined until the library is
    loaded); catch that here rather than at load time."""
    res = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    if res.returncode != 0:
        return   # no nm: the load-time check in the binding still applies
    missing = [ln.split()[-1] for ln in res.stdout.splitlines() if "_ZN4astr" in ln]
    if missing:
        os.remove(lib)
        raise RuntimeError(f"{len(missing)} library symbols left undefined, e.g. {missing[0]}")


PROBES = os.path.join(PKG, "probes")


def build_probes(verbose: bool = False):
    """Standalone measurement programs (not part of the library): probes/<name>.hip -> probes/<name>."""
    out = []
    for f in sorted(os.listdir(PROBES)) if os.path.isdir(PROBES) else []:
        if not f.endswith(".hip"):
            continue
        src = os.path.join(PROBES, f)
        exe = os.path.join(PROBES, f[:-4])
        # Probes may call the library (include/astr_attn.h, linked from the package directory).
        cmd = [hipcc(), "-O3", "-std=c++17"] + HIP_FLAGS + ["-I", os.path.join(ROOT, "include"), src, "-o", exe,
                                                            "-L", PKG, "-lastr_attn", "-Wl,-rpath,$ORIGIN/.."]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        out.append(exe)
        if verbose:
            print(f"built {exe}")
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--probes", action="store_true", help="also build the measurement programs in probes/")
    ap.add_argument("--stamps", action="store_true", help="also build the phase/timeline-stamp library")
    args = ap.parse_args(argv)
    build(args.jobs, verbose=True)
    if args.probes:
        build_probes(verbose=True)
    if args.stamps:
        build_stamps(args.jobs, verbose=True)


if __name__ == "__main__":
    sys.exit(main())
