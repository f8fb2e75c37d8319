"""Shared helpers for the GPU parity tests (oracle on the host, HIP path on the GPU)."""
import sys

import numpy as np
import torch

import oracle
from paged_gqa_decode_astr_amd import tensors

ATOL = 1e-2   # max-abs bar against the fp64 oracle
RTOL = 2e-2   # max-rel bar against the fp64 oracle

# Every assert_close call's measured errors, in call order: (what, max_abs, max_rel over |ref| >= 1e-2,
# elements).  conftest.py writes them to the file named by ASTR_PARITY_REPORT at the end of a session.
PARITY_RECORDS = []


def announce(msg: str):
    """Name the case before a GPU step, flushed, so a dying run still says what it ran."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def oracle_of(inp):
    return oracle.paged_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                  inp["req_to_token_stride"], inp["kv_indptr"], inp["sm_scale"],
                                  qo_indptr=inp.get("qo_indptr"))


def assert_close(got: torch.Tensor, ref: np.ndarray, what: str, atol=ATOL, rtol=RTOL, ulp_check=True):
    """Element-wise |got - ref| <= atol + rtol |ref| (max-abs 1e-2 and max-rel 2e-2 read together).

    An absolute bound alone cannot hold for a bf16 output: for |O| in [4, 8) the
    rounding step alone is up to 2^-6 = 0.0156.  Also checked: the output is
    within one bf16 ulp of the fp64 value plus a small fp32 margin (ulp_check;
    off for prefill, whose PV product takes the softmax weights as bf16, which
    moves an output by up to 2^-9 of its V spread).
    """
    g = tensors.bf16_to_f64(got) if got.dtype == torch.bfloat16 else got.detach().double().cpu().numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bad = err > atol + rtol * np.abs(ref)
    big = np.abs(ref) >= 1e-2
    max_rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    PARITY_RECORDS.append({"what": what, "max_abs": float(err.max()), "max_rel": max_rel, "elements": int(err.size),
                           "atol": atol, "rtol": rtol})
    msg = f"{what}: max_abs={err.max():.3e} max_rel(|ref|>=1e-2)={max_rel:.3e} bad={int(bad.sum())}"
    if bad.any():
        idx = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        msg += f" worst at {idx}: got {g[idx]} ref {ref[idx]}"
    assert not bad.any(), msg
    if ulp_check and got.dtype == torch.bfloat16:
        _, e = np.frexp(ref)
        ulp = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)   # bf16 spacing at |ref|
        over = err - (ulp + 2e-3 * np.maximum(1.0, np.abs(ref)))
        assert not (over > 0).any(), f"{what}: error above one bf16 ulp (+2e-3 rel) at {int((over > 0).sum())} elements; {msg}"
    return float(err.max()), max_rel
