"""Move seeded inputs (numpy bit patterns from workloads.py) onto the GPU and
allocate outputs / workspaces with torch.  Memory plumbing only."""
from __future__ import annotations

import numpy as np
import torch

from . import _lib


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_device(inp: dict, device="cuda") -> dict:
    """Device copies of one batch from workloads.build_paged_inputs / make_inputs."""
    d = {
        "q": bf16_tensor(inp["q"], device),
        "k_pool": bf16_tensor(inp["k_pool"], device),
        "v_pool": bf16_tensor(inp["v_pool"], device),
        "req_to_token": torch.from_numpy(np.ascontiguousarray(inp["req_to_token"])).to(device),
        "kv_indptr": torch.from_numpy(inp["kv_indptr"]).to(device),
        "kv_indptr_host": np.ascontiguousarray(inp["kv_indptr"], dtype=np.int32),
        "req_to_token_stride": int(inp["req_to_token_stride"]),
        "sm_scale": float(inp["sm_scale"]),
        "qo_indptr": None, "qo_indptr_host": None,
        "page_size": int(inp.get("page_size", 1)),
    }
    if inp.get("k_new") is not None:
        d["k_new"] = bf16_tensor(inp["k_new"], device)
        d["v_new"] = bf16_tensor(inp["v_new"], device)
    if inp.get("qo_indptr") is not None:
        d["qo_indptr"] = torch.from_numpy(inp["qo_indptr"]).to(device)
        d["qo_indptr_host"] = np.ascontiguousarray(inp["qo_indptr"], dtype=np.int32)
    return d


def decode_workspace(batch: int, num_qo_heads: int, head_dim: int, device="cuda", max_splits: int = 0,
                     fill: float | None = None) -> torch.Tensor:
    nbytes = _lib.astr_workspace_size(batch, num_qo_heads, head_dim, max_splits)
    n = (nbytes + 3) // 4
    if fill is None:
        return torch.empty(n, dtype=torch.float32, device=device)
    return torch.full((n,), fill, dtype=torch.float32, device=device)


def run_decode(dev: dict, o=None, lse=None, workspace=None, num_splits=0, stream=None, timing_events=None,
               mask=None):
    q = dev["q"]
    if o is None:
        o = torch.empty_like(q)
    if workspace is None:
        workspace = decode_workspace(q.shape[0], q.shape[1], q.shape[2], q.device,
                                     max_splits=max(num_splits, 0))
    _lib.astr_paged_decode(q, dev["k_pool"], dev["v_pool"], dev["req_to_token"], dev["kv_indptr"],
                           dev["kv_indptr_host"], o, workspace, sm_scale=dev["sm_scale"],
                           req_to_token_stride=dev["req_to_token_stride"], lse=lse, num_splits=num_splits,
                           stream=stream, timing_events=timing_events, mask=mask,
                           page_size=dev.get("page_size", 1))
    return o


def run_append(dev: dict, stream=None, timing_events=None, max_q_len=0):
    """Write dev["k_new"] / dev["v_new"] into the device pools (one token per request without qo_indptr)."""
    _lib.astr_kv_append(dev["k_new"], dev["v_new"], dev["k_pool"], dev["v_pool"], dev["req_to_token"],
                        dev["kv_indptr"], dev["kv_indptr_host"], req_to_token_stride=dev["req_to_token_stride"],
                        qo_indptr=dev["qo_indptr"], qo_indptr_host=dev["qo_indptr_host"], max_q_len=max_q_len,
                        stream=stream, timing_events=timing_events, page_size=dev.get("page_size", 1))


def run_decode_append(dev: dict, o=None, lse=None, workspace=None, num_splits=0, stream=None, timing_events=None,
                      mask=None):
    """Fused append of dev["k_new"] / dev["v_new"] and decode."""
    q = dev["q"]
    if o is None:
        o = torch.empty_like(q)
    if workspace is None:
        workspace = decode_workspace(q.shape[0], q.shape[1], q.shape[2], q.device,
                                     max_splits=max(num_splits, 0))
    _lib.astr_paged_decode_append(q, dev["k_new"], dev["v_new"], dev["k_pool"], dev["v_pool"], dev["req_to_token"],
                                  dev["kv_indptr"], dev["kv_indptr_host"], o, workspace, sm_scale=dev["sm_scale"],
                                  req_to_token_stride=dev["req_to_token_stride"], lse=lse, num_splits=num_splits,
                                  stream=stream, timing_events=timing_events, mask=mask,
                           page_size=dev.get("page_size", 1))
    return o


def prefill_workspace(dev: dict, non_causal=False, mask=None, max_q_len=0, device=None):
    """A zeroed workspace sized by astr_plan_prefill for this batch (None when its plan splits nothing)."""
    q = dev["q"]
    a, keep = _lib.make_args(q, dev["k_pool"], dev["v_pool"], dev["req_to_token"], dev["kv_indptr"],
                             dev["kv_indptr_host"], q, sm_scale=dev["sm_scale"],
                             req_to_token_stride=dev["req_to_token_stride"], qo_indptr=dev["qo_indptr"],
                             qo_indptr_host=dev["qo_indptr_host"], max_q_len=max_q_len, non_causal=non_causal,
                             mask=mask, page_size=dev.get("page_size", 1))
    nbytes = _lib.astr_plan_prefill(a, 0).workspace_bytes
    del keep
    if nbytes == 0:
        return None
    return torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device=device or q.device)


def run_prefill(dev: dict, o=None, lse=None, max_q_len=0, stream=None, timing_events=None, non_causal=False,
                mask=None, workspace="auto"):
    """workspace: "auto" (a fresh zeroed workspace from the plan, so long tiles are split), None (every
    query tile whole) or a zeroed tensor reused across calls."""
    q = dev["q"]
    if o is None:
        o = torch.empty_like(q)
    if isinstance(workspace, str):
        workspace = prefill_workspace(dev, non_causal=non_causal, mask=mask, max_q_len=max_q_len)
    _lib.astr_paged_prefill(q, dev["k_pool"], dev["v_pool"], dev["req_to_token"], dev["kv_indptr"],
                            dev["kv_indptr_host"], dev["qo_indptr"], dev["qo_indptr_host"], o,
                            sm_scale=dev["sm_scale"], req_to_token_stride=dev["req_to_token_stride"], lse=lse,
                            max_q_len=max_q_len, stream=stream, timing_events=timing_events,
                            non_causal=non_causal, mask=mask, page_size=dev.get("page_size", 1),
                            workspace=workspace)
    return o


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def decode_sets(config: str, nsets: int, device="cuda", num_splits: int = 0, new_tokens: bool = False):
    """`nsets` independent seeded batches of a decode workload, resident on the device, each with its
    own output, lse and workspace.  Rotating over them keeps each call's K/V out of the caches.
    new_tokens: each request's last token is held back as k_new / v_new (for the append paths)."""
    from .workloads import make_inputs
    sets = []
    for t in range(nsets):
        inp = make_inputs(config, t, new_tokens=1) if new_tokens else make_inputs(config, t)
        d = to_device(inp, device)
        B, Hq, D = inp["q"].shape
        d["o"] = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=device)
        d["lse"] = torch.empty(B, Hq, dtype=torch.float32, device=device)
        d["ws"] = decode_workspace(B, Hq, D, device, max_splits=num_splits)
        sets.append((inp, d))
    return sets


def decode_step(sets, k: int, num_splits: int = 0, timing_events=None):
    """One decode call on set k mod len(sets)."""
    _, d = sets[k % len(sets)]
    run_decode(d, o=d["o"], lse=d["lse"], workspace=d["ws"], timing_events=timing_events, num_splits=num_splits)
