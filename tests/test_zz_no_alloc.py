"""GPU checks of the allocation-free decode entry point (astr_paged_decode_noalloc).

It runs the same kernels as astr_paged_decode, with the split partials in the
library's own device scratch array instead of a caller workspace, so with the
same plan its output, lse and bits must equal astr_paged_decode's.  Calls go
through the C ABI; the second call of a pair is smaller than the first, so any
dependence on what the previous call left in the shared scratch would show.
"""
import numpy as np
import pytest
import torch

from paged_gqa_decode_astr_amd import _lib, tensors
from paged_gqa_decode_astr_amd.workloads import build_paged_inputs, make_inputs

from _gpu_helpers import announce, assert_close, oracle_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _with_workspace(dev, num_splits=0, mask=None):
    B, Hq, D = dev["q"].shape
    o = torch.empty_like(dev["q"])
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    ws = tensors.decode_workspace(B, Hq, D, DEV, max_splits=num_splits)
    _lib.astr_paged_decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["req_to_token"], dev["kv_indptr"],
                           dev["kv_indptr_host"], o, ws, sm_scale=dev["sm_scale"],
                           req_to_token_stride=dev["req_to_token_stride"], lse=lse, num_splits=num_splits,
                           mask=mask, page_size=dev.get("page_size", 1))
    return o, lse


def _noalloc(dev, num_splits=0, mask=None):
    B, Hq, _ = dev["q"].shape
    o = torch.full_like(dev["q"], float("nan"))
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    _lib.astr_paged_decode_noalloc(dev["q"], dev["k_pool"], dev["v_pool"], dev["req_to_token"], dev["kv_indptr"],
                                   dev["kv_indptr_host"], o, sm_scale=dev["sm_scale"],
                                   req_to_token_stride=dev["req_to_token_stride"], lse=lse, num_splits=num_splits,
                                   mask=mask, page_size=dev.get("page_size", 1))
    return o, lse


def _same_bits(a, b, what):
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), what


@pytest.mark.parametrize("first,second", [("decode_b32", "tiny"), ("ragged_b256", "decode_b32"),
                                          ("long_b4", "long_b1")])
def test_noalloc_matches_workspace_entry_two_calls(first, second):
    """Two allocation-free calls in a row (the second on a smaller input), each equal bit for bit to
    astr_paged_decode with a caller workspace and within tolerance of the oracle."""
    for cid in (first, second):
        inp = make_inputs(cid, 0)
        announce(f"noalloc {cid} seed {inp['seed']} B={inp['q'].shape[0]} N={inp['kv_indptr'][-1]}")
        dev = tensors.to_device(inp, DEV)
        o_na, lse_na = _noalloc(dev)
        torch.cuda.synchronize()
        o_ws, lse_ws = _with_workspace(dev)
        torch.cuda.synchronize()
        _same_bits(o_na, o_ws, f"{cid}: O differs from astr_paged_decode")
        _same_bits(lse_na, lse_ws, f"{cid}: lse differs from astr_paged_decode")
        ref_o, ref_lse = oracle_of(inp)
        assert_close(o_na, ref_o, f"noalloc {cid} O")
        assert_close(lse_na, ref_lse, f"noalloc {cid} lse", atol=1e-3, rtol=1e-4)


def test_noalloc_fixed_plan_mask_and_pages():
    """Fixed split counts, a 2-D mask and a page size above one through the allocation-free call."""
    seq = np.array([700, 1, 64, 65, 1200, 33, 300])
    inp = build_paged_inputs(seq, 32, 8, 128, 1 << 14, seed=515, page_size=16)
    dev = tensors.to_device(inp, DEV)
    rng = np.random.default_rng(5)
    m = (rng.random((len(seq), 1200)) < 0.7).astype(np.uint8)
    m[:, 0] = 1
    mask = torch.from_numpy(m).to(DEV)
    for ns, mk in ((7, None), (96, mask), (1, mask), (0, None)):
        announce(f"noalloc pages=16 num_splits={ns} mask={mk is not None}")
        o_na, lse_na = _noalloc(dev, num_splits=ns, mask=mk)
        torch.cuda.synchronize()
        o_ws, lse_ws = _with_workspace(dev, num_splits=ns, mask=mk)
        torch.cuda.synchronize()
        _same_bits(o_na, o_ws, f"ns={ns}: O differs from astr_paged_decode")
        _same_bits(lse_na, lse_ws, f"ns={ns}: lse differs from astr_paged_decode")


def test_noalloc_rejects_plans_beyond_the_scratch():
    """A plan whose partials exceed the fixed scratch is refused before anything is enqueued."""
    B = 2600
    inp = build_paged_inputs(np.ones(B, dtype=np.int64), 32, 8, 128, 4096, seed=3)
    dev = tensors.to_device(inp, DEV)
    a, keep = _lib.make_args(dev["q"], dev["k_pool"], dev["v_pool"], dev["req_to_token"], dev["kv_indptr"],
                             dev["kv_indptr_host"], dev["q"], sm_scale=1.0,
                             req_to_token_stride=dev["req_to_token_stride"])
    need = _lib.astr_plan_decode(a, 0).workspace_bytes
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    announce(f"noalloc rejects B={B} needing {need} bytes")
    o = torch.full_like(dev["q"], 7.0)
    with pytest.raises(_lib.AstrError) as ei:
        _lib.astr_paged_decode_noalloc(dev["q"], dev["k_pool"], dev["v_pool"], dev["req_to_token"],
                                       dev["kv_indptr"], dev["kv_indptr_host"], o, sm_scale=dev["sm_scale"],
                                       req_to_token_stride=dev["req_to_token_stride"])
    assert ei.value.status == _lib.ASTR_ERR_WORKSPACE
    assert "scratch" in ei.value.message
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()), "a rejected call wrote its output"
    del keep
    # A call that fits still runs after a rejection.
    small = tensors.to_device(build_paged_inputs(np.arange(600) % 50 + 1, 32, 8, 128, 1 << 15, seed=4), DEV)
    o2, _ = _noalloc(small, num_splits=1)
    torch.cuda.synchronize()
    o3, _ = _with_workspace(small, num_splits=1)
    torch.cuda.synchronize()
    _same_bits(o2, o3, "call after a rejection")
