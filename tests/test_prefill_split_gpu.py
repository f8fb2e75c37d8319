"""GPU parity of prefill with split key ranges (the automatic plan with a workspace).

A query tile whose key range is longer than the plan's chunk length runs as up
to 16 work groups, each over a contiguous chunk of the key tiles; the last one
to finish merges the others' partials.  Every case is compared with the
fp64 oracle, and with the same call made without a workspace (every tile whole).
"""
import numpy as np
import pytest
import torch

from paged_gqa_decode_astr_amd import _lib, tensors
from paged_gqa_decode_astr_amd.workloads import build_paged_inputs, make_inputs

from _gpu_helpers import announce, assert_close, oracle_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _plan(dev, **kw):
    q = dev["q"]
    a, keep = _lib.make_args(q, dev["k_pool"], dev["v_pool"], dev["req_to_token"], dev["kv_indptr"],
                             dev["kv_indptr_host"], q, sm_scale=dev["sm_scale"],
                             req_to_token_stride=dev["req_to_token_stride"], qo_indptr=dev["qo_indptr"],
                             qo_indptr_host=dev["qo_indptr_host"], page_size=dev.get("page_size", 1), **kw)
    plan = _lib.astr_plan_prefill(a, 0)
    del keep
    return plan


def _run(dev, workspace, **kw):
    rows, Hq, _ = dev["q"].shape
    o = torch.full_like(dev["q"], float("nan"))
    lse = torch.full((rows, Hq), float("nan"), dtype=torch.float32, device=DEV)
    tensors.run_prefill(dev, o=o, lse=lse, workspace=workspace, **kw)
    torch.cuda.synchronize()
    return o, lse


def _check_split_and_whole(inp, what, min_split=1, **kw):
    dev = tensors.to_device(inp, DEV)
    plan = _plan(dev, **{k: v for k, v in kw.items() if k in ("non_causal", "mask")})
    assert plan.num_items > 0 and plan.split_tiles >= min_split, (plan.num_items, plan.split_tiles)
    ws = tensors.prefill_workspace(dev, **{k: v for k, v in kw.items() if k in ("non_causal", "mask")})
    announce(f"prefill split {what}: items={plan.num_items} split_tiles={plan.split_tiles} "
             f"chunk_tiles={plan.chunk_tiles}")
    o_s, lse_s = _run(dev, ws, **kw)
    n_cnt = _lib.WORKSPACE_COUNTER_BYTES // 4                    # the counter region opens the workspace
    assert plan.workspace_bytes == _lib.WORKSPACE_COUNTER_BYTES + plan.partial_bytes
    assert bool((ws[:n_cnt] == 0).all()), f"{what}: arrival counters not reset"
    announce(f"prefill whole {what}")
    o_w, lse_w = _run(dev, None, **kw)
    ref_o = ref_lse = None
    if "mask" not in kw and not kw.get("non_causal"):
        import oracle
        ref_o, ref_lse = oracle.paged_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                                inp["req_to_token_stride"], inp["kv_indptr"], inp["sm_scale"],
                                                qo_indptr=inp["qo_indptr"], page_size=inp.get("page_size", 1))
    return o_s, lse_s, o_w, lse_w, ws, ref_o, ref_lse


def test_prefill_b8_split_plan():
    """prefill_b8 has 448 (query tile, kv head) work groups against the 512 slots of 256 CUs:
    the plan halves only its longest tiles, as many as the spare 64 slots allow (7 tiles x 8 kv
    heads), and the split call matches the whole-tile call and the oracle."""
    inp = make_inputs("prefill_b8", 0)
    plan = _plan(tensors.to_device(inp, DEV))
    assert plan.num_items == 504 and plan.split_tiles == 56, (plan.num_items, plan.split_tiles)
    o_s, lse_s, o_w, lse_w, _, ref_o, ref_lse = _check_split_and_whole(inp, "prefill_b8", min_split=56)
    for o, lse, tag in ((o_s, lse_s, "split"), (o_w, lse_w, "whole")):
        assert_close(o, ref_o, f"prefill_b8 {tag} O", ulp_check=False)
        assert_close(lse, ref_lse, f"prefill_b8 {tag} lse", atol=2e-3, rtol=1e-4)


@pytest.mark.parametrize("seq,ql", [(20000, 64), (9000, 300), (33000, 1)])
def test_prefill_split_very_long_prefix(seq, ql):
    """One request with a long cached prefix and few new tokens: few query tiles of 140-520 key
    tiles each, cut into up to 16 chunks."""
    inp = build_paged_inputs(np.array([seq]), 32, 8, 128, 1 << 16, seed=seq + ql, q_lens=np.array([ql]))
    o_s, lse_s, o_w, lse_w, _, ref_o, ref_lse = _check_split_and_whole(inp, f"L={seq} q={ql}", min_split=8)
    for o, lse, tag in ((o_s, lse_s, "split"), (o_w, lse_w, "whole")):
        assert_close(o, ref_o, f"L={seq} q={ql} {tag} O", ulp_check=False)
        assert_close(lse, ref_lse, f"L={seq} q={ql} {tag} lse", atol=2e-3, rtol=1e-4)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 4, 64), (16, 2, 128), (8, 8, 32), (16, 16, 64), (8, 2, 256)])
def test_prefill_split_long_prefixes(Hq, Hkv, D):
    """Long cached prefixes with few new tokens: tiles of 40-90 key tiles, cut into four chunks."""
    seq = np.array([4000, 2600, 5000, 700, 3333])
    ql = np.array([40, 120, 7, 200, 129])
    inp = build_paged_inputs(seq, Hq, Hkv, D, 1 << 15, seed=Hq * 31 + Hkv + D, q_lens=ql)
    o_s, lse_s, o_w, lse_w, _, ref_o, ref_lse = _check_split_and_whole(inp, f"Hq={Hq} Hkv={Hkv} D={D}",
                                                                        min_split=Hkv)
    for o, lse, tag in ((o_s, lse_s, "split"), (o_w, lse_w, "whole")):
        assert_close(o, ref_o, f"long prefixes {tag} O", ulp_check=False)
        assert_close(lse, ref_lse, f"long prefixes {tag} lse", atol=2e-3, rtol=1e-4)


def test_prefill_split_reuses_one_workspace():
    """One zeroed workspace serves consecutive calls of different plans (the counters, at the
    start of the workspace, are left at zero): the same inputs give the same bits every time,
    other inputs in between do not disturb them, and a smaller plan after a larger one (whose
    partials cover more of the workspace) is still right."""
    a = build_paged_inputs(np.array([3000, 1800, 400]), 32, 8, 128, 1 << 14, seed=91, q_lens=np.array([64, 500, 33]))
    b = build_paged_inputs(np.array([2500, 90]), 32, 8, 128, 1 << 14, seed=92, q_lens=np.array([100, 90]))
    da, db = tensors.to_device(a, DEV), tensors.to_device(b, DEV)
    wa, wb = tensors.prefill_workspace(da), tensors.prefill_workspace(db)
    ws = torch.zeros(max(wa.numel(), wb.numel()), dtype=torch.int32, device=DEV)
    announce("prefill split: one workspace, five calls")
    pa, pb = _plan(da), _plan(db)
    assert pa.split_tiles > 0 and pb.split_tiles > 0 and pa.partial_bytes > pb.partial_bytes
    ref_b, _ = oracle_of(b)
    first, _ = _run(da, ws)
    for rep in range(2):
        ob, _ = _run(db, ws)
        assert_close(ob, ref_b, f"reused workspace, smaller plan, call {rep} O", ulp_check=False)
        again, _ = _run(da, ws)
        assert torch.equal(first.view(torch.int16), again.view(torch.int16)), f"call {rep}"
    ref_o, _ = oracle_of(a)
    assert_close(first, ref_o, "reused workspace O", ulp_check=False)
    assert bool((ws[: _lib.WORKSPACE_COUNTER_BYTES // 4] == 0).all()), "arrival counters not reset"


def test_prefill_split_with_masks_and_noncausal():
    seq = np.array([3100, 1900, 2222])
    ql = np.array([50, 300, 1])
    inp = build_paged_inputs(seq, 32, 8, 128, 1 << 14, seed=404, q_lens=ql)
    rng = np.random.default_rng(404)
    m3 = (rng.random((3, 300, 3104)) < 0.5).astype(np.uint8)
    m3[1, :3, :] = 0          # rows of request 1 with no visible key at all
    mask = torch.from_numpy(m3).to(DEV)
    import oracle
    for kw in ({"mask": mask}, {"non_causal": True}, {"non_causal": True, "mask": mask}):
        o_s, lse_s, o_w, lse_w, _, _, _ = _check_split_and_whole(inp, f"{sorted(kw)}", min_split=8, **kw)
        ref_o, ref_lse = oracle.paged_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                                inp["req_to_token_stride"], inp["kv_indptr"], inp["sm_scale"],
                                                qo_indptr=inp["qo_indptr"], non_causal=kw.get("non_causal", False),
                                                mask=m3 if "mask" in kw else None)
        for o, lse, tag in ((o_s, lse_s, "split"), (o_w, lse_w, "whole")):
            assert_close(o, ref_o, f"{sorted(kw)} {tag} O", ulp_check=False)
            fin = np.isfinite(ref_lse)
            got = lse.detach().cpu().numpy()
            assert np.array_equal(np.isfinite(got), fin), f"{sorted(kw)} {tag}: lse -inf rows differ"
            assert np.all(np.abs(got[fin] - ref_lse[fin]) <= 2e-3 + 1e-4 * np.abs(ref_lse[fin])), tag


def test_prefill_split_pages():
    seq = np.array([3000, 2048, 999])
    ql = np.array([200, 48, 300])
    inp = build_paged_inputs(seq, 32, 8, 128, 1 << 14, seed=616, q_lens=ql, page_size=16)
    o_s, lse_s, o_w, lse_w, _, ref_o, ref_lse = _check_split_and_whole(inp, "page_size 16", min_split=8)
    for o, lse, tag in ((o_s, lse_s, "split"), (o_w, lse_w, "whole")):
        assert_close(o, ref_o, f"pages {tag} O", ulp_check=False)
        assert_close(lse, ref_lse, f"pages {tag} lse", atol=2e-3, rtol=1e-4)


def test_prefill_split_rejects_small_workspace():
    inp = build_paged_inputs(np.array([3000, 100]), 32, 8, 128, 1 << 13, seed=5, q_lens=np.array([30, 100]))
    dev = tensors.to_device(inp, DEV)
    plan = _plan(dev)
    assert plan.workspace_bytes > 0
    small = torch.zeros(plan.workspace_bytes // 8, dtype=torch.int32, device=DEV)
    o = torch.full_like(dev["q"], 5.0)
    announce("prefill split: workspace too small")
    with pytest.raises(_lib.AstrError) as ei:
        tensors.run_prefill(dev, o=o, workspace=small)
    assert ei.value.status == _lib.ASTR_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 5.0).all())
