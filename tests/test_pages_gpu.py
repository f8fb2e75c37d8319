"""GPU parity of page sizes above one and of head_dim 32 and 256.

Paged inputs come from the generator's page-by-page layout; expected values
from the fp64 oracle with the same page size.  The same keys addressed
through a page-size-one table (the generator's flat list of token slots) must
give the same bits: the kernels see the same values in the same order.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_gqa_decode_astr_amd import tensors
from paged_gqa_decode_astr_amd.workloads import build_paged_inputs

from _gpu_helpers import announce, assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _oracle(inp):
    return oracle.paged_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                  inp["req_to_token_stride"], inp["kv_indptr"], inp["sm_scale"],
                                  qo_indptr=inp.get("qo_indptr"), page_size=inp.get("page_size", 1))


def _token_table(inp):
    """The same inputs addressed through a page-size-one flat table."""
    t = dict(inp)
    t["req_to_token"] = np.ascontiguousarray(inp["token_slots"], dtype=np.int32)
    t["req_to_token_stride"] = 0
    t["page_size"] = 1
    return t


def _decode(inp, num_splits=0):
    dev = tensors.to_device(inp, DEV)
    B, Hq, D = inp["q"].shape
    o = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    tensors.run_decode(dev, o=o, lse=lse, num_splits=num_splits,
                       workspace=tensors.decode_workspace(B, Hq, D, DEV, max_splits=max(num_splits, 0)))
    torch.cuda.synchronize()
    return o, lse


def _prefill(inp, max_q_len=0):
    dev = tensors.to_device(inp, DEV)
    rows, Hq, D = inp["q"].shape
    o = torch.empty(rows, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(rows, Hq, dtype=torch.float32, device=DEV)
    tensors.run_prefill(dev, o=o, lse=lse, max_q_len=max_q_len)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("P", [2, 16, 64, 256])
def test_decode_pages(P):
    rng = np.random.default_rng(P)
    seq = rng.integers(200, 2001, size=32)
    seq[:3] = [1, P, P + 1]
    inp = build_paged_inputs(seq, 32, 8, 128, 1 << 17, seed=P, page_size=P)
    announce(f"decode page_size={P}")
    ref_o, ref_lse = _oracle(inp)
    for ns in (0, 7):
        o, lse = _decode(inp, ns)
        assert_close(o, ref_o, f"pages {P} ns={ns} O")
        assert_close(lse, ref_lse, f"pages {P} ns={ns} lse", atol=1e-3, rtol=1e-4)
        o1, lse1 = _decode(_token_table(inp), ns)
        assert torch.equal(o.view(torch.int16), o1.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), lse1.view(torch.int32))


@pytest.mark.parametrize("P", [4, 64])
def test_prefill_pages(P):
    rng = np.random.default_rng(40 + P)
    q_lens = rng.integers(1, 300, size=6)
    seq = q_lens + rng.integers(0, 900, size=6)
    inp = build_paged_inputs(seq, 32, 8, 128, 1 << 15, seed=P, q_lens=q_lens, page_size=P)
    announce(f"prefill page_size={P}")
    o, lse = _prefill(inp)
    ref_o, ref_lse = _oracle(inp)
    assert_close(o, ref_o, f"prefill pages {P} O", ulp_check=False)
    assert_close(lse, ref_lse, f"prefill pages {P} lse", atol=2e-3, rtol=1e-4)
    o1, lse1 = _prefill(_token_table(inp))
    assert torch.equal(o.view(torch.int16), o1.view(torch.int16))


@pytest.mark.parametrize("P", [8, 32])
def test_append_with_pages(P):
    rng = np.random.default_rng(60 + P)
    seq = rng.integers(1, 400, size=10)
    # decode shape: one new token per request; fused and separate paths
    inp = build_paged_inputs(seq, 32, 8, 128, 1 << 14, seed=P, page_size=P, new_tokens=1)
    announce(f"append decode page_size={P}")
    dev = tensors.to_device(inp, DEV)
    tensors.run_append(dev)
    torch.cuda.synchronize()
    k_full = dev["k_pool"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(k_full, inp["k_pool_full"])
    B, Hq, D = inp["q"].shape
    o_sep = tensors.run_decode(dev, workspace=tensors.decode_workspace(B, Hq, D, DEV))
    dev2 = tensors.to_device(inp, DEV)
    o_fused = tensors.run_decode_append(dev2, workspace=tensors.decode_workspace(B, Hq, D, DEV))
    torch.cuda.synchronize()
    assert torch.equal(o_sep.view(torch.int16), o_fused.view(torch.int16))
    assert torch.equal(dev["v_pool"].view(torch.int16), dev2["v_pool"].view(torch.int16))
    # prefill shape: q_len new tokens per request
    ql = np.minimum(seq, rng.integers(1, 50, size=10))
    pin = build_paged_inputs(seq, 8, 2, 64, 1 << 13, seed=P + 1, page_size=P, q_lens=ql, new_tokens=ql)
    announce(f"append prefill page_size={P}")
    pdev = tensors.to_device(pin, DEV)
    tensors.run_append(pdev)
    torch.cuda.synchronize()
    assert np.array_equal(pdev["v_pool"].view(torch.int16).cpu().numpy().view(np.uint16), pin["v_pool_full"])


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 4), (16, 4), (32, 4)])
def test_head_dim_32_decode_and_prefill(Hq, Hkv):
    rng = np.random.default_rng(Hq)
    seq = rng.integers(1, 900, size=12)
    seq[:4] = [1, 16, 17, 64]
    inp = build_paged_inputs(seq, Hq, Hkv, 32, 1 << 14, seed=Hq + 32)
    announce(f"decode head_dim 32 Hq={Hq} Hkv={Hkv}")
    ref_o, ref_lse = _oracle(inp)
    for ns in (0, 5):
        o, lse = _decode(inp, ns)
        assert_close(o, ref_o, f"D32 decode ns={ns} O")
        assert_close(lse, ref_lse, f"D32 decode ns={ns} lse", atol=1e-3, rtol=1e-4)
    q_lens = np.minimum(seq, rng.integers(1, 200, size=12))
    pin = build_paged_inputs(seq, Hq, Hkv, 32, 1 << 14, seed=Hq + 33, q_lens=q_lens)
    announce(f"prefill head_dim 32 Hq={Hq} Hkv={Hkv}")
    pref_o, pref_lse = _oracle(pin)
    for mq in (0, 256):
        o, lse = _prefill(pin, max_q_len=mq)
        assert_close(o, pref_o, f"D32 prefill mq={mq} O", ulp_check=False)
        assert_close(lse, pref_lse, f"D32 prefill mq={mq} lse", atol=2e-3, rtol=1e-4)


def test_head_dim_32_with_pages_and_mask():
    seq = np.array([300, 1, 77, 640, 33])
    inp = build_paged_inputs(seq, 16, 2, 32, 1 << 13, seed=5, page_size=16)
    mask = (np.random.default_rng(6).random((5, 640)) < 0.7).astype(np.uint8)
    announce("decode head_dim 32, page_size 16, 2-D mask")
    dev = tensors.to_device(inp, DEV)
    o = tensors.run_decode(dev, workspace=tensors.decode_workspace(5, 16, 32, DEV),
                           mask=torch.from_numpy(mask).to(DEV))
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.paged_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                            inp["req_to_token_stride"], inp["kv_indptr"], inp["sm_scale"],
                                            mask=mask, page_size=16)
    empty = np.isneginf(ref_lse)
    assert_close(o, np.where(empty[..., None], 0.0, ref_o), "D32 pages mask O")


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8), (16, 4), (64, 8)])
def test_head_dim_256_decode_and_prefill(Hq, Hkv):
    rng = np.random.default_rng(256 + Hq + Hkv)
    seq = rng.integers(1, 1200, size=10)
    seq[:4] = [1, 16, 17, 129]
    inp = build_paged_inputs(seq, Hq, Hkv, 256, 1 << 14, seed=Hq + 256)
    announce(f"decode head_dim 256 Hq={Hq} Hkv={Hkv}")
    ref_o, ref_lse = _oracle(inp)
    for ns in (0, 3):
        o, lse = _decode(inp, ns)
        assert_close(o, ref_o, f"D256 decode ns={ns} O")
        assert_close(lse, ref_lse, f"D256 decode ns={ns} lse", atol=1e-3, rtol=1e-4)
    q_lens = np.minimum(seq, rng.integers(1, 160, size=10))
    pin = build_paged_inputs(seq, Hq, Hkv, 256, 1 << 14, seed=Hq + 257, q_lens=q_lens)
    announce(f"prefill head_dim 256 Hq={Hq} Hkv={Hkv}")
    pref_o, pref_lse = _oracle(pin)
    o, lse = _prefill(pin)
    assert_close(o, pref_o, "D256 prefill O", ulp_check=False)
    assert_close(lse, pref_lse, "D256 prefill lse", atol=2e-3, rtol=1e-4)


def test_head_dim_256_fused_append_pages_and_mask():
    seq = np.array([300, 1, 77, 640, 33, 1000])
    inp = build_paged_inputs(seq, 16, 4, 256, 1 << 13, seed=7, page_size=16, new_tokens=1)
    mask = (np.random.default_rng(8).random((6, 1000)) < 0.8).astype(np.uint8)
    mt = torch.from_numpy(mask).to(DEV)
    announce("decode_append head_dim 256, page_size 16, 2-D mask")
    dev = tensors.to_device(inp, DEV)
    o = tensors.run_decode_append(dev, workspace=tensors.decode_workspace(6, 16, 256, DEV), mask=mt)
    dev2 = tensors.to_device(inp, DEV)
    tensors.run_append(dev2)
    o2 = tensors.run_decode(dev2, workspace=tensors.decode_workspace(6, 16, 256, DEV), mask=mt)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    k2, v2 = oracle.kv_append(inp["k_pool"], inp["v_pool"], inp["k_new"], inp["v_new"], inp["req_to_token"],
                              inp["req_to_token_stride"], inp["kv_indptr"], page_size=16)
    ref_o, ref_lse = oracle.paged_attention(inp["q"], k2, v2, inp["req_to_token"], inp["req_to_token_stride"],
                                            inp["kv_indptr"], inp["sm_scale"], mask=mask, page_size=16)
    empty = np.isneginf(ref_lse)
    assert_close(o, np.where(empty[..., None], 0.0, ref_o), "D256 fused append pages mask O")
