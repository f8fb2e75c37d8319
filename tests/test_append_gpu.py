"""GPU parity of the KV append (standalone kernel and the append fused into decode).

Every call goes through the C ABI.  The pools start with the new tokens'
slots unused (NaN), so a new row that is not written, or one that is read from
the pool before it is written, shows up.  Expected pools come from the
oracle's slot list (oracle.new_token_slots) and the generator's new rows;
expected attention outputs from the fp64 oracle run on the oracle's appended
pools.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_gqa_decode_astr_amd import tensors
from paged_gqa_decode_astr_amd.workloads import build_paged_inputs, make_inputs

from _gpu_helpers import announce, assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _i16(t):
    return t.view(torch.int16)


def _expected_pools(inp, dev):
    """Device pools before the append with the oracle's new-token slots overwritten by the new rows."""
    slots = oracle.new_token_slots(inp["req_to_token"], inp["req_to_token_stride"], inp["kv_indptr"],
                                   inp.get("qo_indptr"))
    idx = torch.from_numpy(slots).to(DEV)
    k = dev["k_pool"].clone()
    v = dev["v_pool"].clone()
    k[idx] = dev["k_new"]
    v[idx] = dev["v_new"]
    return k, v


def _oracle_after_append(inp):
    k2, v2 = oracle.kv_append(inp["k_pool"], inp["v_pool"], inp["k_new"], inp["v_new"], inp["req_to_token"],
                              inp["req_to_token_stride"], inp["kv_indptr"], inp.get("qo_indptr"))
    return oracle.paged_attention(inp["q"], k2, v2, inp["req_to_token"], inp["req_to_token_stride"],
                                  inp["kv_indptr"], inp["sm_scale"], qo_indptr=inp.get("qo_indptr"))


@pytest.mark.parametrize("flat", [False, True])
@pytest.mark.parametrize("cid", ["tiny", "decode_b32"])
def test_kv_append_decode_pools_bit_exact(cid, flat):
    inp = make_inputs(cid, 0, new_tokens=1, flat_table=flat)
    announce(f"kv_append decode {cid} flat={flat} seed {inp['seed']}")
    dev = tensors.to_device(inp, DEV)
    k_want, v_want = _expected_pools(inp, dev)
    tensors.run_append(dev)
    torch.cuda.synchronize()
    assert torch.equal(_i16(dev["k_pool"]), _i16(k_want))
    assert torch.equal(_i16(dev["v_pool"]), _i16(v_want))
    # The generator's fully stored pools agree (oracle-independent cross-check).
    assert np.array_equal(dev["k_pool"].view(torch.int16).cpu().numpy().view(np.uint16), inp["k_pool_full"])


@pytest.mark.parametrize("max_q", [0, 600])
def test_kv_append_prefill_then_prefill(max_q):
    """Prefill shape: q_len new tokens per request, appended by the standalone kernel (fixed grid with
    max_q_len), then attended by the prefill kernel."""
    rng = np.random.default_rng(71 + max_q)
    q_lens = rng.integers(1, 300, size=6)
    q_lens[2] = 1
    seq = q_lens + rng.integers(0, 900, size=6)
    seq[4] = q_lens[4]                 # a request with no prefix
    inp = build_paged_inputs(seq, 32, 8, 128, 1 << 14, seed=72 + max_q, q_lens=q_lens, new_tokens=q_lens)
    announce(f"kv_append prefill max_q_len={max_q} q_lens={q_lens.tolist()}")
    dev = tensors.to_device(inp, DEV)
    k_want, v_want = _expected_pools(inp, dev)
    tensors.run_append(dev, max_q_len=max_q)
    torch.cuda.synchronize()
    assert torch.equal(_i16(dev["k_pool"]), _i16(k_want))
    assert torch.equal(_i16(dev["v_pool"]), _i16(v_want))
    o = tensors.run_prefill(dev)
    torch.cuda.synchronize()
    ref_o, _ = _oracle_after_append(inp)
    assert_close(o, ref_o, "prefill after append O", ulp_check=False)


def _separate_and_fused(inp, num_splits=0):
    """(o, lse, pools) of append-then-decode and of the fused call, on two device copies."""
    B, Hq, D = inp["q"].shape
    res = []
    for fused in (False, True):
        dev = tensors.to_device(inp, DEV)
        o = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
        ws = tensors.decode_workspace(B, Hq, D, DEV, max_splits=max(num_splits, 0))
        if fused:
            tensors.run_decode_append(dev, o=o, lse=lse, workspace=ws, num_splits=num_splits)
        else:
            tensors.run_append(dev)
            tensors.run_decode(dev, o=o, lse=lse, workspace=ws, num_splits=num_splits)
        torch.cuda.synchronize()
        res.append((o, lse, dev))
    return res


def _check_fused(inp, what, num_splits=0):
    (o_s, lse_s, dev_s), (o_f, lse_f, dev_f) = _separate_and_fused(inp, num_splits)
    assert torch.equal(_i16(o_s), _i16(o_f)), f"{what}: fused O differs from append + decode"
    assert torch.equal(lse_s.view(torch.int32), lse_f.view(torch.int32)), f"{what}: fused lse differs"
    assert torch.equal(_i16(dev_s["k_pool"]), _i16(dev_f["k_pool"])), f"{what}: pools differ"
    assert torch.equal(_i16(dev_s["v_pool"]), _i16(dev_f["v_pool"])), f"{what}: pools differ"
    return o_f, lse_f, dev_f


@pytest.mark.parametrize("cid", ["tiny", "decode_b32", "ragged_b256", "long_b1"])
def test_decode_append_matches_separate_and_oracle(cid):
    inp = make_inputs(cid, 1, new_tokens=1)
    announce(f"decode_append {cid} seed {inp['seed']} B={inp['q'].shape[0]} N={inp['kv_indptr'][-1]}")
    o, lse, dev = _check_fused(inp, cid)
    # Pools after the fused call: exactly the oracle's slots hold the new rows.
    slots = torch.from_numpy(oracle.new_token_slots(inp["req_to_token"], inp["req_to_token_stride"],
                                                    inp["kv_indptr"])).to(DEV)
    assert torch.equal(_i16(dev["k_pool"][slots]), _i16(dev["k_new"]))
    assert torch.equal(_i16(dev["v_pool"][slots]), _i16(dev["v_new"]))
    ref_o, ref_lse = _oracle_after_append(inp)
    assert_close(o, ref_o, f"{cid} fused O")
    assert_close(lse, ref_lse, f"{cid} fused lse", atol=1e-3, rtol=1e-4)


@pytest.mark.parametrize("Hq,Hkv,D,flat", [(4, 1, 64, False), (8, 4, 64, True), (16, 2, 128, False),
                                           (8, 8, 128, True), (32, 4, 128, False), (64, 8, 128, True)])
def test_decode_append_variants_and_splits(Hq, Hkv, D, flat):
    seq = np.array([1, 2, 15, 16, 17, 33, 64, 65, 128, 129, 130, 300, 1, 511, 1, 700])
    inp = build_paged_inputs(seq, Hq, Hkv, D, 8192, seed=Hq + Hkv + D, flat_table=flat, new_tokens=1)
    ref_o, ref_lse = _oracle_after_append(inp)
    for ns in (0, 1, 3, 16, 200):
        announce(f"decode_append Hq={Hq} Hkv={Hkv} D={D} flat={flat} num_splits={ns}")
        o, lse, _ = _check_fused(inp, f"variant ns={ns}", num_splits=ns)
        assert_close(o, ref_o, f"variant ns={ns} O")
        assert_close(lse, ref_lse, f"variant ns={ns} lse", atol=1e-3, rtol=1e-4)


def test_decode_append_single_key_returns_new_v_bits():
    """seq_len 1: the only key is the new one, so O is the new V row bit for bit."""
    inp = build_paged_inputs(np.ones(24, np.int64), 32, 8, 128, 2048, seed=8, new_tokens=1)
    announce("decode_append single key")
    o, _, _ = _check_fused(inp, "single key", num_splits=5)
    got = o.view(torch.int16).cpu().numpy().view(np.uint16)
    for h in range(32):
        assert np.array_equal(got[:, h, :], inp["v_new"][:, h // 4, :])


def test_decode_append_pool_beyond_32bit_offsets():
    """64-bit addressing path (rows more than 4 GiB above the kv-head base): fused output and pools are
    bit-identical to the same inputs in a small pool."""
    seq = np.array([300, 1, 777, 64, 129, 16, 17])
    inp = build_paged_inputs(seq, 32, 8, 128, 4096, seed=23, new_tokens=1)
    small = tensors.to_device(inp, DEV)
    big_slots = (1 << 21) + 4096
    shift = big_slots - 4096
    big = dict(small)
    big["k_pool"] = torch.full((big_slots, 8, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    big["v_pool"] = torch.full((big_slots, 8, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    big["k_pool"][shift:] = small["k_pool"]
    big["v_pool"][shift:] = small["v_pool"]
    r2t = inp["req_to_token"].copy()
    r2t[r2t >= 0] += shift
    big["req_to_token"] = torch.from_numpy(r2t).to(DEV)
    B, Hq, D = inp["q"].shape
    announce("decode_append with a pool beyond 32-bit row offsets")
    outs = []
    for dev in (small, big):
        o = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
        tensors.run_decode_append(dev, o=o, lse=lse, num_splits=5,
                                  workspace=tensors.decode_workspace(B, Hq, D, DEV, max_splits=5))
        torch.cuda.synchronize()
        outs.append((o, lse))
    assert torch.equal(_i16(outs[0][0]), _i16(outs[1][0]))
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(_i16(big["k_pool"][shift:]), _i16(small["k_pool"]))
    assert torch.equal(_i16(big["v_pool"][shift:]), _i16(small["v_pool"]))
    del big
    ref_o, ref_lse = _oracle_after_append(inp)
    assert_close(outs[0][0], ref_o, "64-bit fused O")


def test_decode_append_graph_capture_replay():
    """Capture the fused call once with a fixed plan, replay it after rewriting every input."""
    B, Hq, Hkv, D, slots = 12, 32, 8, 128, 1 << 14
    rng = np.random.default_rng(45)
    cases = [build_paged_inputs(rng.integers(1, 1200, size=B), Hq, Hkv, D, slots, seed=300 + i,
                                row_stride=1200, new_tokens=1) for i in range(3)]
    dev0 = tensors.to_device(cases[0], DEV)
    o = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    ws = tensors.decode_workspace(B, Hq, D, DEV, max_splits=24)
    announce("decode_append graph capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        tensors.run_decode_append(dev0, o=o, lse=lse, workspace=ws, num_splits=24)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tensors.run_decode_append(dev0, o=o, lse=lse, workspace=ws, num_splits=24)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, inp in enumerate(cases):
            for key in ("q", "k_pool", "v_pool", "k_new", "v_new"):
                dev0[key].copy_(tensors.bf16_tensor(inp[key], DEV))
            dev0["req_to_token"].copy_(torch.from_numpy(inp["req_to_token"]))
            dev0["kv_indptr"].copy_(torch.from_numpy(inp["kv_indptr"]))
            o.fill_(float("nan"))
            torch.cuda.synchronize()
            announce(f"decode_append graph replay {rep}/{i}")
            g.replay()
            torch.cuda.synchronize()
            ref_o, ref_lse = _oracle_after_append(inp)
            assert_close(o, ref_o, f"graph replay {rep}/{i} O")
            assert_close(lse, ref_lse, f"graph replay {rep}/{i} lse", atol=1e-3, rtol=1e-4)
            k_want, _ = _expected_pools(inp, tensors.to_device(inp, DEV))
            assert torch.equal(_i16(dev0["k_pool"]), _i16(k_want))
