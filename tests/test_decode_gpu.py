"""GPU parity of paged GQA decode (split kernel + combine) against the fp64 oracle.

Every call goes through the C ABI (libastr_attn.so via ctypes).  Unused pool
slots hold NaN in every case, so any read outside a request's keys shows up.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_gqa_decode_astr_amd import _lib, tensors
from paged_gqa_decode_astr_amd.workloads import build_paged_inputs, make_inputs

from _gpu_helpers import announce, assert_close, oracle_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _decode(inp, num_splits=0, with_lse=True, ws_fill=None, o=None):
    dev = tensors.to_device(inp, DEV)
    B, Hq, D = inp["q"].shape
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV) if with_lse else None
    ws = tensors.decode_workspace(B, Hq, D, DEV, max_splits=max(num_splits, 0), fill=ws_fill)
    out = tensors.run_decode(dev, o=o, lse=lse, workspace=ws, num_splits=num_splits)
    torch.cuda.synchronize()
    return out, lse, ws, dev


@pytest.mark.parametrize("trial", [0, 1, 2])
@pytest.mark.parametrize("cid", ["tiny", "decode_b32", "long_b1", "long_b4", "ragged_b256"])
def test_decode_parity_configs(cid, trial):
    inp = make_inputs(cid, trial)
    announce(f"decode parity {cid} trial {trial} seed {inp['seed']} B={inp['q'].shape[0]} N={inp['kv_indptr'][-1]}")
    o, lse, _, _ = _decode(inp)
    ref_o, ref_lse = oracle_of(inp)
    assert_close(o, ref_o, f"{cid}/{trial} O")
    assert_close(lse, ref_lse, f"{cid}/{trial} lse", atol=1e-3, rtol=1e-4)


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 1, 64), (8, 4, 64), (16, 2, 128), (8, 8, 128), (32, 4, 128), (16, 16, 64)])
def test_decode_group_and_head_dim_variants(Hq, Hkv, D):
    rng = np.random.default_rng(Hq * 100 + Hkv * 10 + D)
    seq = rng.integers(1, 700, size=9)
    inp = build_paged_inputs(seq, Hq, Hkv, D, 8192, seed=int(seq.sum()))
    announce(f"decode variant Hq={Hq} Hkv={Hkv} D={D} seq={seq.tolist()}")
    for ns in (0, 3):
        o, lse, _, _ = _decode(inp, num_splits=ns)
        ref_o, ref_lse = oracle_of(inp)
        assert_close(o, ref_o, f"variant ns={ns} O")
        assert_close(lse, ref_lse, f"variant ns={ns} lse", atol=1e-3, rtol=1e-4)


@pytest.mark.parametrize("D", [128, 64])
def test_decode_combine_head_blocks_with_several_groups(D):
    """256 short requests and one long one: the combine's grid is large enough for several head
    blocks per work group (4 at head_dim 128, 2 at 64) and the long request spans more than 8
    pieces, so each block also has several thread groups merging through their own LDS slots."""
    seq = np.full(256, 60)
    seq[101] = 6000
    inp = build_paged_inputs(seq, 32, 8, D, 1 << 15, seed=D + 7)
    announce(f"decode combine head blocks D={D} B=256 N={int(seq.sum())}")
    o, lse, _, _ = _decode(inp)
    ref_o, ref_lse = oracle_of(inp)
    assert_close(o, ref_o, f"combine head blocks D={D} O")
    assert_close(lse, ref_lse, f"combine head blocks D={D} lse", atol=1e-3, rtol=1e-4)


def test_decode_tile_boundary_lengths():
    seq = np.array([1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513])
    inp = build_paged_inputs(seq, 32, 8, 128, 8192, seed=99)
    ref_o, ref_lse = oracle_of(inp)
    for ns in (0, 1, 2, 5, 13, 64, 1000):
        announce(f"decode tile boundaries num_splits={ns}")
        o, lse, _, _ = _decode(inp, num_splits=ns)
        assert_close(o, ref_o, f"boundaries ns={ns} O")
        assert_close(lse, ref_lse, f"boundaries ns={ns} lse", atol=1e-3, rtol=1e-4)


@pytest.mark.parametrize("ns", [1, 2, 4, 9, 23])
def test_decode_block_split_edges(ns):
    """Inside a work group the window's 32-key pairs are cut into four
    contiguous blocks, one per wavefront.  These lengths and split counts give
    windows with fewer pairs than wavefronts (empty blocks), pieces that start
    inside a block and cross its end (the leader's second slot), pieces that
    span three or four blocks, one-key pieces, and windows limited by the q
    batch (more pieces than one batch holds)."""
    seq = np.array([1, 33, 64, 65, 2, 31, 32, 97, 1, 1, 1, 200, 5, 129, 3, 1, 1, 40, 96, 1])
    inp = build_paged_inputs(seq, 16, 4, 128, 4096, seed=77 + ns)
    announce(f"decode block-split edges num_splits={ns}")
    o, lse, _, _ = _decode(inp, num_splits=ns)
    ref_o, ref_lse = oracle_of(inp)
    assert_close(o, ref_o, f"block split ns={ns} O")
    assert_close(lse, ref_lse, f"block split ns={ns} lse", atol=1e-3, rtol=1e-4)


def test_decode_single_key_returns_v_bits():
    """seq_len 1: the weight is exactly 1, so O must equal the V row bit for bit (right kv head)."""
    inp = build_paged_inputs(np.ones(40, np.int64), 32, 8, 128, 4096, seed=5)
    announce("decode single key")
    o, lse, _, _ = _decode(inp, num_splits=7)
    got = o.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(40):
        slot = int(inp["req_to_token"][b * inp["req_to_token_stride"]])
        want = inp["v_pool"][slot][np.arange(32) // 4]
        assert np.array_equal(got[b], want), b


def test_decode_slot_permutation_bit_identical():
    """Moving K/V rows to other pool slots (and remapping the table) changes no output bit."""
    seq = np.array([300, 1, 1200, 77, 640])
    inp = build_paged_inputs(seq, 32, 8, 128, 4096, seed=8)
    perm = np.random.default_rng(3).permutation(4096)
    moved = dict(inp)
    moved["k_pool"] = np.empty_like(inp["k_pool"])
    moved["v_pool"] = np.empty_like(inp["v_pool"])
    moved["k_pool"][perm] = inp["k_pool"]
    moved["v_pool"][perm] = inp["v_pool"]
    r2t = inp["req_to_token"].copy()
    r2t[r2t >= 0] = perm[r2t[r2t >= 0]]
    moved["req_to_token"] = r2t
    announce("decode slot permutation")
    o1, l1, _, _ = _decode(inp, num_splits=9)
    o2, l2, _, _ = _decode(moved, num_splits=9)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_decode_flat_table_and_strided_views():
    seq = np.array([5, 900, 33, 1, 260])
    flat = build_paged_inputs(seq, 16, 4, 128, 2048, seed=12, flat_table=True)
    twod = build_paged_inputs(seq, 16, 4, 128, 2048, seed=12, flat_table=False, row_stride=1000)
    announce("decode flat table / strided q,o")
    o_flat, _, _, _ = _decode(flat, num_splits=4)
    o_2d, _, _, _ = _decode(twod, num_splits=4)
    assert torch.equal(o_flat.view(torch.int16), o_2d.view(torch.int16))
    ref_o, _ = oracle_of(flat)
    assert_close(o_flat, ref_o, "flat table O")
    # q and o as views with padded head and token strides
    dev = tensors.to_device(flat, DEV)
    B, Hq, D = flat["q"].shape
    qbig = torch.zeros(B, Hq, 2 * D, dtype=torch.bfloat16, device=DEV)
    qbig[:, :, :D] = dev["q"]
    dev["q"] = qbig[:, :, :D]
    obig = torch.full((B, Hq + 3, D + 8), float("nan"), dtype=torch.bfloat16, device=DEV)
    oview = obig[:, 1:Hq + 1, :D]
    ws = tensors.decode_workspace(B, Hq, D, DEV)
    lse_big = torch.full((B, Hq + 5), float("nan"), dtype=torch.float32, device=DEV)
    tensors.run_decode(dev, o=oview, lse=lse_big[:, :Hq], workspace=ws, num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(oview.contiguous().view(torch.int16), o_flat.view(torch.int16))
    assert torch.isnan(obig[:, 0]).all() and torch.isnan(obig[:, Hq + 1:]).all() and torch.isnan(obig[:, :, D:]).all()
    assert torch.isnan(lse_big[:, Hq:]).all()


@pytest.mark.parametrize("ns", [1, 3, 64])
def test_decode_partial_layout_matches_oracle(ns):
    """Workspace prefilled with NaN: exactly the planned slots are written, with the oracle's values."""
    inp = make_inputs("decode_b32", 0)
    B, Hq, D = inp["q"].shape
    announce(f"decode partial layout num_splits={ns}")
    o, lse, ws, _ = _decode(inp, num_splits=ns, ws_fill=float("nan"))
    P = ns + B - 1
    wsn = ws.cpu().numpy()
    o_part = wsn[: Hq * P * D].reshape(Hq, P, D)
    ml_off = ((Hq * P * D * 4 + 255) // 256 * 256) // 4
    ml_part = wsn[ml_off: ml_off + Hq * P * 2].reshape(Hq, P, 2)
    ref_o, ref_ml = oracle.split_partials(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                          inp["req_to_token_stride"], inp["kv_indptr"], inp["sm_scale"], ns)
    written = np.isfinite(ref_ml[:, :, 0])
    assert np.array_equal(np.isfinite(ml_part[:, :, 0]), written)
    assert np.array_equal(np.isfinite(ml_part[:, :, 1]), written)
    assert np.array_equal(np.isfinite(o_part).all(axis=2), written)
    assert np.isnan(o_part[~written]).all()
    np.testing.assert_allclose(ml_part[written][:, 0], ref_ml[written][:, 0], atol=2e-3, rtol=0)
    np.testing.assert_allclose(ml_part[written][:, 1], ref_ml[written][:, 1], rtol=2e-3)
    np.testing.assert_allclose(o_part[written], ref_o[written], atol=1e-3, rtol=1e-3)


def test_decode_graph_capture_replay_with_new_lengths():
    """Capture once with a fixed plan, then replay after rewriting the device index arrays."""
    B, Hq, Hkv, D, slots = 16, 32, 8, 128, 1 << 15
    rng = np.random.default_rng(44)
    cases = [build_paged_inputs(rng.integers(1, 1500, size=B), Hq, Hkv, D, slots, seed=100 + i,
                                row_stride=1500) for i in range(4)]
    dev0 = tensors.to_device(cases[0], DEV)
    o = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    ws = tensors.decode_workspace(B, Hq, D, DEV, max_splits=32)
    announce("decode graph capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        tensors.run_decode(dev0, o=o, lse=lse, workspace=ws, num_splits=32)   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tensors.run_decode(dev0, o=o, lse=lse, workspace=ws, num_splits=32)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, inp in enumerate(cases):
            dev0["q"].copy_(tensors.bf16_tensor(inp["q"], DEV))
            dev0["k_pool"].copy_(tensors.bf16_tensor(inp["k_pool"], DEV))
            dev0["v_pool"].copy_(tensors.bf16_tensor(inp["v_pool"], DEV))
            dev0["req_to_token"].copy_(torch.from_numpy(inp["req_to_token"]))
            dev0["kv_indptr"].copy_(torch.from_numpy(inp["kv_indptr"]))
            o.fill_(float("nan"))
            torch.cuda.synchronize()
            announce(f"decode graph replay {rep}/{i}")
            g.replay()
            torch.cuda.synchronize()
            ref_o, ref_lse = oracle_of(inp)
            assert_close(o, ref_o, f"graph replay {rep}/{i} O")
            assert_close(lse, ref_lse, f"graph replay {rep}/{i} lse", atol=1e-3, rtol=1e-4)


def test_decode_runs_on_the_callers_stream():
    inp = make_inputs("tiny", 1)
    dev = tensors.to_device(inp, DEV)
    B, Hq, D = inp["q"].shape
    s = torch.cuda.Stream()
    o = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    ws = tensors.decode_workspace(B, Hq, D, DEV)
    announce("decode on a side stream")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        tensors.run_decode(dev, o=o, workspace=ws)
    s.synchronize()
    ref_o, _ = oracle_of(inp)
    assert_close(o, ref_o, "side stream O")


def test_decode_pool_beyond_32bit_offsets():
    """Rows more than 4 GiB above the kv-head base take the 64-bit addressing path; results are
    bit-identical to the same rows in a small pool (32-bit buffer path) and match the oracle."""
    seq = np.array([300, 1, 777, 64, 129])
    inp = build_paged_inputs(seq, 32, 8, 128, 4096, seed=21)
    small = tensors.to_device(inp, DEV)
    big_slots = (1 << 21) + 4096          # 2^21 slots x 2 KiB rows: > 4 GiB per pool
    shift = big_slots - 4096              # small-pool slot s lives at s + shift
    big = dict(small)
    big["k_pool"] = torch.full((big_slots, 8, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    big["v_pool"] = torch.full((big_slots, 8, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    big["k_pool"][shift:] = small["k_pool"]
    big["v_pool"][shift:] = small["v_pool"]
    r2t = inp["req_to_token"].copy()
    r2t[r2t >= 0] += shift
    big["req_to_token"] = torch.from_numpy(r2t).to(DEV)
    B, Hq, D = inp["q"].shape
    announce("decode with a pool beyond 32-bit row offsets")
    outs = []
    for dev in (small, big):
        o = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
        tensors.run_decode(dev, o=o, lse=lse, workspace=tensors.decode_workspace(B, Hq, D, DEV, max_splits=7),
                           num_splits=7)
        torch.cuda.synchronize()
        outs.append((o, lse))
    del big
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    ref_o, ref_lse = oracle_of(inp)
    assert_close(outs[1][0], ref_o, "64-bit pool O")
    assert_close(outs[1][1], ref_lse, "64-bit pool lse", atol=1e-3, rtol=1e-4)


@pytest.mark.parametrize("scale", [0.03, 0.5])
def test_decode_other_softmax_scales(scale):
    seq = np.array([900, 5, 1300, 64])
    inp = build_paged_inputs(seq, 32, 8, 128, 4096, seed=33)
    inp["sm_scale"] = scale
    announce(f"decode sm_scale={scale}")
    o, lse, _, _ = _decode(inp, num_splits=5)
    ref_o, ref_lse = oracle_of(inp)
    assert_close(o, ref_o, f"scale {scale} O")
    assert_close(lse, ref_lse, f"scale {scale} lse", atol=1e-3, rtol=1e-4)


@pytest.mark.parametrize("ns", [0, 1, 7])
def test_decode_more_requests_than_one_kv_indptr_window(ns):
    """B = 2600 short requests: a work group's range spans more requests than
    one LDS window of kv_indptr holds (1023 pieces), so the window is
    re-staged mid-range; with one work group per head every request goes
    through the same work group."""
    rng = np.random.default_rng(2600 + ns)
    seq = rng.integers(1, 12, size=2600)
    seq[::97] = 300          # a few long requests among them
    inp = build_paged_inputs(seq, 8, 2, 64, 1 << 16, seed=17 + ns, flat_table=(ns == 7))
    announce(f"decode B=2600 windows num_splits={ns} N={int(seq.sum())}")
    o, lse, _, _ = _decode(inp, num_splits=ns)
    ref_o, ref_lse = oracle_of(inp)
    assert_close(o, ref_o, f"B=2600 ns={ns} O")
    assert_close(lse, ref_lse, f"B=2600 ns={ns} lse", atol=1e-3, rtol=1e-4)
