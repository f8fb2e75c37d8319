"""GPU parity of the causal switch, 2-D / 3-D boolean masks and head-major layouts.

Every call goes through the C ABI; expected values come from the fp64 oracle
with the same mask (oracle.paged_attention's non_causal / mask).  Masks are
seeded uint8 arrays with kv_len padded to a multiple of 4 (the ABI's
alignment rule); padding entries are random too, so a read past a request's
keys would show.
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


def _mask(inp, three_d, p, seed):
    rng = np.random.default_rng(seed)
    kv = inp["kv_indptr"]
    B = len(kv) - 1
    kv_len = (int(np.diff(kv).max()) + 3) // 4 * 4
    qmax = 1 if inp.get("qo_indptr") is None else int(np.diff(inp["qo_indptr"]).max())
    shape = (B, qmax, kv_len) if three_d else (B, kv_len)
    return (rng.random(shape) < p).astype(np.uint8)


def _oracle(inp, mask=None, non_causal=False):
    return oracle.paged_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                  inp["req_to_token_stride"], inp["kv_indptr"], inp["sm_scale"],
                                  qo_indptr=inp.get("qo_indptr"), non_causal=non_causal, mask=mask)


def _check(o, lse, ref_o, ref_lse, what, ulp_check=True):
    """Rows with visible keys within tolerance; rows without are exact zeros with lse = -inf.

    Prefill (ulp_check False) rounds its softmax weights to bf16 for the P.V product, so its lse is
    held to 2e-3, as in the unmasked prefill tests; decode to 1e-3."""
    empty = np.isneginf(ref_lse)
    got_o = tensors.bf16_to_f64(o)
    got_l = lse.double().cpu().numpy()
    assert np.all(got_o[empty] == 0.0), f"{what}: rows with no visible key are not zero"
    assert np.all(np.isneginf(got_l[empty])), f"{what}: lse of rows with no visible key is not -inf"
    ref_o2 = np.where(empty[..., None], 0.0, ref_o)
    assert_close(o, ref_o2, f"{what} O", ulp_check=ulp_check)
    keep = ~empty
    np.testing.assert_allclose(got_l[keep], ref_lse[keep], atol=1e-3 if ulp_check else 2e-3, rtol=1e-4,
                               err_msg=f"{what} lse")


def _decode(inp, mask_t, num_splits=0, fused=False):
    dev = tensors.to_device(inp, DEV)
    B, Hq, D = inp["q"].shape
    o = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    ws = tensors.decode_workspace(B, Hq, D, DEV, max_splits=max(num_splits, 0))
    run = tensors.run_decode_append if fused else tensors.run_decode
    run(dev, o=o, lse=lse, workspace=ws, num_splits=num_splits, mask=mask_t)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("three_d", [False, True])
@pytest.mark.parametrize("cid", ["tiny", "decode_b32", "ragged_b256"])
def test_decode_mask_configs(cid, three_d):
    inp = make_inputs(cid, 2)
    mask = _mask(inp, three_d, 0.6, seed={"tiny": 1, "decode_b32": 2, "ragged_b256": 3}[cid] * 10 + three_d)
    announce(f"decode mask {cid} 3d={three_d}")
    o, lse = _decode(inp, torch.from_numpy(mask).to(DEV))
    ref_o, ref_lse = _oracle(inp, mask)
    _check(o, lse, ref_o, ref_lse, f"{cid} mask")


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 1, 64), (8, 4, 64), (16, 2, 128), (8, 8, 128), (64, 8, 128)])
def test_decode_mask_variants_and_splits(Hq, Hkv, D):
    seq = np.array([1, 2, 15, 16, 17, 33, 64, 65, 128, 129, 130, 300, 1, 511, 2, 700])
    inp = build_paged_inputs(seq, Hq, Hkv, D, 8192, seed=Hq * 3 + D)
    mask = _mask(inp, False, 0.5, seed=D + Hq)
    mask[3, :] = 0                    # a request with every key hidden
    mask[5, :] = 0
    mask[5, 20] = 1                   # ... and one with a single visible key
    ref_o, ref_lse = _oracle(inp, mask)
    mt = torch.from_numpy(mask).to(DEV)
    for ns in (0, 1, 3, 16, 200):
        announce(f"decode mask Hq={Hq} Hkv={Hkv} D={D} num_splits={ns}")
        o, lse = _decode(inp, mt, num_splits=ns)
        _check(o, lse, ref_o, ref_lse, f"variant ns={ns}")
        slot = int(oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], inp["kv_indptr"], 5)[20])
        got = o[5].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, inp["v_pool"][slot][np.arange(Hq) // (Hq // Hkv)])


def test_decode_all_ones_mask_is_bit_identical_to_no_mask():
    inp = make_inputs("decode_b32", 1)
    ones = torch.ones(32, 2048, dtype=torch.uint8, device=DEV)
    announce("decode all-ones mask")
    o1, l1 = _decode(inp, ones)
    o0, l0 = _decode(inp, None)
    assert torch.equal(o1.view(torch.int16), o0.view(torch.int16))
    assert torch.equal(l1, l0)


def test_decode_append_with_mask_matches_separate():
    inp = make_inputs("decode_b32", 0, new_tokens=1)
    mask = _mask(inp, False, 0.7, seed=5)
    mt = torch.from_numpy(mask).to(DEV)
    announce("decode_append with mask")
    of, lf = _decode(inp, mt, fused=True)
    dev = tensors.to_device(inp, DEV)
    tensors.run_append(dev)
    B, Hq, D = inp["q"].shape
    o = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    tensors.run_decode(dev, o=o, lse=lse, workspace=tensors.decode_workspace(B, Hq, D, DEV), mask=mt)
    torch.cuda.synchronize()
    assert torch.equal(of.view(torch.int16), o.view(torch.int16))
    assert torch.equal(lf.view(torch.int32), lse.view(torch.int32))


def _prefill(inp, mask_t=None, non_causal=False, max_q_len=0):
    dev = tensors.to_device(inp, DEV)
    rows, Hq, D = inp["q"].shape
    o = torch.empty(rows, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(rows, Hq, dtype=torch.float32, device=DEV)
    tensors.run_prefill(dev, o=o, lse=lse, mask=mask_t, non_causal=non_causal, max_q_len=max_q_len)
    torch.cuda.synchronize()
    return o, lse


def _prefill_case(seed, B=6, Hq=32, Hkv=8, D=128, qmax=300, prefix=900):
    rng = np.random.default_rng(seed)
    q_lens = rng.integers(1, qmax, size=B)
    q_lens[1] = 1
    seq = q_lens + rng.integers(0, prefix, size=B)
    seq[2] = q_lens[2]
    return build_paged_inputs(seq, Hq, Hkv, D, 1 << 14, seed=seed, q_lens=q_lens)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 8, 128), (16, 2, 64), (8, 1, 64)])
def test_prefill_non_causal(Hq, Hkv, D):
    inp = _prefill_case(31 + D + Hq, Hq=Hq, Hkv=Hkv, D=D)
    announce(f"prefill non-causal Hq={Hq} Hkv={Hkv} D={D}")
    o, lse = _prefill(inp, non_causal=True)
    ref_o, ref_lse = _oracle(inp, non_causal=True)
    _check(o, lse, ref_o, ref_lse, "non-causal", ulp_check=False)


@pytest.mark.parametrize("three_d", [False, True])
@pytest.mark.parametrize("non_causal", [False, True])
def test_prefill_masks(three_d, non_causal):
    inp = _prefill_case(50 + 2 * three_d + non_causal)
    mask = _mask(inp, three_d, 0.6, seed=7 + three_d)
    if three_d:
        mask[0, 3, :] = 0             # a query row with every key hidden
    else:
        mask[4, :] = 0                # a request with every key hidden
    announce(f"prefill mask 3d={three_d} non_causal={non_causal}")
    o, lse = _prefill(inp, torch.from_numpy(mask).to(DEV), non_causal=non_causal)
    ref_o, ref_lse = _oracle(inp, mask, non_causal=non_causal)
    _check(o, lse, ref_o, ref_lse, f"prefill mask 3d={three_d} nc={non_causal}", ulp_check=False)


def test_prefill_mask_variants_and_fixed_grid():
    for Hq, Hkv, D in [(8, 1, 64), (16, 2, 64), (32, 4, 128), (64, 8, 128)]:
        inp = _prefill_case(80 + Hq, Hq=Hq, Hkv=Hkv, D=D, qmax=140, prefix=300)
        mask = _mask(inp, True, 0.5, seed=Hq)
        announce(f"prefill 3-D mask Hq={Hq} Hkv={Hkv} D={D} fixed grid")
        o, lse = _prefill(inp, torch.from_numpy(mask).to(DEV), max_q_len=200)
        ref_o, ref_lse = _oracle(inp, mask)
        _check(o, lse, ref_o, ref_lse, f"prefill mask Hq={Hq} D={D}", ulp_check=False)


@pytest.mark.parametrize("three_d,non_causal", [(False, False), (True, False), (True, True), (None, True)])
def test_prefill_head_dim_256_masks_and_grids(three_d, non_causal):
    """head_dim 256 prefill (8 wavefronts of one 16-row block each) with 2-D / 3-D masks and the
    non-causal switch, on the work-list grid (split plan) and on the fixed grid."""
    inp = _prefill_case(300 + 3 * (three_d is True) + 2 * (three_d is False) + non_causal, Hq=16, Hkv=4, D=256,
                        qmax=140, prefix=300)
    mask = None if three_d is None else _mask(inp, three_d, 0.6, seed=31 + (three_d is True))
    if three_d:
        mask[0, 3, :] = 0             # a query row with every key hidden
    mt = None if mask is None else torch.from_numpy(mask).to(DEV)
    ref_o, ref_lse = _oracle(inp, mask, non_causal=non_causal)
    for mq in (0, 200):
        announce(f"prefill head_dim 256 mask 3d={three_d} non_causal={non_causal} max_q_len={mq}")
        o, lse = _prefill(inp, mt, non_causal=non_causal, max_q_len=mq)
        _check(o, lse, ref_o, ref_lse, f"D256 prefill mask 3d={three_d} nc={non_causal} grid={mq}", ulp_check=False)


def test_prefill_all_ones_mask_matches_no_mask():
    """An all-ones mask hides nothing: the masked kernel (every tile through the mask code) agrees with
    the oracle run without a mask.  (It is a different kernel from the unmasked one and rounds its bf16
    softmax weights on its own, so the two are compared through the oracle, not bit for bit.)"""
    inp = make_inputs("prefill_b8", 1)
    qmax = int(np.diff(inp["qo_indptr"]).max())
    ones = torch.ones(8, qmax, 2564, dtype=torch.uint8, device=DEV)
    announce("prefill all-ones mask")
    o1, l1 = _prefill(inp, ones)
    ref_o, ref_lse = _oracle(inp)
    _check(o1, l1, ref_o, ref_lse, "all-ones mask", ulp_check=False)


def test_head_major_layouts():
    """Pools stored head-major ([Hkv, slots, D], the pages' "bhld") and prefill q / o stored head-major
    ([Hq, rows, D]), passed as strided views: results are bit-identical to the token-major layout."""
    inp = _prefill_case(90, B=4, qmax=200, prefix=500)
    dev = tensors.to_device(inp, DEV)
    rows, Hq, D = inp["q"].shape
    hm = dict(dev)
    hm["k_pool"] = dev["k_pool"].permute(1, 0, 2).contiguous().permute(1, 0, 2)
    hm["v_pool"] = dev["v_pool"].permute(1, 0, 2).contiguous().permute(1, 0, 2)
    hm["q"] = dev["q"].permute(1, 0, 2).contiguous().permute(1, 0, 2)
    assert hm["k_pool"].stride() == (D, dev["k_pool"].shape[0] * D, 1)
    announce("head-major layouts: prefill and decode")
    outs = []
    for d in (dev, hm):
        o = torch.empty(Hq, rows, D, dtype=torch.bfloat16, device=DEV).permute(1, 0, 2) if d is hm \
            else torch.empty(rows, Hq, D, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(rows, Hq, dtype=torch.float32, device=DEV)
        tensors.run_prefill(d, o=o, lse=lse)
        torch.cuda.synchronize()
        outs.append((o, lse))
    assert torch.equal(outs[0][0].contiguous().view(torch.int16), outs[1][0].contiguous().view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    # Decode over the same head-major pools (one query row per request).
    dinp = build_paged_inputs(np.array([700, 1, 64, 1500]), 32, 8, 128, 1 << 14, seed=91)
    dd = tensors.to_device(dinp, DEV)
    dh = dict(dd)
    dh["k_pool"] = dd["k_pool"].permute(1, 0, 2).contiguous().permute(1, 0, 2)
    dh["v_pool"] = dd["v_pool"].permute(1, 0, 2).contiguous().permute(1, 0, 2)
    r = []
    for d in (dd, dh):
        o = tensors.run_decode(d, workspace=tensors.decode_workspace(4, 32, 128, DEV))
        torch.cuda.synchronize()
        r.append(o)
    assert torch.equal(r[0].view(torch.int16), r[1].view(torch.int16))


@pytest.mark.parametrize("P,ns", [(1, 0), (1, 5), (16, 0), (64, 3)])
def test_decode_gather_indices_exact(P, ns):
    """Gather indices, bit for bit: every V row holds its own slot id
    (slot = v[0] + 256 * v[1], kv head = v[2]; integers below 256 are exact in
    bf16), and a mask leaves one key t_b of each request visible, whose
    weight is then exactly 1.  So each output row is the V row the kernel
    gathered for position t_b, and it must name the oracle's slot for it
    (req_to_token lookup, page arithmetic and all)."""
    rng = np.random.default_rng(700 + P + ns)
    seq = rng.integers(1, 1500, size=24)
    seq[:3] = [1, 2, P + 1]
    inp = build_paged_inputs(seq, 16, 4, 128, 1 << 16, seed=P * 10 + ns, page_size=P)
    S = inp["v_pool"].shape[0]
    v = np.zeros((S, 4, 128), np.float32)
    v[:, :, 0] = np.arange(S)[:, None] % 256
    v[:, :, 1] = np.arange(S)[:, None] // 256
    v[:, :, 2] = np.arange(4)[None, :]
    inp["v_pool"] = (v.view(np.uint32) >> 16).astype(np.uint16)
    dev = tensors.to_device(inp, DEV)
    kv = inp["kv_indptr"]
    ws = tensors.decode_workspace(24, 16, 128, DEV, max_splits=ns)
    for trial in range(6):
        t = np.array([rng.integers(0, kv[b + 1] - kv[b]) for b in range(24)])
        t[0] = 0
        mask = np.zeros((24, (int(seq.max()) + 3) // 4 * 4), np.uint8)   # row stride: a multiple of 4 bytes
        mask[np.arange(24), t] = 1
        announce(f"gather indices page_size={P} num_splits={ns} trial {trial}")
        o = tensors.run_decode(dev, workspace=ws, num_splits=ns, mask=torch.from_numpy(mask).to(DEV))
        torch.cuda.synchronize()
        got = o.float().cpu().numpy()
        for b in range(24):
            want = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], kv, b, page_size=P)[t[b]]
            for h in range(16):
                row = got[b, h]
                assert row[0] + 256 * row[1] == want and row[2] == h // 4, (b, h, t[b], row[:3], want)
                assert np.all(row[3:] == 0)


@pytest.mark.parametrize("P", [1, 16])
def test_prefill_gather_indices_exact(P):
    """The prefill gather (slot ids -> LDS tiles) bit for bit: V rows hold
    their own slot ids, and a 3-D mask leaves one causally visible key t per
    query row, whose weight is then exactly 1 (also after rounding to bf16),
    so each output row names the slot gathered for (b, t)."""
    rng = np.random.default_rng(900 + P)
    q_lens = rng.integers(1, 200, size=6)
    seq = q_lens + rng.integers(0, 700, size=6)
    inp = build_paged_inputs(seq, 16, 4, 128, 1 << 15, seed=950 + P, q_lens=q_lens, page_size=P)
    S = inp["v_pool"].shape[0]
    v = np.zeros((S, 4, 128), np.float32)
    v[:, :, 0] = np.arange(S)[:, None] % 256
    v[:, :, 1] = np.arange(S)[:, None] // 256
    v[:, :, 2] = np.arange(4)[None, :]
    inp["v_pool"] = (v.view(np.uint32) >> 16).astype(np.uint16)
    dev = tensors.to_device(inp, DEV)
    kv, qo = inp["kv_indptr"], inp["qo_indptr"]
    cols = (int(seq.max()) + 3) // 4 * 4      # row stride: a multiple of 4 bytes
    mask = np.zeros((6, int(q_lens.max()), cols), np.uint8)
    pick = {}
    for b in range(6):
        L, ql = int(kv[b + 1] - kv[b]), int(q_lens[b])
        for i in range(ql):
            t = int(rng.integers(0, L - ql + i + 1))   # within the causal limit of row i
            mask[b, i, t] = 1
            pick[(b, i)] = t
    announce(f"prefill gather indices page_size={P}")
    o = tensors.run_prefill(dev, mask=torch.from_numpy(mask).to(DEV))
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    for b in range(6):
        slots = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], kv, b, page_size=P)
        for i in range(int(q_lens[b])):
            want = slots[pick[(b, i)]]
            rows = got[int(qo[b]) + i]
            assert np.all(rows[:, 0] + 256 * rows[:, 1] == want), (b, i, rows[:, :2], want)
            assert np.all(rows[:, 2] == np.arange(16) // 4) and np.all(rows[:, 3:] == 0)
