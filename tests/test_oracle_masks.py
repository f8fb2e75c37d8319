"""Pins for the oracle's causal switch and boolean masks (oracle.paged_attention's non_causal / mask).

Checked against torch's fp64 scaled_dot_product_attention with the combined
boolean mask built here from the definition's three parts (causal rule, mask
row, key range), scalar brute force, closed forms (one visible key returns
its V row; non-causal rows equal decode over the whole sequence), and
invariants (an all-ones mask changes nothing; a 3-D mask with equal rows is
the 2-D mask; hiding a key equals dropping it from the page table; a row
with no visible key is zero with lse = -inf).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_gqa_decode_astr_amd.workloads import build_paged_inputs

RNG = np.random.default_rng(99)


def _case(B=4, Hq=4, Hkv=2, D=8, seq=(1, 24), prefill=True, seed=0, flat=False):
    seq_lens = RNG.integers(seq[0], seq[1] + 1, size=B)
    q_lens = np.array([RNG.integers(1, L + 1) for L in seq_lens]) if prefill else None
    return build_paged_inputs(seq_lens, Hq, Hkv, D, 256, seed, q_lens=q_lens, flat_table=flat)


def _rows(inp):
    kv = inp["kv_indptr"]
    B = len(kv) - 1
    qo = inp["qo_indptr"]
    for b in range(B):
        L = int(kv[b + 1] - kv[b])
        r0, qb = (b, 1) if qo is None else (int(qo[b]), int(qo[b + 1] - qo[b]))
        yield b, L, r0, qb


def _random_mask(inp, three_d, p=0.7):
    kv = inp["kv_indptr"]
    B = len(kv) - 1
    kv_len = int(np.diff(kv).max())
    qmax = 1 if inp["qo_indptr"] is None else int(np.diff(inp["qo_indptr"]).max())
    shape = (B, qmax, kv_len) if three_d else (B, kv_len)
    return (RNG.random(shape) < p).astype(np.uint8)


def _run(inp, **kw):
    return oracle.paged_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                  inp["req_to_token_stride"], inp["kv_indptr"], inp["sm_scale"],
                                  qo_indptr=inp["qo_indptr"], **kw)


@pytest.mark.parametrize("non_causal", [False, True])
@pytest.mark.parametrize("mask_kind", [None, "2d", "3d"])
def test_matches_torch_sdpa_fp64(non_causal, mask_kind):
    inp = _case(seed=3 + non_causal)
    mask = None if mask_kind is None else _random_mask(inp, mask_kind == "3d")
    o, lse = _run(inp, non_causal=non_causal, mask=mask)
    sig = float(np.float32(inp["sm_scale"]))
    Hq, Hkv = inp["num_qo_heads"], inp["num_kv_heads"]
    for b, L, r0, qb in _rows(inp):
        sl = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], inp["kv_indptr"], b)
        K = torch.from_numpy(oracle.bf16_bits_to_f64(inp["k_pool"][sl])).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        V = torch.from_numpy(oracle.bf16_bits_to_f64(inp["v_pool"][sl])).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        Q = torch.from_numpy(oracle.bf16_bits_to_f64(inp["q"][r0:r0 + qb])).permute(1, 0, 2)
        vis = torch.ones(qb, L, dtype=torch.bool)
        if not non_causal:
            vis &= torch.arange(L)[None, :] <= (L - qb + torch.arange(qb))[:, None]
        if mask is not None:
            mrow = torch.from_numpy(mask[b, :L][None, :] if mask.ndim == 2 else mask[b, :qb, :L]) != 0
            vis &= mrow
        ok = vis.any(dim=1)
        if ok.any():
            ref = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=vis,
                                                                   scale=sig)[0].permute(1, 0, 2).numpy()
            np.testing.assert_allclose(o[r0:r0 + qb][ok.numpy()], ref[ok.numpy()], atol=1e-12, rtol=0)
            logits = (Q @ K.transpose(1, 2)) * sig
            ref_lse = torch.logsumexp(logits.masked_fill(~vis[None], float("-inf")), -1).T.numpy()
            np.testing.assert_allclose(lse[r0:r0 + qb][ok.numpy()], ref_lse[ok.numpy()], atol=1e-12)
        if (~ok).any():
            assert np.all(o[r0:r0 + qb][~ok.numpy()] == 0.0)
            assert np.all(np.isneginf(lse[r0:r0 + qb][~ok.numpy()]))


def test_brute_force_loops_with_mask():
    inp = _case(B=3, D=4, seq=(1, 8), seed=12)
    mask = _random_mask(inp, True, p=0.6)
    o, lse = _run(inp, mask=mask)
    sig = float(np.float32(inp["sm_scale"]))
    for b, L, r0, qb in _rows(inp):
        sl = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], inp["kv_indptr"], b)
        K = oracle.bf16_bits_to_f64(inp["k_pool"][sl]).tolist()
        V = oracle.bf16_bits_to_f64(inp["v_pool"][sl]).tolist()
        for i in range(qb):
            qrow = oracle.bf16_bits_to_f64(inp["q"][r0 + i]).tolist()
            keys = [t for t in range(L) if t <= L - qb + i and mask[b, i, t]]
            for h in range(4):
                g = h // 2
                if not keys:
                    assert all(x == 0.0 for x in o[r0 + i, h]) and lse[r0 + i, h] == -math.inf
                    continue
                s = {t: sig * sum(qrow[h][d] * K[t][g][d] for d in range(4)) for t in keys}
                mx = max(s.values())
                e = {t: math.exp(s[t] - mx) for t in keys}
                tot = sum(e.values())
                ref = [sum(e[t] * V[t][g][d] for t in keys) / tot for d in range(4)]
                np.testing.assert_allclose(o[r0 + i, h], ref, atol=1e-13)
                assert lse[r0 + i, h] == pytest.approx(mx + math.log(tot), abs=1e-13)


def test_single_visible_key_returns_its_v_row():
    inp = _case(B=5, Hq=4, Hkv=1, prefill=False, seq=(3, 20), seed=5)
    kv = inp["kv_indptr"]
    mask = np.zeros((5, int(np.diff(kv).max())), np.uint8)
    keep = [int(RNG.integers(0, int(kv[b + 1] - kv[b]))) for b in range(5)]
    for b, t in enumerate(keep):
        mask[b, t] = 1
    o, _ = _run(inp, mask=mask)
    for b, t in enumerate(keep):
        slot = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], kv, b)[t]
        v = oracle.bf16_bits_to_f64(inp["v_pool"][slot][0])
        for h in range(4):
            assert np.array_equal(o[b, h], v)


def test_non_causal_rows_equal_decode_over_the_whole_sequence():
    inp = _case(B=3, seed=6)
    o, lse = _run(inp, non_causal=True)
    for b, L, r0, qb in _rows(inp):
        for i in range(qb):
            one = dict(inp)
            one["q"] = inp["q"][r0 + i][None]
            one["kv_indptr"] = np.array([0, L], np.int32)
            sl = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], inp["kv_indptr"], b)
            one["req_to_token"] = sl.astype(np.int32)
            one["req_to_token_stride"] = 0
            one["qo_indptr"] = None
            od, ld = _run(one)   # one query row: the matrix products round differently, hence 1e-13
            np.testing.assert_allclose(o[r0 + i], od[0], atol=1e-13, rtol=0)
            np.testing.assert_allclose(lse[r0 + i], ld[0], atol=1e-13, rtol=0)


def test_all_ones_and_equal_rows_invariants():
    inp = _case(B=4, seed=8)
    base_o, base_lse = _run(inp)
    kv_len = int(np.diff(inp["kv_indptr"]).max())
    qmax = int(np.diff(inp["qo_indptr"]).max())
    o1, l1 = _run(inp, mask=np.ones((4, kv_len), np.uint8))
    assert np.array_equal(o1, base_o) and np.array_equal(l1, base_lse)
    m2 = _random_mask(inp, False)
    o2, l2 = _run(inp, mask=m2)
    o3, l3 = _run(inp, mask=np.repeat(m2[:, None, :], qmax, axis=1))
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3)


def test_hiding_a_key_equals_dropping_it_from_the_table():
    inp = _case(B=3, Hq=4, Hkv=2, prefill=False, seq=(4, 30), seed=9)
    kv = inp["kv_indptr"]
    mask = np.ones((3, int(np.diff(kv).max())), np.uint8)
    drop = [1, 0, 2]
    for b, t in enumerate(drop):
        mask[b, t] = 0
    o, lse = _run(inp, mask=mask)
    rows, lens = [], []
    for b, t in enumerate(drop):
        sl = list(oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], kv, b))
        del sl[t]
        rows += sl
        lens.append(len(sl))
    short = dict(inp)
    short["req_to_token"] = np.asarray(rows, np.int32)
    short["req_to_token_stride"] = 0
    short["kv_indptr"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o2, lse2 = _run(short)
    np.testing.assert_allclose(o, o2, atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse, lse2, atol=1e-14, rtol=0)


def test_fully_masked_rows_are_zero_with_neg_inf_lse():
    inp = _case(B=2, seed=10)
    kv_len = int(np.diff(inp["kv_indptr"]).max())
    o, lse = _run(inp, mask=np.zeros((2, kv_len), np.uint8))
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))
