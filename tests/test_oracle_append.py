"""Pins for the KV-append oracle (oracle/kv_append.py).

Each test checks the oracle against something it does not compute itself:
hand-worked fixtures, pools that the input generator fills position by
position in flat key order (it never looks up req_to_token by request and
position), the one-key closed form of attention after an append, and untouched
slots keeping their bits.  A slip such as writing position L_b instead of
L_b - 1, taking the first instead of the last positions, using b * stride for a
flat table or mixing kv heads fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from paged_gqa_decode_astr_amd.workloads import BF16_QNAN, build_paged_inputs


def _bits(arr, Hkv):
    out = np.full((len(arr), Hkv, len(next(r for r in arr if r is not None)[0])), BF16_QNAN, dtype=np.uint16)
    for i, r in enumerate(arr):
        if r is None:
            continue
        f = np.asarray(r, dtype=np.float32)
        assert np.array_equal(f.astype(np.float64), np.asarray(r, dtype=np.float64))
        out[i] = (f.view(np.uint32) >> 16).astype(np.uint16)
    return out


def _new_bits(rows):
    f = np.asarray(rows, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_golden_fixtures(golden_dir):
    with open(os.path.join(golden_dir, "kv_append_examples.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        Hkv = c["num_kv_heads"]
        kp = _bits(c["k_pool"], Hkv)
        vp = _bits(c["v_pool"], Hkv)
        qo = None if c["qo_indptr"] is None else np.asarray(c["qo_indptr"], dtype=np.int32)
        k2, v2 = oracle.kv_append(kp, vp, _new_bits(c["k_new"]), _new_bits(c["v_new"]),
                                  np.asarray(c["req_to_token"], dtype=np.int32), c["req_to_token_stride"],
                                  np.asarray(c["kv_indptr"], dtype=np.int32), qo)
        assert np.array_equal(k2, _bits(c["k_pool_after"], Hkv)), c["name"]
        assert np.array_equal(v2, _bits(c["v_pool_after"], Hkv)), c["name"]
        # The inputs are not modified.
        assert np.array_equal(kp, _bits(c["k_pool"], Hkv))


@pytest.mark.parametrize("flat", [False, True])
@pytest.mark.parametrize("prefill", [False, True])
def test_matches_generator_full_pools(flat, prefill):
    """The generator stores every position by flat key index; appending the rows it held back must
    give exactly its fully stored pools (and NaN stays in every slot no request uses)."""
    rng = np.random.default_rng(5)
    B = 7
    seq = rng.integers(1, 40, B)
    n_new = np.ones(B, dtype=np.int64) if not prefill else np.minimum(seq, rng.integers(1, 9, B))
    inp = build_paged_inputs(seq, 4, 2, 8, 512, seed=11, flat_table=flat, new_tokens=n_new,
                             q_lens=n_new if prefill else None)
    qo = inp["qo_indptr"] if prefill else None
    k2, v2 = oracle.kv_append(inp["k_pool"], inp["v_pool"], inp["k_new"], inp["v_new"], inp["req_to_token"],
                              inp["req_to_token_stride"], inp["kv_indptr"], qo)
    assert np.array_equal(k2, inp["k_pool_full"])
    assert np.array_equal(v2, inp["v_pool_full"])
    if prefill:
        assert np.array_equal(inp["new_indptr"], inp["qo_indptr"])


def test_untouched_slots_keep_bits():
    inp = build_paged_inputs([5, 1, 9], 2, 1, 8, 64, seed=3, new_tokens=1)
    slots = oracle.new_token_slots(inp["req_to_token"], inp["req_to_token_stride"], inp["kv_indptr"])
    k2, v2 = oracle.kv_append(inp["k_pool"], inp["v_pool"], inp["k_new"], inp["v_new"], inp["req_to_token"],
                              inp["req_to_token_stride"], inp["kv_indptr"])
    keep = np.setdiff1d(np.arange(64), slots)
    assert np.array_equal(k2[keep], inp["k_pool"][keep])
    assert np.array_equal(v2[keep], inp["v_pool"][keep])
    # Before the append the new slots were unused (NaN); after it they hold the rows.
    assert np.all(inp["k_pool"][slots] == BF16_QNAN)
    assert np.array_equal(k2[slots], inp["k_new"])


def test_one_key_attention_returns_appended_row():
    """After appending the only token of a one-token request, attention over it returns the new V
    row exactly (closed form: a single visible key has weight one)."""
    inp = build_paged_inputs([1, 1, 1], 4, 2, 8, 32, seed=9, new_tokens=1)
    k2, v2 = oracle.kv_append(inp["k_pool"], inp["v_pool"], inp["k_new"], inp["v_new"], inp["req_to_token"],
                              inp["req_to_token_stride"], inp["kv_indptr"])
    o, _ = oracle.paged_attention(inp["q"], k2, v2, inp["req_to_token"], inp["req_to_token_stride"],
                                  inp["kv_indptr"], inp["sm_scale"])
    vnew = oracle.bf16_bits_to_f64(inp["v_new"])   # [B, Hkv, D]
    for h in range(4):
        assert np.array_equal(o[:, h, :], vnew[:, h // 2, :])


def test_rejects_bad_counts_and_shared_slots():
    inp = build_paged_inputs([3, 2], 2, 1, 8, 16, seed=1, new_tokens=1)
    with pytest.raises(ValueError):
        oracle.kv_append(inp["k_pool"], inp["v_pool"], inp["k_new"], inp["v_new"], inp["req_to_token"],
                         inp["req_to_token_stride"], inp["kv_indptr"], qo_indptr=np.array([0, 4, 5]))
    r2t = inp["req_to_token"].copy().reshape(2, -1)
    r2t[1, 1] = r2t[0, 2]   # both requests' last positions on one slot
    with pytest.raises(ValueError):
        oracle.new_token_slots(r2t.reshape(-1), inp["req_to_token_stride"], inp["kv_indptr"])
