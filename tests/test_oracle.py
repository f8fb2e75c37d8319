"""Pins for the CPU oracle: closed forms, a library routine, brute force, invariants, fixtures.

Each test checks the oracle against something other than itself, chosen so
that a plausible slip (dropped scale, wrong kv-head map, causal off-by-one,
wrong row base, missing max subtraction, transposed operand) fails at least
one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from paged_gqa_decode_astr_amd.workloads import build_paged_inputs, make_inputs

RNG = np.random.default_rng(1234)


def f64_to_bits_exact(x):
    """Bits of values that are exactly representable in bf16 (asserted)."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), x, equal_nan=True)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), x, equal_nan=True), "value not bf16-exact"
    return bits


def _load_golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as fh:
        return json.load(fh)


def _pool_from_json(rows, D, Hkv):
    arr = np.full((len(rows), Hkv, D), np.nan)
    for i, r in enumerate(rows):
        if r is not None:
            arr[i] = np.asarray(r, dtype=np.float64)
    return f64_to_bits_exact(arr)


# --------------------------------------------------------------------------- bf16 helpers

def test_bf16_widen_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_bits_to_f64(bits)
    assert np.array_equal(got, ref, equal_nan=True)


def test_bf16_round_matches_torch_rne():
    x = RNG.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    x = np.concatenate([x, np.float32([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8,
                                       2.0 ** -130, 3.3895314e38, 0.0, -0.0])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)
    # ties to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert oracle.f64_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert oracle.f64_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82


# --------------------------------------------------------------------------- hand-worked fixtures

def test_golden_attention_examples(golden_dir):
    data = _load_golden(golden_dir, "attention_examples.json")
    for case in data["cases"]:
        Hkv = case["num_kv_heads"]
        D = len(case["q"][0][0])
        k_pool = _pool_from_json(case["k_pool"], D, Hkv)
        v_pool = _pool_from_json(case["v_pool"], D, Hkv)
        q = f64_to_bits_exact(np.asarray(case["q"], dtype=np.float64))
        qo = None if case["qo_indptr"] is None else np.asarray(case["qo_indptr"], np.int32)
        mask = None if case.get("mask") is None else np.asarray(case["mask"], np.uint8)
        o, lse = oracle.paged_attention(q, k_pool, v_pool, np.asarray(case["req_to_token"], np.int32),
                                        case["req_to_token_stride"], np.asarray(case["kv_indptr"], np.int32),
                                        case["sm_scale"], qo_indptr=qo, non_causal=case.get("non_causal", False),
                                        mask=mask)
        assert np.array_equal(o, np.asarray(case["o"], dtype=np.float64)), case["name"]
        want = np.asarray([[-np.inf if x is None else x for x in r] for r in case["lse"]])
        np.testing.assert_allclose(lse, want, rtol=0, atol=1e-14, err_msg=case["name"])


def test_golden_partition_examples(golden_dir):
    data = _load_golden(golden_dir, "partition_examples.json")
    for case in data["cases"]:
        kv = case["kv_indptr"]
        Wh = case["Wh"]
        assert [list(p) for p in oracle.piece_table(kv, Wh)] == case["pieces"]
        for b, exp in enumerate(case["request_pieces"]):
            assert list(oracle.pieces_of_request(kv, Wh, b)) == exp


# --------------------------------------------------------------------------- closed forms

def _random_case(B=3, Hq=4, Hkv=2, D=8, seq=(1, 9), q_lens=None, slots=64, seed=0, flat=False):
    seq_lens = RNG.integers(seq[0], seq[1] + 1, size=B)
    if q_lens == "random":
        q_lens = np.array([RNG.integers(1, L + 1) for L in seq_lens])
    return build_paged_inputs(seq_lens, Hq, Hkv, D, slots, seed, q_lens=q_lens, flat_table=flat)


def _run(inp, **kw):
    return oracle.paged_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                  inp["req_to_token_stride"], inp["kv_indptr"], kw.get("sm_scale", inp["sm_scale"]),
                                  qo_indptr=inp["qo_indptr"])


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (4, 2), (8, 2), (3, 3)])
def test_single_key_returns_v_exactly(Hq, Hkv):
    """One visible key has weight exactly 1, so O is that key's V row for the right kv head."""
    inp = build_paged_inputs(np.ones(5, np.int64), Hq, Hkv, 16, 40, seed=11)
    o, lse = _run(inp)
    group = Hq // Hkv
    sigma = float(np.float32(inp["sm_scale"]))
    for b in range(5):
        slot = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], inp["kv_indptr"], b)[0]
        for h in range(Hq):
            v = oracle.bf16_bits_to_f64(inp["v_pool"][slot, h // group])
            k = oracle.bf16_bits_to_f64(inp["k_pool"][slot, h // group])
            qv = oracle.bf16_bits_to_f64(inp["q"][b, h])
            assert np.array_equal(o[b, h], v)
            assert lse[b, h] == pytest.approx(sigma * float(qv @ k), abs=1e-12)


def test_identical_keys_and_zero_query_give_mean_v():
    inp = build_paged_inputs(np.array([7, 3, 12]), 4, 2, 8, 64, seed=5)
    # Make all keys of each request identical (copy position 0's row).
    for b in range(3):
        sl = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], inp["kv_indptr"], b)
        inp["k_pool"][sl] = inp["k_pool"][sl[0]]
    o, lse = _run(inp)
    zq = dict(inp)
    zq["q"] = np.zeros_like(inp["q"])
    o0, lse0 = _run(zq)
    for b in range(3):
        sl = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], inp["kv_indptr"], b)
        L = len(sl)
        for h in range(4):
            mean_v = oracle.bf16_bits_to_f64(inp["v_pool"][sl, h // 2]).mean(axis=0)
            np.testing.assert_allclose(o[b, h], mean_v, atol=1e-14)
            np.testing.assert_allclose(o0[b, h], mean_v, atol=1e-14)
            assert lse0[b, h] == pytest.approx(math.log(L), abs=1e-14)


def test_two_keys_sigmoid_weights_with_scale():
    """Two keys: weight of key 1 is sigmoid(s1 - s0) with s = sm_scale * q.k."""
    inp = build_paged_inputs(np.array([2, 2]), 2, 1, 32, 16, seed=9)
    for scale in (1.0 / math.sqrt(32), 0.3, 2.0):
        o, lse = _run(inp, sm_scale=scale)
        sig = float(np.float32(scale))
        for b in range(2):
            sl = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], inp["kv_indptr"], b)
            K = oracle.bf16_bits_to_f64(inp["k_pool"][sl, 0])
            V = oracle.bf16_bits_to_f64(inp["v_pool"][sl, 0])
            for h in range(2):
                qv = oracle.bf16_bits_to_f64(inp["q"][b, h])
                s0, s1 = sig * (qv @ K[0]), sig * (qv @ K[1])
                w1 = 1.0 / (1.0 + math.exp(s0 - s1))
                np.testing.assert_allclose(o[b, h], (1 - w1) * V[0] + w1 * V[1], atol=1e-13)
                assert lse[b, h] == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))), abs=1e-12)


def test_large_logits_do_not_overflow():
    """Logits near 1e4 would overflow exp() without the max shift; the answer is the arg-max V."""
    inp = build_paged_inputs(np.array([3]), 1, 1, 4, 8, seed=3)
    sl = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], inp["kv_indptr"], 0)
    inp["q"][0, 0] = f64_to_bits_exact([64.0, 0, 0, 0])
    for i, kv in enumerate([100.0, 256.0, -256.0]):
        inp["k_pool"][sl[i], 0] = f64_to_bits_exact([kv, 0, 0, 0])
    o, lse = _run(inp, sm_scale=1.0)
    V = oracle.bf16_bits_to_f64(inp["v_pool"][sl, 0])
    assert np.all(np.isfinite(o))
    np.testing.assert_allclose(o[0, 0], V[1], atol=1e-12)      # weight of key 0 is e^-9984
    assert lse[0, 0] == pytest.approx(64.0 * 256.0, abs=1e-9)


# --------------------------------------------------------------------------- library routine and brute force

@pytest.mark.parametrize("kind", ["decode", "prefill"])
@pytest.mark.parametrize("Hq,Hkv,D", [(4, 1, 8), (8, 2, 16), (6, 3, 8)])
def test_matches_torch_sdpa_fp64(kind, Hq, Hkv, D):
    """torch's fp64 SDPA on gathered keys, heads expanded by repeat-interleave, explicit causal mask."""
    q_lens = "random" if kind == "prefill" else None
    inp = _random_case(B=4, Hq=Hq, Hkv=Hkv, D=D, seq=(1, 20), q_lens=q_lens, slots=128, seed=21)
    o, lse = _run(inp)
    sig = float(np.float32(inp["sm_scale"]))
    kv = inp["kv_indptr"]
    for b in range(4):
        L = int(kv[b + 1] - kv[b])
        r0, qb = (b, 1) if inp["qo_indptr"] is None else (int(inp["qo_indptr"][b]),
                                                          int(inp["qo_indptr"][b + 1] - inp["qo_indptr"][b]))
        sl = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], kv, b)
        K = torch.from_numpy(oracle.bf16_bits_to_f64(inp["k_pool"][sl])).permute(1, 0, 2)   # [Hkv, L, D]
        V = torch.from_numpy(oracle.bf16_bits_to_f64(inp["v_pool"][sl])).permute(1, 0, 2)
        Q = torch.from_numpy(oracle.bf16_bits_to_f64(inp["q"][r0:r0 + qb])).permute(1, 0, 2)  # [Hq, qb, D]
        K = K.repeat_interleave(Hq // Hkv, dim=0)
        V = V.repeat_interleave(Hq // Hkv, dim=0)
        mask = torch.arange(L)[None, :] <= (L - qb + torch.arange(qb))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=mask,
                                                               scale=sig)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(o[r0:r0 + qb], ref, atol=1e-12, rtol=0)
        logits = torch.einsum("hqd,hkd->hqk", Q, K) * sig
        logits = logits.masked_fill(~mask[None], float("-inf"))
        np.testing.assert_allclose(lse[r0:r0 + qb], torch.logsumexp(logits, -1).T.numpy(), atol=1e-12)


def test_brute_force_loops_tiny():
    """Scalar triple loops over a contiguous copy of each request's keys."""
    inp = _random_case(B=3, Hq=4, Hkv=2, D=8, seq=(1, 9), q_lens="random", slots=40, seed=8)
    o, lse = _run(inp)
    sig = float(np.float32(inp["sm_scale"]))
    kv = inp["kv_indptr"]
    qo = inp["qo_indptr"]
    for b in range(3):
        sl = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], kv, b)
        K = oracle.bf16_bits_to_f64(inp["k_pool"][sl]).tolist()
        V = oracle.bf16_bits_to_f64(inp["v_pool"][sl]).tolist()
        L = len(sl)
        qb = int(qo[b + 1] - qo[b])
        for i in range(qb):
            qrow = oracle.bf16_bits_to_f64(inp["q"][int(qo[b]) + i]).tolist()
            last = L - qb + i
            for h in range(4):
                g = h // 2
                s = [sig * sum(qrow[h][d] * K[t][g][d] for d in range(8)) for t in range(last + 1)]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = sum(e)
                ref = [sum(e[t] * V[t][g][d] for t in range(last + 1)) / tot for d in range(8)]
                np.testing.assert_allclose(o[int(qo[b]) + i, h], ref, atol=1e-13)
                assert lse[int(qo[b]) + i, h] == pytest.approx(mx + math.log(tot), abs=1e-13)


# --------------------------------------------------------------------------- invariants

def test_slot_permutation_is_bit_identical():
    """Moving K/V rows to other slots and remapping the table changes no output bit."""
    inp = _random_case(B=5, Hq=8, Hkv=2, D=16, seq=(1, 30), slots=256, seed=4)
    o, lse = _run(inp)
    perm = RNG.permutation(256)             # new slot of old slot s is perm[s]
    moved = dict(inp)
    moved["k_pool"] = np.empty_like(inp["k_pool"])
    moved["v_pool"] = np.empty_like(inp["v_pool"])
    moved["k_pool"][perm] = inp["k_pool"]
    moved["v_pool"][perm] = inp["v_pool"]
    r2t = inp["req_to_token"].copy()
    r2t[r2t >= 0] = perm[r2t[r2t >= 0]]
    moved["req_to_token"] = r2t
    o2, lse2 = _run(moved)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_flat_and_2d_tables_agree():
    seq_lens = np.array([5, 1, 17, 9])
    a = build_paged_inputs(seq_lens, 4, 2, 8, 64, seed=6, flat_table=False, row_stride=20)
    b = build_paged_inputs(seq_lens, 4, 2, 8, 64, seed=6, flat_table=True)
    oa, la = _run(a)
    ob, lb = _run(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_unused_slots_poisoned_do_not_leak():
    inp = _random_case(B=4, Hq=4, Hkv=1, D=8, seq=(1, 12), q_lens="random", slots=80, seed=2)
    assert np.isnan(oracle.bf16_bits_to_f64(inp["k_pool"])).any()
    o, lse = _run(inp)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_prefill_rows_equal_decode_on_truncated_sequence():
    """Prefill row i of request b equals decode over that request's first c_b + i + 1 keys."""
    inp = _random_case(B=3, Hq=4, Hkv=2, D=8, seq=(2, 15), q_lens="random", slots=64, seed=12)
    o, lse = _run(inp)
    kv, qo = inp["kv_indptr"], inp["qo_indptr"]
    for b in range(3):
        L = int(kv[b + 1] - kv[b])
        qb = int(qo[b + 1] - qo[b])
        sl = oracle.request_slots(inp["req_to_token"], inp["req_to_token_stride"], kv, b)
        for i in range(qb):
            n = L - qb + i + 1
            od, ld = oracle.paged_attention(inp["q"][int(qo[b]) + i][None], inp["k_pool"], inp["v_pool"],
                                            sl[:n].astype(np.int32), 0, np.array([0, n], np.int32),
                                            inp["sm_scale"])
            np.testing.assert_allclose(o[int(qo[b]) + i], od[0], atol=1e-14)
            np.testing.assert_allclose(lse[int(qo[b]) + i], ld[0], atol=1e-14)


def test_prefill_with_one_row_is_decode():
    seq_lens = np.array([4, 9, 1])
    inp = build_paged_inputs(seq_lens, 4, 2, 8, 32, seed=13, q_lens=np.ones(3, np.int64))
    o, lse = _run(inp)
    dec = dict(inp)
    dec["qo_indptr"] = None
    o2, lse2 = _run(dec)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


# --------------------------------------------------------------------------- split partition and merge

def _random_indptr(B, lo, hi, rng):
    L = rng.integers(lo, hi + 1, size=B)
    return np.concatenate([[0], np.cumsum(L)]).astype(np.int64)


def test_partition_properties_random():
    rng = np.random.default_rng(77)
    for _ in range(300):
        B = int(rng.integers(1, 12))
        kv = _random_indptr(B, 1, 50, rng)
        N = int(kv[-1])
        Wh = int(rng.integers(1, 2 * N + 3))
        pieces = oracle.piece_table(kv, Wh)
        slots = [p[4] for p in pieces]
        assert len(set(slots)) == len(slots)
        assert all(0 <= s < Wh + B - 1 for s in slots)
        W = oracle.active_groups(N, Wh)
        sizes = [oracle.wg_bounds(N, Wh, w)[1] - oracle.wg_bounds(N, Wh, w)[0] for w in range(Wh)]
        assert min(sizes[:W]) >= 1 and max(sizes[:W]) - min(sizes[:W]) <= 1 and sum(sizes) == N
        assert all(s == 0 for s in sizes[W:])
        for b in range(B):
            mine = sorted((p[2], p[3], p[0]) for p in pieces if p[1] == b)
            assert mine[0][0] == 0 and mine[-1][1] == kv[b + 1] - kv[b]
            assert all(mine[i][1] == mine[i + 1][0] for i in range(len(mine) - 1))
            ws = [m[2] for m in mine]
            assert ws == list(range(ws[0], ws[-1] + 1))
            assert (ws[0], ws[-1]) == oracle.pieces_of_request(kv, Wh, b)


@pytest.mark.parametrize("Wh", [1, 2, 3, 7, 16, 64, 1000])
def test_split_merge_equals_definition(Wh):
    inp = _random_case(B=4, Hq=8, Hkv=2, D=16, seq=(1, 60), slots=256, seed=31)
    o, lse = _run(inp)
    o2, lse2 = oracle.decode_via_splits(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                        inp["req_to_token_stride"], inp["kv_indptr"], inp["sm_scale"], Wh)
    np.testing.assert_allclose(o2, o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse2, lse, atol=1e-12, rtol=0)


def test_split_partials_only_planned_slots_written():
    inp = _random_case(B=3, Hq=4, Hkv=1, D=8, seq=(1, 40), slots=128, seed=17)
    Wh = 5
    o_part, ml_part = oracle.split_partials(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                            inp["req_to_token_stride"], inp["kv_indptr"], inp["sm_scale"], Wh)
    written = {p[4] for p in oracle.piece_table(inp["kv_indptr"], Wh)}
    for s in range(Wh + 3 - 1):
        assert np.all(np.isfinite(ml_part[:, s])) == (s in written)
        assert np.all(np.isnan(ml_part[:, s])) == (s not in written)


def test_plan_num_splits_examples():
    # 32 requests, 8 kv heads, 256 CUs: target ceil(3*256/8) = 96 work groups per kv head.
    kv = np.concatenate([[0], np.cumsum(np.full(32, 1100))])
    assert oracle.plan_num_splits(kv, 8, 256) == 96
    # Short batch: 130 keys in total -> ceil(130/64) = 3 work groups.
    assert oracle.plan_num_splits(np.array([0, 60, 130]), 1, 256) == 3
    # Single key -> one work group; forced value wins.
    assert oracle.plan_num_splits(np.array([0, 1]), 8, 256) == 1
    assert oracle.plan_num_splits(np.array([0, 1]), 8, 256, forced=9) == 9
    # One kv head on 256 CUs with a long sequence is capped at max_splits.
    assert oracle.plan_num_splits(np.array([0, 1 << 20]), 1, 256) == 256
    # head_dim 256: one work group per CU -> ceil(256 / 8) = 32 per kv head
    assert oracle.plan_num_splits(kv, 8, 256, head_dim=256) == 32


def test_generator_is_deterministic_and_shaped():
    a = make_inputs("tiny", 0)
    b = make_inputs("tiny", 0)
    c = make_inputs("tiny", 1)
    assert all(np.array_equal(a[k], b[k]) for k in ("q", "k_pool", "v_pool", "req_to_token", "kv_indptr"))
    assert not np.array_equal(a["q"], c["q"])
    L = np.diff(a["kv_indptr"])
    assert L.min() >= 1 and L.max() <= 64 and a["k_pool"].shape == (512, 1, 64)
    used = a["req_to_token"][a["req_to_token"] >= 0]
    assert len(set(used.tolist())) == len(used) == int(L.sum())


# ----------------------------------------------------------------------------- prefill chunks

@pytest.mark.parametrize("forced", [1, 2, 3, 7])
def test_prefill_chunks_merge_to_the_definition(forced):
    """Cutting every query tile's key tiles into `forced` chunks (partials merged by the
    log-sum-exp rule) gives the definition's O and lse to 1e-12."""
    seq = np.array([300, 70, 777, 129])
    ql = np.array([40, 70, 200, 1])
    inp = build_paged_inputs(seq, 8, 2, 16, 2048, seed=41, q_lens=ql)
    ns = {(b, qt): forced for b, qt, _ in oracle.prefill_tiles(inp["qo_indptr"], inp["kv_indptr"], 4)}
    o, lse = oracle.prefill_via_chunks(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                      inp["req_to_token_stride"], inp["kv_indptr"], inp["qo_indptr"], inp["sm_scale"],
                                      ns, 4)
    ref_o, ref_lse = oracle.paged_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["req_to_token"],
                                            inp["req_to_token_stride"], inp["kv_indptr"], inp["sm_scale"],
                                            qo_indptr=inp["qo_indptr"])
    assert np.abs(o - ref_o).max() < 1e-12
    assert np.abs(lse - ref_lse).max() < 1e-12


def test_prefill_plan_chunks_tile_the_key_range():
    rng = np.random.default_rng(17)
    for _ in range(200):
        B = int(rng.integers(1, 9))
        L = rng.integers(1, 40000, size=B)
        q = np.array([int(rng.integers(1, min(int(x), 600) + 1)) for x in L])
        kv = np.concatenate([[0], np.cumsum(L)])
        qo = np.concatenate([[0], np.cumsum(q)])
        summary, ns = oracle.prefill_plan(qo, kv, 32, 8, 128, 256)
        for (b, qt, nt) in oracle.prefill_tiles(qo, kv, 4):
            n = ns[(b, qt)]
            assert 1 <= n <= oracle.PREFILL["max_chunks"]
            cuts = [nt * s // n for s in range(n + 1)]
            assert cuts[0] == 0 and cuts[-1] == nt and all(cuts[s + 1] > cuts[s] for s in range(n)), (nt, n)
        assert summary["num_items"] == sum(ns.values()) * 8
