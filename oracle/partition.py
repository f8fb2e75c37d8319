"""Split-KV decode: work partition, per-split partials and their log-sum-exp merge (fp64).

Test infrastructure.  This is an independent statement of the split planner,
of what each split's partial holds, and of the combine step, so that the
library's plan and its workspace contents can be checked exactly.

The pages fix only the shape of the method, not the plan:
* [extension @6f67ba8], the commit moving decode onto split-KV: each split
  writes an output partial (o_part) and a (max, sum) partial (ml_part), and a
  separate combine kernel merges the splits into the final output.
* [extension @6f67ba8], the commit extracting shared helpers, which names a
  compute_num_splits helper without giving its rule.
* [extension @6f67ba8], the commit dropping the partial memset: every slot a
  split owns is written, so unowned slots are never read.

The rule below is this project's reading (the pages leave it open):

Balanced flat partition.  Let N = kv_indptr[B] be the total number of keys.
The keys of one kv head are laid end to end in request order and cut into
W = min(Wh, N) contiguous ranges of near-equal length: work group w
(0 <= w < W) takes flat positions [floor(w*N/W), floor((w+1)*N/W)), which
holds at least one key; work groups w >= W (possible when a fixed Wh exceeds
the key count) do nothing.  A range cut by request
boundaries yields one *piece* per request it touches; piece (w, b) writes
partial slot w + b.  Consecutive pieces advance w, b or both, so slots are
unique and lie in [0, W + B - 1), within the Wh + B - 1 slots the workspace
holds.  Request b's pieces are the work groups w_first(b)..w_last(b), all
non-empty, where the work group holding flat position x is
ceil((x + 1) * W / N) - 1.

Planner (integers only): Wh = forced value if given, else
min(ceil(WG_PER_CU * num_cus / Hkv), max(1, ceil(N / MIN_TOKENS)), MAX_SPLITS),
and at least 1.  WG_PER_CU is 3, or 1 at head_dim 256 (where the library's
split kernel fits one work group per CU).

Partial of one piece and query head: m = max of the scaled logits over the
piece's keys, l = sum exp(s - m), o = sum exp(s - m) v / l (normalised).
Merge: M = max m_s, w_s = l_s exp(m_s - M), O = sum w_s o_s / sum w_s,
lse = M + ln sum w_s.

Prefill split plan (end of this file): pinned in tests/test_oracle.py -- the
chunked computation equals the definition to 1e-12 for every chunk count (so
any chunking of a tile's key tiles is a correct result), and the chunks tile
each query tile's key range exactly; the C++ planner's summary equals
prefill_plan's exactly (tests/test_abi_cpu.py).

Parity: pinned in tests/test_oracle.py -- the merge of split partials equals
the direct definition (oracle.attention) to 1e-12 for every split count,
pieces tile each request exactly, slots are unique, ranges differ by at most
one key, the closed-form work-group lookup matches the table, and a
hand-worked partition fixture in tests/golden/.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_over_range, bf16_bits_to_f64, request_slots

DEFAULTS = {
    "wg_per_cu": 3,        # work groups per compute unit the plan aims for
    "min_tokens": 64,      # fewest keys per work group on average
    "max_splits": 256,     # cap on work groups per kv head
}


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def plan_num_splits(kv_indptr, num_kv_heads, num_cus, forced=0, head_dim=128, **consts):
    """Work groups per kv head (Wh) for a decode batch."""
    c = dict(DEFAULTS)
    if head_dim == 256:
        c["wg_per_cu"] = 1
    c.update(consts)
    if forced and forced > 0:
        return int(forced)
    N = int(kv_indptr[-1])
    target = _ceil_div(c["wg_per_cu"] * int(num_cus), int(num_kv_heads))
    by_len = max(1, _ceil_div(N, c["min_tokens"]))
    return max(1, min(target, by_len, c["max_splits"]))


def active_groups(N: int, Wh: int) -> int:
    """Work groups that hold keys: min(Wh, N)."""
    return min(int(Wh), int(N))


def wg_bounds(N: int, Wh: int, w: int):
    """Flat key range [lo, hi) of work group w (empty for w >= min(Wh, N))."""
    W = active_groups(N, Wh)
    if w >= W:
        return N, N
    return (w * N) // W, ((w + 1) * N) // W


def piece_table(kv_indptr, Wh: int):
    """All pieces as (w, b, t_begin, t_end, slot); t_* are positions inside request b."""
    kv = [int(x) for x in kv_indptr]
    B = len(kv) - 1
    N = kv[-1]
    pieces = []
    for w in range(Wh):
        lo, hi = wg_bounds(N, Wh, w)
        for b in range(B):
            a = max(lo, kv[b])
            e = min(hi, kv[b + 1])
            if a < e:
                pieces.append((w, b, a - kv[b], e - kv[b], w + b))
    return pieces


def pieces_of_request(kv_indptr, Wh: int, b: int):
    """(w_first, w_last) of request b, from the closed-form lookup."""
    N = int(kv_indptr[-1])
    W = active_groups(N, Wh)
    x0 = int(kv_indptr[b])
    x1 = int(kv_indptr[b + 1]) - 1
    return _ceil_div((x0 + 1) * W, N) - 1, _ceil_div((x1 + 1) * W, N) - 1


def split_partials(q_bits, k_pool_bits, v_pool_bits, req_to_token, req_to_token_stride,
                   kv_indptr, sm_scale, Wh):
    """Per-piece partials. Returns (o_part [Hq, P, D], ml_part [Hq, P, 2]); unwritten slots are NaN."""
    q_bits = np.asarray(q_bits)
    B, Hq, D = q_bits.shape
    Hkv = k_pool_bits.shape[1]
    group = Hq // Hkv
    sigma = float(np.float32(sm_scale))
    P = Wh + B - 1
    o_part = np.full((Hq, P, D), np.nan)
    ml_part = np.full((Hq, P, 2), np.nan)
    for (w, b, t0, t1, slot) in piece_table(kv_indptr, Wh):
        slots = request_slots(req_to_token, req_to_token_stride, kv_indptr, b)[t0:t1]
        K = bf16_bits_to_f64(k_pool_bits[slots])
        V = bf16_bits_to_f64(v_pool_bits[slots])
        Q = bf16_bits_to_f64(q_bits[b])
        vis = np.ones((1, t1 - t0), dtype=bool)
        for h in range(Hq):
            g = h // group
            o, m, l = attention_over_range(Q[h][None, :], K[:, g, :], V[:, g, :], sigma, vis)
            o_part[h, slot] = o[0]
            ml_part[h, slot] = (m[0], l[0])
    return o_part, ml_part


def combine_partials(o_part, ml_part, kv_indptr, Wh):
    """Log-sum-exp merge of each request's pieces. Returns (o [B, Hq, D], lse [B, Hq])."""
    Hq, _, D = o_part.shape
    B = len(kv_indptr) - 1
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        wf, wl = pieces_of_request(kv_indptr, Wh, b)
        sl = np.arange(wf, wl + 1) + b
        m = ml_part[:, sl, 0]       # [Hq, n]
        l = ml_part[:, sl, 1]
        M = m.max(axis=1)
        wgt = l * np.exp(m - M[:, None])
        tot = wgt.sum(axis=1)
        out[b] = np.einsum("hs,hsd->hd", wgt, o_part[:, sl, :]) / tot[:, None]
        lse[b] = M + np.log(tot)
    return out, lse


def decode_via_splits(q_bits, k_pool_bits, v_pool_bits, req_to_token, req_to_token_stride,
                      kv_indptr, sm_scale, Wh):
    o_part, ml_part = split_partials(q_bits, k_pool_bits, v_pool_bits, req_to_token,
                                     req_to_token_stride, kv_indptr, sm_scale, Wh)
    return combine_partials(o_part, ml_part, kv_indptr, Wh)


# ----------------------------------------------------------------------------- prefill split plan
#
# Ragged prefill runs one work group per query tile: 128 // G query positions
# of one request times the G query heads of one kv head.  Query tile qt of
# request b (q_b new tokens, L_b keys) covers positions [qt*BQ, min((qt+1)*BQ,
# q_b)); its rows see keys up to (L_b - q_b) + min((qt+1)*BQ, q_b) - 1
# (all L_b keys when non-causal), i.e. nt = ceil(kv_end / 64) key tiles of 64.
#
# This project's split rule (the pages only say that long key ranges are
# split into partials merged by a combine step, for decode): with S slots
# (two work groups per CU, one at head_dim 256), a tile of nt key tiles is cut
# into ns = min(16, ceil(nt / T)) chunks, chunk s covering key tiles
# [floor(nt*s/ns), floor(nt*(s+1)/ns)), where T is the smallest chunk length
# of at least 8 key tiles at which all chunks, times Hkv, still fit in S --
# and nothing is split when the whole tiles, times Hkv, already number more
# than S, or when the chunks of split tiles, times Hkv, would not fit the
# workspace's counter region (8192 counters at its start, before the
# partials).  The plan applies to the automatic grid of at most 96 requests.

PREFILL = {"rows": 128, "key_tile": 64, "min_chunk_tiles": 8, "max_chunks": 16, "max_reqs": 96,
           "counter_bytes": 32768}


def prefill_tiles(qo_indptr, kv_indptr, group, non_causal=False):
    """[(b, qt, nt)] for every query tile of the batch."""
    BQ = PREFILL["rows"] // group
    KT = PREFILL["key_tile"]
    out = []
    for b in range(len(kv_indptr) - 1):
        qb = int(qo_indptr[b + 1] - qo_indptr[b])
        L = int(kv_indptr[b + 1] - kv_indptr[b])
        for qt in range(_ceil_div(qb, BQ)):
            kv_end = L if non_causal else L - qb + min(BQ * (qt + 1), qb)
            out.append((b, qt, _ceil_div(kv_end, KT)))
    return out


def prefill_plan(qo_indptr, kv_indptr, num_qo_heads, num_kv_heads, head_dim, num_cus, non_causal=False,
                 split=True):
    """The split plan's summary (num_items, split_tiles, chunk_tiles, max_chunks, partial_bytes,
    workspace_bytes) and the chunk count of every query tile {(b, qt): ns}."""
    B = len(kv_indptr) - 1
    group = num_qo_heads // num_kv_heads
    if B < 1 or B > PREFILL["max_reqs"]:
        return None, {}
    tiles = prefill_tiles(qo_indptr, kv_indptr, group, non_causal)
    slots = (1 if head_dim == 256 else 2) * num_cus

    def items_at(T):
        return sum(min(PREFILL["max_chunks"], _ceil_div(nt, T)) for _, _, nt in tiles) * num_kv_heads

    T = max(PREFILL["min_chunk_tiles"], max(nt for _, _, nt in tiles))
    splitting = split and items_at(T) <= slots
    if splitting:
        # The smallest T >= min_chunk_tiles with items_at(T) <= slots, by trying each in turn
        # (items_at only falls as T grows).
        for t in range(PREFILL["min_chunk_tiles"], T + 1):
            if items_at(t) <= slots:
                T = t
                break
    max_chunks = PREFILL["max_chunks"] if splitting else 1
    ns = {(b, qt): min(max_chunks, _ceil_div(nt, T)) for b, qt, nt in tiles}
    items = sum(ns.values()) * num_kv_heads
    split_chunks = sum(n for n in ns.values() if n > 1) * num_kv_heads
    split_tiles = sum(1 for n in ns.values() if n > 1) * num_kv_heads
    part_one = 4 * 2 * (head_dim // 16) * 64 * 16 + 4 * 2 * 64 * 8
    if split_chunks > PREFILL["counter_bytes"] // 4:
        return prefill_plan(qo_indptr, kv_indptr, num_qo_heads, num_kv_heads, head_dim, num_cus, non_causal,
                            split=False)
    partial_bytes = split_chunks * part_one
    ws = PREFILL["counter_bytes"] + partial_bytes if split_chunks else 0
    return {"num_items": items, "split_tiles": split_tiles, "chunk_tiles": T, "max_chunks": max_chunks,
            "partial_bytes": partial_bytes, "workspace_bytes": ws}, ns


def prefill_via_chunks(q_bits, k_pool_bits, v_pool_bits, req_to_token, req_to_token_stride, kv_indptr, qo_indptr,
                       sm_scale, ns_of, group, non_causal=False):
    """Prefill computed chunk by chunk: each query tile's key tiles cut as the plan says, each
    chunk's (m, l, o) partial over its keys, merged by the log-sum-exp rule.  Returns (O, lse)."""
    BQ = PREFILL["rows"] // group
    KT = PREFILL["key_tile"]
    qf = bf16_bits_to_f64(q_bits)
    kf = bf16_bits_to_f64(k_pool_bits)
    vf = bf16_bits_to_f64(v_pool_bits)
    rows, Hq, D = qf.shape
    Hkv = kf.shape[1]
    sigma = float(np.float32(sm_scale))
    O = np.zeros((rows, Hq, D))
    lse = np.full((rows, Hq), -np.inf)
    for b, qt, nt in prefill_tiles(qo_indptr, kv_indptr, group, non_causal):
        q0 = int(qo_indptr[b])
        qb = int(qo_indptr[b + 1]) - q0
        L = int(kv_indptr[b + 1] - kv_indptr[b])
        slots = request_slots(req_to_token, req_to_token_stride, kv_indptr, b)
        ns = ns_of[(b, qt)]
        for i in range(qt * BQ, min((qt + 1) * BQ, qb)):
            last = L - 1 if non_causal else L - qb + i
            for h in range(Hq):
                g = h * Hkv // Hq
                parts = []
                for s in range(ns):
                    t0, t1 = (nt * s // ns) * KT, min((nt * (s + 1) // ns) * KT, last + 1)
                    if t1 <= t0:
                        continue
                    keys = slots[t0:t1]
                    logits = sigma * (kf[keys, g, :] @ qf[q0 + i, h, :])
                    m = logits.max()
                    p = np.exp(logits - m)
                    parts.append((m, p.sum(), p @ vf[keys, g, :] / p.sum()))
                M = max(m for m, _, _ in parts)
                w = [l * np.exp(m - M) for m, l, _ in parts]
                O[q0 + i, h] = sum(wi * o for wi, (_, _, o) in zip(w, parts)) / sum(w)
                lse[q0 + i, h] = M + np.log(sum(w))
    return O, lse
