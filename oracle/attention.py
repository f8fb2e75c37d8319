"""Paged GQA attention, written out from its definition in fp64 (test infrastructure).

What is computed (the masked SDPA that the AstrAI pages describe):

* [attention.py @c9ceca1], the commit that batches the torch-native path into one
  masked SDPA call: per request b, query row i sits at absolute position
  c_b + i with c_b = seq_len_b - q_len_b; key t is visible to row i iff
  t <= c_b + i; masked keys get a weight of exactly zero; outputs come back in
  flat qo_indptr order.
* [extension @6f67ba8], the commit wiring paged decode into the CUDA backend:
  K/V of position t of request b live in pool slot req_to_token[row_b + t]
  (a page table with page size one); kv_indptr is the prefix sum of seq_lens;
  decode is always causal, i.e. the single query sees all seq_len keys.
* [extension @6f67ba8], the commit adding the torch fallback with GQA head
  expansion: query head h reads kv head floor(h / (Hq / Hkv)) (repeat-interleave
  reading; the alternative h mod Hkv is not used).
* [extension @6f67ba8], the commits unifying is_causal and causal_offset into
  one causal offset that can be switched off, letting a boolean mask coexist
  with it, and accepting a 2-D [batch, kv_len] or 3-D [batch, q_len, kv_len]
  mask.  Readings: switched off (non_causal), every row sees all L_b keys; a
  mask entry that is zero hides the key from that row on top of the causal
  rule (2-D: one row per request, used by every query row); a row left with
  no visible key outputs zeros with lse = -inf (the empty sum is taken as
  zero weight everywhere).

Precision: bf16 inputs are widened exactly to fp64; sm_scale is first rounded to
fp32 (the precision the library receives it in), then widened.  Everything
else is fp64.  Output rounding is not part of the definition: callers compare
the fp64 result with the bf16 output under a tolerance.

Parity: pinned (tests/test_oracle.py) by closed forms (one key returns V
exactly; identical keys or a zero query return the mean of V; two keys give
sigmoid weights), torch's fp64 scaled_dot_product_attention on the gathered
keys, a brute-force loop on tiny inputs, slot-permutation invariance and the
hand-derived fixtures in tests/golden/.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 with round-to-nearest-even, returning uint16 bits.

    Rounds once, directly from fp64 (no intermediate fp32 rounding): the value is
    scaled by its bf16 quantum (2^(e-7), floored at the subnormal quantum
    2^-133), rounded to the nearest integer with ties to even, and scaled back.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)            # xf = m * 2^e with 0.5 <= |m| < 1, so 2^(e-1) <= |xf|
    e = np.maximum(e - 1, -126)     # unbiased exponent, clamped to the normal minimum
    quantum = np.ldexp(1.0, e - 7)
    r = np.rint(xf / quantum) * quantum   # np.rint rounds half to even
    r32 = r.astype(np.float32)            # exact: r has <= 8 significant bits (or is inf)
    bits = (r32.view(np.uint32) >> 16).astype(np.uint16)
    out[...] = bits
    out[np.isnan(x)] = 0x7FC0
    out[np.isposinf(x)] = 0x7F80
    out[np.isneginf(x)] = 0xFF80
    return out


def request_slots(req_to_token, req_to_token_stride, kv_indptr, b, page_size=1) -> np.ndarray:
    """Pool slots of request b's positions 0..L_b-1.

    Row base is b * stride for a 2-D table, or kv_indptr[b] for a flat table
    (stride 0).  With page size one, entry t of the row is position t's slot.
    With page size P > 1 (the pages name a paged allocation strategy beside
    the page-size-one table; reading taken: a 2-D table whose entries are page
    ids, P token slots per page), position t lives in slot
    row[t // P] * P + t % P.
    """
    L = int(kv_indptr[b + 1]) - int(kv_indptr[b])
    P = int(page_size)
    if P == 1:
        base = b * int(req_to_token_stride) if req_to_token_stride > 0 else int(kv_indptr[b])
        return np.asarray(req_to_token[base: base + L], dtype=np.int64)
    if req_to_token_stride <= 0:
        raise ValueError("a page size above one needs a 2-D page table (row stride > 0)")
    row = np.asarray(req_to_token[b * int(req_to_token_stride): b * int(req_to_token_stride) + (L + P - 1) // P],
                     dtype=np.int64)
    t = np.arange(L)
    return row[t // P] * P + t % P


def attention_over_range(qf, kf, vf, sigma, visible):
    """Masked softmax attention for one head.

    qf [R, D], kf [T, D], vf [T, D] float64; visible [R, T] bool.
    Returns (o [R, D], m [R], l [R]) where m is the row max of the visible
    scaled logits, l = sum of exp(s - m) over visible keys, and
    o = sum exp(s - m) v / l.  A row with no visible key gets o = 0,
    m = -inf and l = 0.
    """
    s = sigma * (qf @ kf.T)
    s_vis = np.where(visible, s, -np.inf)
    empty = ~visible.any(axis=1)
    m = np.where(empty, -np.inf, s_vis.max(axis=1, initial=-np.inf))
    p = np.where(visible, np.exp(s_vis - np.where(empty, 0.0, m)[:, None]), 0.0)
    l = p.sum(axis=1)
    o = (p @ vf) / np.where(empty, 1.0, l)[:, None]
    return o, m, l


def paged_attention(q_bits, k_pool_bits, v_pool_bits, req_to_token, req_to_token_stride,
                    kv_indptr, sm_scale, qo_indptr=None, non_causal=False, mask=None, page_size=1):
    """Reference paged GQA attention.

    q_bits: [rows, Hq, D] bf16 bits; rows = B for decode (qo_indptr None) or
    qo_indptr[B] for prefill, in flat qo_indptr order.
    k_pool_bits, v_pool_bits: [num_slots, Hkv, D] bf16 bits.
    non_causal: every query row sees all L_b keys (decode is the same either
    way: its one row sees all keys).
    mask: None, a 2-D [B, kv_len] or a 3-D [B, max_q_len, kv_len] array; key t
    is hidden from row i of request b when mask[b, t] (2-D) or mask[b, i, t]
    (3-D) is zero, on top of the causal rule.
    Returns (o [rows, Hq, D] float64, lse [rows, Hq] float64 natural log);
    rows with no visible key get o = 0 and lse = -inf.
    page_size: token slots per page of req_to_token's entries (see request_slots).
    Requires 1 <= q_len_b <= seq_len_b for every request.
    """
    q_bits = np.asarray(q_bits)
    rows, Hq, D = q_bits.shape
    Hkv = k_pool_bits.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    sigma = float(np.float32(sm_scale))
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    B = kv_indptr.shape[0] - 1
    out = np.zeros((rows, Hq, D), dtype=np.float64)
    lse = np.zeros((rows, Hq), dtype=np.float64)
    for b in range(B):
        L = int(kv_indptr[b + 1] - kv_indptr[b])
        if qo_indptr is None:
            row0, qb = b, 1
        else:
            row0 = int(qo_indptr[b])
            qb = int(qo_indptr[b + 1]) - row0
        if not (1 <= qb <= L):
            raise ValueError(f"request {b}: need 1 <= q_len ({qb}) <= seq_len ({L})")
        c = L - qb  # absolute position of the first query row
        slots = request_slots(req_to_token, req_to_token_stride, kv_indptr, b, page_size)
        K = bf16_bits_to_f64(k_pool_bits[slots])   # [L, Hkv, D]
        V = bf16_bits_to_f64(v_pool_bits[slots])
        Q = bf16_bits_to_f64(q_bits[row0: row0 + qb])  # [qb, Hq, D]
        if non_causal:
            visible = np.ones((qb, L), dtype=bool)
        else:
            visible = np.arange(L)[None, :] <= (c + np.arange(qb))[:, None]
        if mask is not None:
            mk = np.asarray(mask)
            rows_mask = mk[b, :L][None, :] if mk.ndim == 2 else mk[b, :qb, :L]
            visible = visible & (rows_mask != 0)
        for h in range(Hq):
            g = h // group
            o, m, l = attention_over_range(Q[:, h, :], K[:, g, :], V[:, g, :], sigma, visible)
            out[row0: row0 + qb, h] = o
            with np.errstate(divide="ignore"):
                lse[row0: row0 + qb, h] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return out, lse
