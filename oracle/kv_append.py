"""KV append into the paged pool, written out from its definition (test infrastructure).

What is computed: before a decode or prefill step attends, the K and V rows of
the step's new tokens are written into the token-slot pool, and the step then
gathers every key of the request, old and new, through req_to_token.

* [attention_backend.py @47b3ed4] -- commits page for
  ``astrai/extension/attention_backend.py`` at commit 47b3ed4: the commit that
  pulls the write-then-gather of K/V into one helper shared by the torch and
  FlashAttention backends.
* [extension @6f67ba8], the commit wiring paged decode into the CUDA backend:
  position t of request b lives in pool slot req_to_token[row_b + t] (page size
  one).  [attention.py @c9ceca1], the batched torch path: the q_len new tokens
  of a request are its last positions seq_len - q_len .. seq_len - 1, stored
  in flat qo_indptr order.

Reading taken here: kv_indptr already counts the new tokens (it is the prefix
sum of the sequence lengths after the append), so new token i of request b
(0 <= i < n_b) is position L_b - n_b + i.  Decode appends one token per request
(n_b = 1, new row b); prefill appends its q_len rows (new rows qo_indptr[b] ..).
Distinct new tokens must map to distinct slots; a repeated slot is rejected.

The values are bit patterns: an append is a copy, so the result is exact.

Parity: pinned (tests/test_oracle_append.py) by hand-worked fixtures in
tests/golden/kv_append_examples.json, by agreement with pools that the input
generator fills position by position in flat order (no req_to_token lookup),
by the one-key closed form of attention after the append (O equals the
appended V row exactly), and by untouched slots keeping their bits.
"""
from __future__ import annotations

import numpy as np

from .attention import request_slots


def new_token_slots(req_to_token, req_to_token_stride, kv_indptr, qo_indptr=None, page_size=1):
    """Pool slot of every new token, in flat new-row order ([sum n_b] int64)."""
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    B = kv_indptr.shape[0] - 1
    out = []
    for b in range(B):
        L = int(kv_indptr[b + 1] - kv_indptr[b])
        n = 1 if qo_indptr is None else int(qo_indptr[b + 1]) - int(qo_indptr[b])
        if not (1 <= n <= L):
            raise ValueError(f"request {b}: need 1 <= new tokens ({n}) <= seq_len ({L})")
        slots = request_slots(req_to_token, req_to_token_stride, kv_indptr, b, page_size)
        for i in range(n):
            out.append(int(slots[L - n + i]))
    out = np.asarray(out, dtype=np.int64)
    if np.unique(out).shape[0] != out.shape[0]:
        raise ValueError("two new tokens map to the same pool slot")
    return out


def kv_append(k_pool_bits, v_pool_bits, k_new_bits, v_new_bits, req_to_token, req_to_token_stride,
              kv_indptr, qo_indptr=None, page_size=1):
    """Pools after writing the new tokens' rows.

    k_pool_bits, v_pool_bits: [num_slots, Hkv, D] bf16 bits (not modified).
    k_new_bits, v_new_bits: [sum n_b, Hkv, D] bf16 bits, new row r of request b
    at r = b (decode, qo_indptr None) or qo_indptr[b] + i (prefill).
    Returns (k_pool', v_pool'): copies with slot(b, L_b - n_b + i) overwritten
    by new row (row0_b + i); every other slot keeps its bits.
    """
    k = np.array(k_pool_bits, copy=True)
    v = np.array(v_pool_bits, copy=True)
    slots = new_token_slots(req_to_token, req_to_token_stride, kv_indptr, qo_indptr, page_size)
    k_new = np.asarray(k_new_bits)
    v_new = np.asarray(v_new_bits)
    if k_new.shape[0] != slots.shape[0] or v_new.shape[0] != slots.shape[0]:
        raise ValueError(f"expected {slots.shape[0]} new rows, got {k_new.shape[0]} / {v_new.shape[0]}")
    for r, s in enumerate(slots):
        k[s] = k_new[r]
        v[s] = v_new[r]
    return k, v
