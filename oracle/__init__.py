"""CPU oracle for paged grouped-query attention (test infrastructure only).

This package is the plain, slow, fp64 statement of what the paged GQA decode
and prefill path computes.  It is test infrastructure: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It imports numpy only, never loads the HIP library, and shares no
code with it.

Sources (the AstrAI commit-list pages; no code, tests or data are on them):

* [attention.py @c9ceca1] -- commits page for
  ``astrai/extension/backend/attention.py`` at commit c9ceca1: the commit that
  replaces the per-request SDPA loop with one masked SDPA call (causal offset
  seq_len - q_len folded into a boolean mask, exact-zero weights for masked
  lanes, output restored to flat qo_indptr order).
* [extension @6f67ba8] -- commits page for ``astrai/extension`` at commit
  6f67ba8: commits on paged decode through req_to_token with page size one,
  kv_indptr as the prefix sum of seq_lens, the unified causal_offset, GQA head
  expansion in the fallback, split-KV partials (o_part, ml_part) merged by a
  combine kernel, and partial slots written without a memset.
* [attention_backend.py @47b3ed4] -- commits page for
  ``astrai/extension/attention_backend.py`` at commit 47b3ed4: the commit that
  shares one write-then-gather K/V helper between backends (the KV append).

Parity status of each function is listed in its module header.
"""
from .attention import (bf16_bits_to_f64, f64_to_bf16_bits, request_slots, paged_attention,
                        attention_over_range)
from .partition import (DEFAULTS, plan_num_splits, active_groups, wg_bounds, piece_table, pieces_of_request,
                        split_partials, combine_partials, decode_via_splits, PREFILL, prefill_tiles, prefill_plan,
                        prefill_via_chunks)
from .kv_append import new_token_slots, kv_append

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "request_slots", "paged_attention",
    "attention_over_range", "DEFAULTS", "plan_num_splits", "active_groups", "wg_bounds", "piece_table",
    "pieces_of_request", "split_partials", "combine_partials", "decode_via_splits", "PREFILL", "prefill_tiles",
    "prefill_plan", "prefill_via_chunks",
    "new_token_slots", "kv_append",
]
