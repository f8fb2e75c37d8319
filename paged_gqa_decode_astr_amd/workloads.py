"""Seeded synthetic inputs for paged GQA decode and prefill.

This module only draws inputs: sequence lengths, a random slot permutation that
plays the role of the page table (page_size = 1), and N(0,1) values rounded to
bf16.  It holds none of the attention arithmetic, so both the HIP path and the
CPU oracle can consume its output without sharing any computation.

Pool layout is token-major ``[num_slots, Hkv, D]`` (one slot per token, as in
the AstrAI commits page for astrai/extension @6f67ba8, entry wiring paged decode
into the CUDA backend with req_to_token as a page table of page size one).
Slots that no request uses are filled with a quiet-NaN bf16 pattern so that any
read outside a request's sequence shows up in the output.

All values are returned as host numpy arrays: bf16 tensors as their raw
``uint16`` bit patterns, index arrays as ``int32``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BF16_QNAN = 0x7FC0


@dataclass(frozen=True)
class Config:
    """One synthetic workload shape."""
    cid: str
    kind: str            # "decode" or "prefill"
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    num_slots: int
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# The five workload shapes. Seeds are ``1000 * config number + trial``.
CONFIGS = {
    "tiny": Config("tiny", "decode", 4, 4, 1, 64, 512,
                   "tiny paged decode, seq_len ~ U{1..64}", {"seq": ("uniform", 1, 64), "num": 1}),
    "decode_b32": Config("decode_b32", "decode", 32, 32, 8, 128, 1 << 17,
                         "decode microbench, seq_len ~ U{200..2000}", {"seq": ("uniform", 200, 2000), "num": 2}),
    "long_b1": Config("long_b1", "decode", 1, 32, 8, 128, 1 << 18,
                      "long context, seq_len = 32768, peaky keys", {"seq": ("const", 32768), "peaky": 16, "num": 3}),
    "long_b4": Config("long_b4", "decode", 4, 32, 8, 128, 1 << 18,
                      "long context, seq_len = 32768, peaky keys", {"seq": ("const", 32768), "peaky": 16, "num": 3}),
    "ragged_b256": Config("ragged_b256", "decode", 256, 32, 8, 128, 1 << 20,
                          "ragged decode, seq_len log-uniform in [1,4096]",
                          {"seq": ("loguniform", 1, 4096), "num": 4}),
    "prefill_b8": Config("prefill_b8", "prefill", 8, 32, 8, 128, 1 << 16,
                         "ragged prefill, prefix ~ U{0..2048}, q_len ~ U{1..512}",
                         {"prefix": (0, 2048), "qlen": (1, 512), "num": 5}),
}


def seed_for(cfg: Config, trial: int = 0) -> int:
    return 1000 * int(cfg.extra["num"]) + int(trial)


def randn_bf16_bits(gen: torch.Generator, shape) -> np.ndarray:
    """N(0,1) float32 samples rounded to bf16 (round-to-nearest-even), as uint16 bits."""
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _draw_seq_lens(cfg: Config, gen: torch.Generator) -> np.ndarray:
    kind = cfg.extra["seq"][0]
    B = cfg.batch
    if kind == "uniform":
        lo, hi = cfg.extra["seq"][1], cfg.extra["seq"][2]
        return torch.randint(lo, hi + 1, (B,), generator=gen).numpy().astype(np.int64)
    if kind == "const":
        return np.full(B, cfg.extra["seq"][1], dtype=np.int64)
    if kind == "loguniform":
        lo, hi = cfg.extra["seq"][1], cfg.extra["seq"][2]
        u = torch.rand(B, generator=gen, dtype=torch.float64).numpy()
        lens = np.floor(np.exp(u * math.log(hi + 1))).astype(np.int64)
        lens = np.clip(lens, lo, hi)
        # A few single-token requests and one at the maximum length, so every
        # batch holds both extremes of the range.
        lens[: min(4, B)] = 1
        if B > 4:
            lens[4] = hi
        return lens
    raise ValueError(kind)


def build_paged_inputs(seq_lens, num_qo_heads, num_kv_heads, head_dim, num_slots, seed,
                       q_lens=None, row_stride=None, peaky_keys=0, flat_table=False,
                       poison_unused=True, new_tokens=None, page_size=1):
    """Build one batch of paged inputs.

    seq_lens: per-request KV length L_b.  q_lens: per-request number of query
    rows (None = decode, one row each).  The page table row of request b holds
    a fresh run of a random permutation of all pool slots, so requests never
    share a slot.  ``flat_table`` returns req_to_token as one flat list indexed
    by kv_indptr (row stride 0); otherwise a 2-D table padded with -1.

    new_tokens: per-request count n_b (1 <= n_b <= L_b) of tokens whose K/V
    are not yet in the pool.  The K/V values of the last n_b positions of each
    request are then returned as ``k_new`` / ``v_new`` ([sum n_b, Hkv, D], in
    request order) instead of being stored, and their slots keep the unused
    fill; ``k_pool_full`` / ``v_pool_full`` hold the pools with every position
    stored, for comparison.

    page_size: P > 1 hands out whole pages of P consecutive slots (a random
    permutation of the num_slots / P pages, fresh pages per request) and
    returns req_to_token as a 2-D table of page ids; ``token_slots`` then
    lists every position's slot in flat key order.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = int(seq_lens.shape[0])
    gen = torch.Generator().manual_seed(int(seed))
    N = int(seq_lens.sum())
    if N > num_slots:
        raise ValueError(f"pool of {num_slots} slots is smaller than total length {N}")
    kv_indptr = np.zeros(B + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(seq_lens)
    P = int(page_size)
    if P > 1:
        if flat_table:
            raise ValueError("a page size above one uses a 2-D page table")
        npages = [(int(L) + P - 1) // P for L in seq_lens]
        if sum(npages) * P > num_slots:
            raise ValueError(f"pool of {num_slots} slots holds fewer than {sum(npages)} pages of {P}")
        pages = torch.randperm(num_slots // P, generator=gen).numpy().astype(np.int32)
        stride = int(row_stride) if row_stride is not None else max(1, max(npages) if B else 1)
        req_to_token = np.full((B, stride), -1, dtype=np.int32)
        slots_flat = np.empty(N, dtype=np.int32)
        nxt = 0
        for b in range(B):
            mine = pages[nxt: nxt + npages[b]]
            nxt += npages[b]
            req_to_token[b, : npages[b]] = mine
            # Page k of the request holds its next run of up to P positions in
            # P consecutive slots starting at slot mine[k] * P.
            for k in range(npages[b]):
                lo = int(kv_indptr[b]) + k * P
                hi = min(lo + P, int(kv_indptr[b + 1]))
                slots_flat[lo:hi] = np.arange(int(mine[k]) * P, int(mine[k]) * P + (hi - lo))
        req_to_token = req_to_token.reshape(-1)
    else:
        perm = torch.randperm(num_slots, generator=gen).numpy().astype(np.int32)
        slots_flat = perm[:N].copy()
    if P > 1:
        pass   # req_to_token is the page table built above
    elif flat_table:
        req_to_token = slots_flat.copy()
        stride = 0
    else:
        stride = int(row_stride) if row_stride is not None else max(1, int(seq_lens.max()) if B else 1)
        req_to_token = np.full((B, stride), -1, dtype=np.int32)
        for b in range(B):
            req_to_token[b, : seq_lens[b]] = slots_flat[kv_indptr[b]: kv_indptr[b + 1]]
        req_to_token = req_to_token.reshape(-1)

    if q_lens is None:
        rows = B
        qo_indptr = None
    else:
        q_lens = np.asarray(q_lens, dtype=np.int64)
        qo_indptr = np.zeros(B + 1, dtype=np.int32)
        qo_indptr[1:] = np.cumsum(q_lens)
        rows = int(qo_indptr[-1])
    q = randn_bf16_bits(gen, (rows, num_qo_heads, head_dim))
    k_vals = randn_bf16_bits(gen, (N, num_kv_heads, head_dim))
    v_vals = randn_bf16_bits(gen, (N, num_kv_heads, head_dim))
    if peaky_keys and N:
        # Scale the whole K row of a few positions per request by 8 (exact in
        # bf16: only the exponent moves) to make the softmax peaky.
        k32 = (k_vals.astype(np.uint32) << 16).view(np.float32)
        for b in range(B):
            L = int(seq_lens[b])
            if L == 0:
                continue
            pos = torch.randint(0, L, (min(peaky_keys, L),), generator=gen).numpy()
            k32[kv_indptr[b] + pos] *= 8.0
        k_vals = (k32.view(np.uint32) >> 16).astype(np.uint16)
    fill = BF16_QNAN if poison_unused else 0
    k_pool = np.full((num_slots, num_kv_heads, head_dim), fill, dtype=np.uint16)
    v_pool = np.full((num_slots, num_kv_heads, head_dim), fill, dtype=np.uint16)
    extra = {}
    if new_tokens is not None:
        n_new = np.broadcast_to(np.asarray(new_tokens, dtype=np.int64), (B,))
        if np.any(n_new < 1) or np.any(n_new > seq_lens):
            raise ValueError("new_tokens must satisfy 1 <= n_b <= seq_len_b")
        is_new = np.zeros(N, dtype=bool)
        for b in range(B):
            is_new[kv_indptr[b + 1] - n_new[b]: kv_indptr[b + 1]] = True
        extra["k_pool_full"] = k_pool.copy()
        extra["v_pool_full"] = v_pool.copy()
        extra["k_pool_full"][slots_flat] = k_vals
        extra["v_pool_full"][slots_flat] = v_vals
        extra["k_new"] = k_vals[is_new].copy()
        extra["v_new"] = v_vals[is_new].copy()
        extra["new_indptr"] = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
        k_pool[slots_flat[~is_new]] = k_vals[~is_new]
        v_pool[slots_flat[~is_new]] = v_vals[~is_new]
    else:
        k_pool[slots_flat] = k_vals
        v_pool[slots_flat] = v_vals
    return {**extra,
        "q": q, "k_pool": k_pool, "v_pool": v_pool,
        "req_to_token": req_to_token, "req_to_token_stride": stride,
        "kv_indptr": kv_indptr, "qo_indptr": qo_indptr,
        "seq_lens": seq_lens.astype(np.int32),
        "num_qo_heads": num_qo_heads, "num_kv_heads": num_kv_heads, "head_dim": head_dim,
        "num_slots": num_slots, "sm_scale": 1.0 / math.sqrt(head_dim),
        "page_size": P, "token_slots": slots_flat,
    }


def make_inputs(cfg_or_id, trial: int = 0, **overrides):
    """Inputs for one of the named workload shapes, seeded by config and trial."""
    cfg = CONFIGS[cfg_or_id] if isinstance(cfg_or_id, str) else cfg_or_id
    seed = seed_for(cfg, trial)
    gen = torch.Generator().manual_seed(seed)
    if cfg.kind == "decode":
        seq_lens = _draw_seq_lens(cfg, gen)
        q_lens = None
    else:
        plo, phi = cfg.extra["prefix"]
        qlo, qhi = cfg.extra["qlen"]
        prefix = torch.randint(plo, phi + 1, (cfg.batch,), generator=gen).numpy().astype(np.int64)
        q_lens = torch.randint(qlo, qhi + 1, (cfg.batch,), generator=gen).numpy().astype(np.int64)
        seq_lens = prefix + q_lens
    kw = dict(peaky_keys=cfg.extra.get("peaky", 0))
    kw.update(overrides)
    out = build_paged_inputs(seq_lens, cfg.num_qo_heads, cfg.num_kv_heads, cfg.head_dim,
                             cfg.num_slots, seed + 7919, q_lens=q_lens, **kw)
    out["config"] = cfg.cid
    out["seed"] = seed
    return out
