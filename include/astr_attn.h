/*
 * astr_attn.h -- C ABI of the paged grouped-query attention library (gfx950).
 *
 * What the calls compute (AstrAI commit-list pages):
 *  - [extension @6f67ba8] (commits page for astrai/extension at 6f67ba8), the
 *    commit wiring paged decode into the CUDA backend: the K/V of position t of
 *    request b sit in pool slot req_to_token[row_b + t] -- a page table with a
 *    page size of one -- and decode is always causal (the single query of a
 *    request sees all of its seq_len keys).
 *  - [extension @6f67ba8], the commit that builds kv_indptr (prefix sum of
 *    seq_lens) once per step, and the one hoisting qo_indptr for prefill.
 *  - [attention.py @c9ceca1] (commits page for
 *    astrai/extension/backend/attention.py at c9ceca1), the commit batching the
 *    torch path: prefill query row i of request b sits at absolute position
 *    seq_len_b - q_len_b + i and sees keys 0 .. that position; masked keys weigh
 *    exactly zero; rows are stored in flat qo_indptr order.
 *  - [extension @6f67ba8], the fallback commit with GQA head expansion: query
 *    head h reads kv head h / (Hq / Hkv).
 *  - [extension @6f67ba8], the split-KV commits: decode writes per-split
 *    partials (o_part, ml_part) that a separate combine kernel merges; the
 *    partials live in a caller-owned, preallocated workspace (the workspace
 *    commit) and are written without a memset.
 *
 * Per request b and query head h (g = h / (Hq / Hkv), sigma = sm_scale):
 *     s_t   = sigma * <q[row, h, :], K[slot_b(t), g, :]>      for visible t
 *     O     = sum_t exp(s_t - m) V[slot_b(t), g, :] / sum_t exp(s_t - m)
 *     lse   = m + ln sum_t exp(s_t - m)                       (m = max_t s_t)
 * computed from bf16 inputs with fp32 accumulation; O is stored as bf16
 * (round to nearest even), lse as fp32.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the name ends in _host.  bf16 data is
 *    passed as its 16-bit storage.  Strides count elements, not bytes.
 *  - The innermost (head_dim) dimension of q, o and the pools is contiguous.
 *    q, o, k_pool, v_pool must be 16-byte aligned and their token/slot/head
 *    strides multiples of 8 elements.
 *  - Ownership: the caller owns every buffer (q, o, lse, pools, index arrays,
 *    workspace).  The library never allocates or frees device memory, never
 *    synchronises the device, never copies host->device and keeps no pointer
 *    after a call returns.  *_host arrays are read only during the call.  The
 *    one library-owned buffer is the fixed device scratch array of the
 *    allocation-free entry point (astr_paged_decode_noalloc).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    null stream).  With a fixed plan (num_splits / max_q_len set) the enqueued
 *    work reads lengths only from device memory, so a call can be captured into
 *    a hip graph and replayed after the device index arrays change (same batch
 *    size).  Concurrent calls need distinct workspaces.
 *  - Errors: every argument is validated on the host before anything is
 *    launched; on failure nothing is enqueued and the call returns a non-zero
 *    astr_status whose message astr_last_error() gives (thread-local).  After
 *    each launch hipGetLastError() is checked (ASTR_ERR_HIP).  No C++ exception
 *    crosses this interface.  There is no fallback path.
 *  - Caller contract not checked on the host (undefined behaviour if broken):
 *    device index arrays hold the same values as their _host copies; every
 *    slot id a request uses is in [0, num_slots); pools hold finite values at
 *    the slots in use.  Slots no request uses are never read.
 */
#ifndef ASTR_ATTN_H
#define ASTR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ASTR_ABI_VERSION 7

/* Default cap on work groups per kv head in an automatic decode plan. */
#define ASTR_DEFAULT_MAX_SPLITS 256

typedef enum astr_status {
  ASTR_OK = 0,
  ASTR_ERR_INVALID_ARG = 1,   /* malformed argument: null pointer, bad length, misalignment */
  ASTR_ERR_UNSUPPORTED = 2,   /* well-formed but not built: head_dim or group size */
  ASTR_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the plan needs */
  ASTR_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} astr_status;

typedef struct astr_paged_args {
  int32_t batch;          /* B >= 0 requests; B == 0 is a no-op */
  int32_t num_qo_heads;   /* Hq >= 1 */
  int32_t num_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0, Hq / Hkv in {1, 2, 4, 8} */
  int32_t head_dim;       /* D in {32, 64, 128, 256} */
  float sm_scale;         /* logit scale, finite and > 0, e.g. 1/sqrt(D) */

  /* Queries, bf16.  Decode: row b is request b's query.  Prefill: rows in flat
   * qo_indptr order (row qo_indptr[b] + i is request b's i-th new token).
   * Element (row, h, d) at q[row * q_stride_tok + h * q_stride_head + d]. */
  const void* q;
  int64_t q_stride_tok, q_stride_head;
  /* Output, bf16, same row convention and indexing as q. */
  void* o;
  int64_t o_stride_tok, o_stride_head;
  /* Optional log-sum-exp (natural log), fp32: lse[row * lse_stride_tok + h].
   * NULL skips it. */
  float* lse;
  int64_t lse_stride_tok;

  /* KV pools, bf16: element (slot, g, d) at pool[slot * kv_stride_slot +
   * g * kv_stride_head + d], slot in [0, num_slots). */
  const void* k_pool;
  const void* v_pool;
  int64_t kv_stride_slot, kv_stride_head;
  int64_t num_slots;

  /* Page table, int32: slot of position t of request b is
   * req_to_token[row_b + t] with row_b = b * req_to_token_stride, or
   * row_b = kv_indptr[b] when req_to_token_stride == 0 (one flat list). */
  const int32_t* req_to_token;
  int64_t req_to_token_stride;

  /* kv_indptr[B+1]: prefix sum of seq_lens, kv_indptr[0] == 0, every
   * seq_len >= 1.  Both the device array and a host copy are required. */
  const int32_t* kv_indptr;
  const int32_t* kv_indptr_host;
  /* Prefill only (NULL for decode): qo_indptr[B+1], prefix sum of q_lens,
   * qo_indptr[0] == 0, 1 <= q_len_b <= seq_len_b. */
  const int32_t* qo_indptr;
  const int32_t* qo_indptr_host;

  /* Decode plan: work groups per kv head.  0 = choose from kv_indptr_host and
   * the device's CU count; > 0 fixes it (fixed grid, e.g. for graph capture). */
  int32_t num_splits;
  /* Prefill grid: 0 = max q_len from qo_indptr_host; > 0 fixes the grid's
   * query-tile count for q_len up to this value (graph capture). */
  int32_t max_q_len;

  /* Optional timing hook: NULL, or an array of hipEvent_t (created with
   * timing enabled) that the kernels' own dispatches stamp at kernel start
   * and end (hipExtLaunchKernel), so that stop - start is one kernel's
   * duration.  Decode: [0]/[1] start/end of the split kernel, [2]/[3]
   * start/end of the combine kernel (4 entries).  Prefill: [0]/[1] (2
   * entries).  Elements may be NULL (not stamped).  Events stay owned by the
   * caller; leave this NULL in code that is captured into a graph. */
  void* const* timing_events;

  /* Causal switch ([extension @6f67ba8], the commit unifying is_causal and
   * causal_offset into one offset that can be turned off): 0 (default) ->
   * prefill row i of request b sees keys 0 .. L_b - q_len_b + i; 1 -> every
   * row sees all L_b keys.  Decode is the same either way. */
  int32_t non_causal;
  /* Optional boolean mask ([extension @6f67ba8], the commits letting a mask
   * coexist with the causal offset and accepting 2-D [batch, kv_len] and 3-D
   * [batch, q_len, kv_len] masks): uint8, key t of request b is hidden from
   * its query row i when mask[b * mask_stride_req + i * mask_stride_row + t]
   * is 0 -- on top of the causal rule.  mask_stride_row == 0 is a 2-D mask
   * (one row per request, used by every query row); decode reads row 0.
   * NULL: no mask.  The mask pointer and both strides must be multiples of
   * 4 bytes; rows must hold max L_b entries (mask_stride_row >= max L_b for a
   * 3-D mask, mask_stride_req >= max L_b for a 2-D one) and a 3-D request
   * block max q_len rows; mask_stride_req < 2^31.  A query row left with no
   * visible key outputs zeros and lse = -inf. */
  const uint8_t* mask;
  int64_t mask_stride_req, mask_stride_row;

  /* Token slots per page of req_to_token's entries: 0 or 1 (default) -- each
   * entry is one position's slot; P > 1 (a power of two, at most 2^16) -- a
   * 2-D table (req_to_token_stride > 0, at least ceil(L_b / P) entries per
   * row) of page ids, position t of request b living in slot
   * req_to_token[b * stride + t / P] * P + t % P, so num_slots counts token
   * slots (pages * P).  The pages call for a paged allocation strategy next to
   * the page-size-one table; this is the reading taken for it. */
  int32_t page_size;
} astr_paged_args;

typedef struct astr_decode_plan {
  int32_t num_splits;      /* Wh: work groups per kv head */
  int32_t num_partials;    /* partial slots per query head = Wh + B - 1 */
  int32_t grid_x, grid_y, grid_z;  /* split-kernel grid: (Wh, Hkv, 1) */
  int64_t workspace_bytes; /* workspace this plan needs */
} astr_decode_plan;

/* Workspace bytes a decode call needs for `batch` requests with up to
 * `max_splits` work groups per kv head (0 = ASTR_DEFAULT_MAX_SPLITS).
 * [extension @6f67ba8], the commit moving the decode split partials
 * (o_part, ml_part) from per-file cached tensors into a preallocated,
 * caller-owned workspace. 
 * Layout (both fp32, offsets from the workspace base, P = Wh + B - 1):
 *   o_part  at 0:                          [Hq][P][D]  normalised split output
 *   ml_part at align256(Hq * P * D * 4):   [Hq][P][2]  (max logit m, sum l)
 * m is in natural-log units of the scaled logits; l = sum exp(s - m).
 * Returns 0 for invalid sizes.  Prefill needs no workspace. */
size_t astr_workspace_size(int32_t batch, int32_t num_qo_heads, int32_t head_dim, int32_t max_splits);

/* Host-only decode plan (no HIP call): the number of work groups per kv head
 * and the workspace it needs.  [extension @6f67ba8], the commit extracting the
 * shared split-count helper (compute_num_splits) and the partial allocation;
 * the pages give only its name, the rule here is this library's balanced flat
 * split (keys of a kv head laid end to end, cut into near-equal ranges).  num_cus > 0 sets the compute-unit count the
 * plan targets; num_cus <= 0 asks the current device.  Needs kv_indptr_host
 * unless a->num_splits > 0.  Returns astr_status. */
int astr_plan_decode(const astr_paged_args* a, int32_t num_cus, astr_decode_plan* out);

/* Paged GQA decode: one query row per request ([extension @6f67ba8], the
 * commits wiring paged decode with req_to_token as a page table of page size
 * one, and turning decode into split-KV partials merged by a separate combine
 * kernel).  Enqueues the split kernel, which writes partials into
 * `workspace`, then the combine kernel, which writes o (and lse).  workspace_bytes must be >= the plan's workspace_bytes.
 * Returns astr_status. */
int astr_paged_decode(const astr_paged_args* a, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the library's own device scratch array used by
 * astr_paged_decode_noalloc (one copy per GPU, held until the process ends). */
#define ASTR_NOALLOC_SCRATCH_BYTES (32ull << 20)

/* Allocation-free paged GQA decode, for callers that cannot allocate device
 * memory or hand over a workspace at call time (code under stream capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * kernels and result bits as astr_paged_decode with the same plan, but the
 * split partials go to a file-scope device array of
 * ASTR_NOALLOC_SCRATCH_BYTES bytes owned by the library (each GPU holds its
 * own copy from its first call until the process ends; its address is looked
 * up once per device).  The call allocates and frees nothing.
 * Limits and sharing: a plan whose partials need more than
 * ASTR_NOALLOC_SCRATCH_BYTES (astr_plan_decode's workspace_bytes) is rejected
 * with ASTR_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU
 * uses the same array, which keeps the last call's contents (nothing in it
 * needs clearing): calls that overlap on one GPU, e.g. on two streams, race
 * and give undefined results; serialise them.  Returns astr_status. */
int astr_paged_decode_noalloc(const astr_paged_args* a, void* stream);

/* The automatic prefill plan (no fixed grid: max_q_len == 0, batch <= 96).
 * Every query tile (128 / G positions x the G heads of one kv head) is one
 * work group.  With a workspace, the key range of a tile with more than
 * chunk_tiles key tiles (64 keys each) is cut into up to max_chunks (16)
 * chunks run as separate work groups and merged by the last one to finish;
 * chunk_tiles is the shortest length (at least 8 key tiles) at which all work
 * groups still fit in one round of the device's work-group slots (two per CU,
 * one at head_dim 256), so the longest work group is as short as one round
 * allows.  When the whole tiles alone exceed the slots nothing is split.
 * Fixed-grid calls (max_q_len set) and batches over 96 requests keep every
 * tile whole and report num_items = 0. */
typedef struct astr_prefill_plan {
  int32_t num_items;       /* work groups of the call (0: fixed-grid mapping) */
  int32_t split_tiles;     /* (query tile, kv head) pairs whose key range is split */
  int32_t chunk_tiles;     /* target key tiles per chunk */
  int32_t max_chunks;      /* chunk cap per query tile */
  int64_t partial_bytes;   /* bytes of chunk partials */
  int64_t workspace_bytes; /* workspace the split plan needs (0: nothing is split) */
} astr_prefill_plan;

/* Bytes at the start of a prefill workspace that hold its int32 arrival
 * counters (one per split query tile).  A fixed region, so that calls with
 * different plans can share one workspace. */
#define ASTR_WORKSPACE_COUNTER_BYTES 32768

/* Host-only prefill plan (validates a first; no HIP call unless num_cus <= 0,
 * which asks the current device's CU count).  [extension @6f67ba8], the
 * commit renaming the prefill kernels with _split_q / _mma suffixes (query
 * tiles split over work groups, matrix-core products); the pages give no
 * rule for the tiling, the one above is this library's.  Returns
 * astr_status. */
int astr_plan_prefill(const astr_paged_args* a, int32_t num_cus, astr_prefill_plan* out);

/* Ragged paged prefill with causal offset seq_len - q_len per request
 * ([attention.py @c9ceca1], the commit that batches the torch path with a
 * causal offset per request in flat qo_indptr order).
 * workspace: NULL (every query tile runs whole in one work group) or at least
 * astr_plan_prefill's workspace_bytes, 16-byte aligned.  Its counter region
 * (the first ASTR_WORKSPACE_COUNTER_BYTES) must be ZERO before its first use;
 * the split tiles' partials follow it, and every call leaves the counters at
 * zero again, so one zeroed workspace serves any number of calls of any plan
 * (calls that overlap need distinct workspaces).  A plan with more split
 * tiles than the region holds keeps every tile whole.  A non-NULL workspace
 * smaller than the plan needs is ASTR_ERR_WORKSPACE.  Returns astr_status. */
int astr_paged_prefill(const astr_paged_args* a, void* workspace, size_t workspace_bytes, void* stream);

/* The K and V rows of a step's new tokens, bf16, [rows, Hkv, D]: element
 * (row, g, d) at k_new[row * stride_tok + g * stride_head + d] (same for
 * v_new).  Row r belongs to request b and is its i-th new token, with
 * r = b for decode (one new token per request) or r = qo_indptr[b] + i for
 * prefill (q_len new tokens).  16-byte aligned; strides are positive
 * multiples of 8 elements. */
typedef struct astr_new_kv {
  const void* k_new;
  const void* v_new;
  int64_t stride_tok, stride_head;
} astr_new_kv;

/* KV append: writes the new tokens' K/V rows into the pools before they are
 * attended, as the pages' shared write-then-gather helper does
 * ([attention_backend.py @47b3ed4], commits page for
 * astrai/extension/attention_backend.py at 47b3ed4, the commit extracting
 * that helper).  kv_indptr already counts the new tokens, so new token i of
 * request b (n_b new tokens) is position L_b - n_b + i and its rows go to
 * pool slot req_to_token[row_b + L_b - n_b + i], every kv head.  n_b = 1 when
 * a->qo_indptr is NULL (decode), else qo_indptr[b+1] - qo_indptr[b] with
 * 1 <= n_b <= L_b.  Uses a's pools (written: they must be writable device
 * memory despite the const in astr_paged_args), strides, num_slots,
 * req_to_token, kv_indptr(+_host), qo_indptr(+_host), batch, num_kv_heads,
 * head_dim (a multiple of 8) and max_q_len (> 0: fixed grid for up to that
 * many new tokens per request, for graph capture); q, o, lse and
 * num_qo_heads are ignored.  The new tokens' slots must be distinct (else the
 * result is unspecified); a slot id outside [0, num_slots) is skipped, so
 * nothing is written outside the pools.  No workspace.  a->timing_events,
 * if set, takes the append kernel's start/end stamps in [0]/[1].  Returns
 * astr_status; on error nothing is enqueued. */
int astr_kv_append(const astr_paged_args* a, const astr_new_kv* nkv, void* stream);

/* Fused KV append + paged decode ([attention_backend.py @47b3ed4], the commit
 * sharing one helper that writes the step's new K/V into the cache and then
 * gathers the request's keys), one launch fewer than astr_kv_append
 * followed by astr_paged_decode, with the same result bit for bit (the same
 * kernels' arithmetic on the same values).  The new token of request b is
 * its last position L_b - 1 (kv_indptr counts it); its K/V row for kv head g
 * is taken from nkv (row b) by the work group that owns that key, which also
 * writes it into the pools at slot req_to_token[row_b + L_b - 1] (skipped for
 * a slot outside [0, num_slots)).  The pool rows of the new tokens are not
 * read.  Arguments, workspace and errors as astr_paged_decode; a->qo_indptr
 * must be NULL.  Returns astr_status. */
int astr_paged_decode_append(const astr_paged_args* a, const astr_new_kv* nkv, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Whole-step decode graph ([attention_backend.py @47b3ed4], commits page for
 * astrai/extension/attention_backend.py at 47b3ed4: the graph context with a
 * warm-up -> capture -> replay lifecycle, one graph per batch size, every
 * input at a fixed address, a live forward before capture).
 *
 * astr_decode_graph_create runs the decode of every layer once on `stream`
 * (live run; it also validates each layer), then captures the same calls
 * into a hipGraph and instantiates it.  layers[l] describes layer l's decode
 * exactly as for astr_paged_decode; new_kv is NULL (plain decode) or an array
 * of num_layers new-token rows (each layer's decode is then the fused
 * append + decode of astr_paged_decode_append).  Every layer needs a fixed
 * plan (num_splits > 0), no timing_events, and the same batch; all layers
 * share `workspace`, which must hold the largest layer's plan.  `stream` must
 * not be NULL (the null stream cannot be captured).
 *
 * The graph keeps the device pointers it was captured with: q, o, lse, pools,
 * index arrays, new rows and workspace must stay allocated at the same
 * addresses for as long as it is launched.  A launch recomputes the step from
 * their current contents, so new sequence lengths in the device kv_indptr /
 * req_to_token (same batch, each within the captured row stride) need no new
 * capture.  The kv_indptr_host copies are read only during create.
 * Ownership: the graph object (host memory, plus what the HIP runtime
 * allocates to instantiate it) belongs to the caller and is released by
 * astr_decode_graph_destroy.  On error *graph is NULL and nothing is
 * captured (the live run may have been enqueued).  Each returns astr_status. */
typedef struct astr_decode_graph astr_decode_graph;

int astr_decode_graph_create(const astr_paged_args* layers, const astr_new_kv* new_kv, int32_t num_layers,
                             void* workspace, size_t workspace_bytes, void* stream, astr_decode_graph** graph);

/* Enqueues one replay of the captured step on `stream`. */
int astr_decode_graph_launch(const astr_decode_graph* graph, void* stream);

/* Releases the graph (NULL is a no-op). */
int astr_decode_graph_destroy(astr_decode_graph* graph);

/* Message for the last non-OK status returned on this thread ("" if none).
 * The pages check every launch through launch-check macros ([backend
 * @c9ceca1], commits page for astrai/extension/backend at c9ceca1, the entry
 * adding them); here each status carries its message instead. */
const char* astr_last_error(void);

/* ASTR_ABI_VERSION of the built library (not from the pages: a check that the
 * header and the loaded library agree). */
int astr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ASTR_ATTN_H */
