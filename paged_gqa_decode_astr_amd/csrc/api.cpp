// C ABI of the paged GQA attention library: argument validation, the split
// planner, workspace layout and kernel launches.  See include/astr_attn.h for
// the contract of each entry point.
//
// Validation mirrors the reference backend's habit of checking a forward call
// before touching the KV cache ([attention.py @c9ceca1], the commit that adds a
// shared forward guard and validates prefill inputs before KV allocation): all
// checks run on the host, before anything is enqueued.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "abi_internal.hpp"
#include "astr_attn.h"
#include "launch.hpp"

namespace astr {

namespace {
thread_local char g_err[512] = "";
}  // namespace

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return ASTR_OK;
}

const char* last_error() { return g_err; }

}  // namespace astr

namespace {

using astr::fail;
using astr::ok;

// Planner constants: work groups per CU (three 4-wavefront work groups fill
// a CU at the head_dim-128 kernel's register budget), fewest keys per work
// group on average (one 16-key tile for each of its wavefronts).
constexpr int64_t kWgPerCu = 3;
// At head_dim 256 the split kernel runs one wave per SIMD: one work group per CU.
int64_t wg_per_cu(int32_t head_dim) { return head_dim == 256 ? 1 : kWgPerCu; }
constexpr int64_t kMinTokens = 64;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

static_assert(astr::kCounterBytes == ASTR_WORKSPACE_COUNTER_BYTES, "counter region size");

int64_t partial_bytes(int64_t batch, int64_t hq, int64_t d, int64_t splits) {
  const int64_t P = splits + batch - 1;
  return align256(hq * P * d * 4) + hq * P * 2 * 4;
}

// Per-device compute-unit count, cached after the first query.
std::mutex g_cu_mu;
std::vector<int> g_cu_count;

int device_cu_count(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ASTR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_cu_mu);
  if ((int)g_cu_count.size() <= dev) g_cu_count.resize(dev + 1, 0);
  if (g_cu_count[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(ASTR_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    g_cu_count[dev] = n;
  }
  *out = g_cu_count[dev];
  return ASTR_OK;
}

// Page size -> log2, or -1 when it is not 0, 1 or a power of two up to 2^16.
int page_shift_of(int32_t page_size) {
  if (page_size == 0 || page_size == 1) return 0;
  for (int s = 1; s <= 16; ++s)
    if (page_size == (1 << s)) return s;
  return -1;
}

// The page-size rules shared by every entry point; *shift receives log2 P.
int validate_pages(const astr_paged_args* a, int* shift) {
  *shift = page_shift_of(a->page_size);
  if (*shift < 0) return fail(ASTR_ERR_INVALID_ARG, "page_size must be 0, 1 or a power of two up to 65536 (got %d)",
                              a->page_size);
  if (*shift > 0 && a->req_to_token_stride <= 0)
    return fail(ASTR_ERR_INVALID_ARG, "a page size above one needs a 2-D page table (req_to_token_stride > 0)");
  return ASTR_OK;
}

// Table entries request b's row needs: L_b, or ceil(L_b / P) with pages.
int64_t row_entries(int64_t L, int shift) { return shift == 0 ? L : ((L - 1) >> shift) + 1; }

// Checks shared by decode and prefill.  Sets *total_keys = kv_indptr[B].
int validate_common(const astr_paged_args* a, bool prefill, int64_t* total_keys) {
  if (a == nullptr) return fail(ASTR_ERR_INVALID_ARG, "args is NULL");
  if (a->batch < 0) return fail(ASTR_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", a->batch);
  if (a->num_qo_heads < 1 || a->num_kv_heads < 1)
    return fail(ASTR_ERR_INVALID_ARG, "head counts must be >= 1 (Hq=%d, Hkv=%d)", a->num_qo_heads, a->num_kv_heads);
  if (a->batch > 65535 || a->num_kv_heads > 65535)
    return fail(ASTR_ERR_INVALID_ARG, "batch (%d) and num_kv_heads (%d) must be <= 65535 (grid limits)", a->batch,
                a->num_kv_heads);
  if (a->num_qo_heads % a->num_kv_heads != 0)
    return fail(ASTR_ERR_INVALID_ARG, "num_qo_heads (%d) must be a multiple of num_kv_heads (%d)", a->num_qo_heads,
                a->num_kv_heads);
  const int group = a->num_qo_heads / a->num_kv_heads;
  const bool supported = prefill ? astr::prefill_supported(a->head_dim, group) : astr::decode_supported(a->head_dim, group);
  if (!supported)
    return fail(ASTR_ERR_UNSUPPORTED, "no kernel for head_dim=%d and group size %d (head_dim in {32,64,128,256}, group in {1,2,4,8})",
                a->head_dim, group);
  if (!(a->sm_scale > 0.f) || a->sm_scale == __builtin_inff())
    return fail(ASTR_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  *total_keys = 0;
  if (a->batch == 0) return ASTR_OK;

  struct { const void* p; const char* name; } req[] = {
      {a->q, "q"}, {a->o, "o"}, {a->k_pool, "k_pool"}, {a->v_pool, "v_pool"},
      {a->req_to_token, "req_to_token"}, {a->kv_indptr, "kv_indptr"}, {a->kv_indptr_host, "kv_indptr_host"}};
  for (auto& r : req)
    if (r.p == nullptr) return fail(ASTR_ERR_INVALID_ARG, "%s is NULL", r.name);
  if (!aligned16(a->q) || !aligned16(a->o) || !aligned16(a->k_pool) || !aligned16(a->v_pool))
    return fail(ASTR_ERR_INVALID_ARG, "q, o, k_pool and v_pool must be 16-byte aligned");
  struct { int64_t v; const char* name; } strides[] = {
      {a->q_stride_tok, "q_stride_tok"}, {a->q_stride_head, "q_stride_head"}, {a->o_stride_tok, "o_stride_tok"},
      {a->o_stride_head, "o_stride_head"}, {a->kv_stride_slot, "kv_stride_slot"}, {a->kv_stride_head, "kv_stride_head"}};
  for (auto& s : strides)
    if (s.v <= 0 || s.v % 8 != 0)
      return fail(ASTR_ERR_INVALID_ARG, "%s must be a positive multiple of 8 elements (got %lld)", s.name, (long long)s.v);
  if (a->lse != nullptr) {
    if ((reinterpret_cast<uintptr_t>(a->lse) & 3u) != 0) return fail(ASTR_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    if (a->lse_stride_tok < 1) return fail(ASTR_ERR_INVALID_ARG, "lse_stride_tok must be >= 1");
  }
  if (a->num_slots < 1 || a->num_slots > (int64_t)INT32_MAX + 1)
    return fail(ASTR_ERR_INVALID_ARG, "num_slots must be in [1, 2^31] (got %lld)", (long long)a->num_slots);
  if (a->req_to_token_stride < 0) return fail(ASTR_ERR_INVALID_ARG, "req_to_token_stride must be >= 0");

  int shift = 0;
  const int pst = validate_pages(a, &shift);
  if (pst != ASTR_OK) return pst;
  const int32_t* kv = a->kv_indptr_host;
  if (kv[0] != 0) return fail(ASTR_ERR_INVALID_ARG, "kv_indptr[0] must be 0 (got %d)", kv[0]);
  for (int b = 0; b < a->batch; ++b) {
    const int64_t L = (int64_t)kv[b + 1] - kv[b];
    if (L < 1) return fail(ASTR_ERR_INVALID_ARG, "request %d: seq_len must be >= 1 (got %lld)", b, (long long)L);
    if (a->req_to_token_stride > 0 && row_entries(L, shift) > a->req_to_token_stride)
      return fail(ASTR_ERR_INVALID_ARG, "request %d: seq_len %lld needs %lld table entries, more than req_to_token_stride %lld",
                  b, (long long)L, (long long)row_entries(L, shift), (long long)a->req_to_token_stride);
  }
  *total_keys = kv[a->batch];
  return ASTR_OK;
}

// The causal switch and the optional mask: alignment, strides, and rows long
// enough for max_len keys and max_rows query rows per request.
int validate_mask(const astr_paged_args* a, int64_t max_len, int64_t max_rows) {
  if (a->non_causal != 0 && a->non_causal != 1) return fail(ASTR_ERR_INVALID_ARG, "non_causal must be 0 or 1");
  if (a->mask == nullptr) return ASTR_OK;
  if ((reinterpret_cast<uintptr_t>(a->mask) & 3u) != 0 || a->mask_stride_req % 4 != 0 || a->mask_stride_row % 4 != 0)
    return fail(ASTR_ERR_INVALID_ARG, "the mask pointer and its strides must be multiples of 4 bytes");
  if (a->mask_stride_req < 0 || a->mask_stride_row < 0 || a->mask_stride_req > INT32_MAX)
    return fail(ASTR_ERR_INVALID_ARG, "mask strides must be in [0, 2^31)");
  const int64_t row_len = a->mask_stride_row == 0 ? a->mask_stride_req : a->mask_stride_row;
  if (row_len < max_len)
    return fail(ASTR_ERR_INVALID_ARG, "mask rows hold %lld entries but a request has %lld keys", (long long)row_len,
                (long long)max_len);
  if (a->mask_stride_row > 0 && a->mask_stride_req < max_rows * a->mask_stride_row)
    return fail(ASTR_ERR_INVALID_ARG, "mask_stride_req %lld is smaller than %lld query rows of %lld bytes",
                (long long)a->mask_stride_req, (long long)max_rows, (long long)a->mask_stride_row);
  return ASTR_OK;
}

int64_t max_seq_len(const astr_paged_args* a) {
  int64_t m = 0;
  for (int b = 0; b < a->batch; ++b) {
    const int64_t L = (int64_t)a->kv_indptr_host[b + 1] - a->kv_indptr_host[b];
    if (L > m) m = L;
  }
  return m;
}

// Bytes from a kv head's base to the end of that head's row in the last
// slot: (num_slots - 1) * kv_stride_slot * 2 + head_dim * 2.  The kernels
// take 32-bit buffer offsets when this is at most kPoolRange32 (the decode
// kernel's offsets above it are its out-of-range marker); prefill also needs
// slot ids and row strides below 2^24 for its 24-bit multiply.
constexpr int64_t kPoolRange32 = 0xFFFFF000;

int64_t pool_range_bytes(const astr_paged_args* a) {
  return (a->num_slots - 1) * a->kv_stride_slot * 2 + (int64_t)a->head_dim * 2;
}

// The caller's timing events i and i + 1 (either may be NULL) as the start
// and end stamps of one kernel.
astr::Timing timing_pair(void* const* events, int i) {
  astr::Timing t;
  if (events != nullptr) {
    t.start = static_cast<hipEvent_t>(events[i]);
    t.stop = static_cast<hipEvent_t>(events[i + 1]);
  }
  return t;
}

// Thread groups for the combine kernel: enough that each group folds one
// batch of 8 pieces (at most 8 groups) for the request with the most pieces.
// The count decides the order in which pieces are folded, so it must not
// depend on lengths when the plan is fixed (a captured graph replays with the
// count it was captured with): then it follows from num_splits alone (a
// request spans at most that many pieces).  An automatic plan takes it from
// the host copy of kv_indptr.
int32_t combine_groups(const astr_paged_args* a, int64_t total_keys, int64_t wh) {
  if (a->num_splits > 0) {
    const int64_t g = ceil_div(wh, 8);
    return (int32_t)(g < 1 ? 1 : (g > 8 ? 8 : g));
  }
  if (a->batch <= 0 || total_keys <= 0) return 1;
  const int64_t W = wh < total_keys ? wh : total_keys;
  const int32_t* kv = a->kv_indptr_host;
  int64_t most = 1;
  for (int32_t b = 0; b < a->batch; ++b) {
    // Work groups holding the request's first and last keys (ceil((x + 1) W / N) - 1).
    const int64_t wf = ceil_div(((int64_t)kv[b] + 1) * W, total_keys) - 1;
    const int64_t wl = ceil_div((int64_t)kv[b + 1] * W, total_keys) - 1;
    if (wl - wf + 1 > most) most = wl - wf + 1;
  }
  const int64_t g = ceil_div(most, 8);
  return (int32_t)(g < 1 ? 1 : (g > 8 ? 8 : g));
}

// Head blocks (of 64 * 4 / head_dim query heads each) per combine work group.
// Large grids launch faster as fewer, larger work groups (measured on MI355X,
// B = 256 and 32 query heads: 8.2 -> 5.6 us from 4096 work groups of one
// block to 1024 of four), small ones lose the parallelism (B = 1: 6.3 ->
// 8.2 us), so blocks are merged only while the grid keeps at least
// kCombineMinGroups work groups, and while groups x blocks fit in 1024
// threads.  The count changes which work group computes a head, not how.
constexpr int32_t kCombineMaxHeadBlocks = 4;
constexpr int64_t kCombineMinGroups = 1024;
int32_t combine_head_blocks(const astr_paged_args* a, int32_t groups) {
  const int32_t per_block = 64 * 4 / a->head_dim;
  const int64_t blocks = (a->num_qo_heads + per_block - 1) / per_block;
  int32_t n = 1;
  while (n < kCombineMaxHeadBlocks && 2 * n * groups <= 16 &&
         (int64_t)a->batch * ceil_div(blocks, 2 * (int64_t)n) >= kCombineMinGroups)
    n *= 2;
  return n;
}

int plan_decode_impl(const astr_paged_args* a, int64_t total_keys, int32_t num_cus, astr_decode_plan* out) {
  int64_t wh;
  if (a->num_splits > 0) {
    wh = a->num_splits;
  } else if (a->num_splits < 0) {
    return fail(ASTR_ERR_INVALID_ARG, "num_splits must be >= 0 (got %d)", a->num_splits);
  } else {
    const int64_t target = ceil_div(wg_per_cu(a->head_dim) * (int64_t)num_cus, a->num_kv_heads);
    const int64_t by_len = total_keys > 0 ? ceil_div(total_keys, kMinTokens) : 1;
    wh = target < by_len ? target : by_len;
    if (wh > ASTR_DEFAULT_MAX_SPLITS) wh = ASTR_DEFAULT_MAX_SPLITS;
    if (wh < 1) wh = 1;
  }
  if (wh > 65535) return fail(ASTR_ERR_INVALID_ARG, "num_splits %lld exceeds 65535", (long long)wh);
  out->num_splits = (int32_t)wh;
  out->num_partials = (int32_t)(wh + a->batch - 1);
  out->grid_x = (int32_t)wh;
  out->grid_y = a->num_kv_heads;
  out->grid_z = 1;
  out->workspace_bytes = a->batch > 0 ? partial_bytes(a->batch, a->num_qo_heads, a->head_dim, wh) : 0;
  return ASTR_OK;
}

// Prefill planner constants: key tiles of 64 keys, 128 (position, head) rows
// per work group, two work groups per CU (one at head_dim 256), chunks of at
// least kMinChunkTiles key tiles and at most kMaxChunks per query tile.
constexpr int64_t kPrefillKeyTile = 64;
constexpr int64_t kPrefillRows = 128;
#ifndef ASTR_PREFILL_MIN_CHUNK_TILES
#define ASTR_PREFILL_MIN_CHUNK_TILES 8
#endif
constexpr int64_t kMinChunkTiles = ASTR_PREFILL_MIN_CHUNK_TILES;
constexpr int32_t kMaxChunks = astr::kPrefillMaxChunks;
int64_t prefill_wg_per_cu(int32_t head_dim) { return head_dim == 256 ? 1 : 2; }

// Key tiles of query tile qt of a request (q_len qb, seq_len L).
int64_t prefill_tile_keys(int64_t qt, int64_t BQ, int64_t qb, int64_t L, bool non_causal) {
  const int64_t kv_end = non_causal ? L : L - qb + std::min(BQ * (qt + 1), qb);
  return ceil_div(kv_end, kPrefillKeyTile);
}

// The automatic prefill plan: the work list (request order, item prefixes)
// and the chunking.  Lengths come from the host copies, already validated
// (1 <= q_len <= seq_len).  split = false keeps every tile whole.
void plan_prefill_impl(const astr_paged_args* a, int32_t num_cus, bool split, astr::PrefillWork* w,
                       astr_prefill_plan* out) {
  memset(out, 0, sizeof(*out));
  w->num_reqs = 0;
  const int32_t B = a->batch;
  const int64_t G = a->num_qo_heads / a->num_kv_heads;
  const int64_t BQ = kPrefillRows / G;
  const bool nc = a->non_causal != 0;
  const int32_t* qo = a->qo_indptr_host;
  const int32_t* kv = a->kv_indptr_host;
  std::vector<int64_t> work(B), biggest(B);
  for (int32_t b = 0; b < B; ++b) {
    const int64_t qb = qo[b + 1] - qo[b], L = kv[b + 1] - kv[b];
    int64_t wsum = 0;
    for (int64_t qt = 0; qt * BQ < qb; ++qt) wsum += prefill_tile_keys(qt, BQ, qb, L, nc);
    work[b] = wsum;
  }
  const int64_t slots = prefill_wg_per_cu(a->head_dim) * (int64_t)(num_cus > 0 ? num_cus : 1);
  // The chunk length T: the shortest (at least kMinChunkTiles key tiles) at
  // which all items still fit in one round of work-group slots, so that every
  // chunk starts at once and the longest item is as short as one round
  // allows (measured: a plan that needs a second round, or one that leaves
  // slots idle with longer chunks, is slower).  When the whole tiles alone
  // fill the slots, nothing is split.
  std::vector<int64_t> nts;
  int64_t max_nt = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t qb = qo[b + 1] - qo[b], L = kv[b + 1] - kv[b];
    for (int64_t qt = 0; qt * BQ < qb; ++qt) {
      nts.push_back(prefill_tile_keys(qt, BQ, qb, L, nc));
      max_nt = std::max(max_nt, nts.back());
    }
  }
  auto items_at = [&](int64_t T) {
    int64_t n = 0;
    for (const int64_t nt : nts) n += std::min<int64_t>(kMaxChunks, ceil_div(nt, T));
    return n * a->num_kv_heads;
  };
  const bool splitting = split && items_at(std::max(kMinChunkTiles, max_nt)) <= slots;
  int64_t T = std::max(kMinChunkTiles, max_nt);
  if (splitting) {
    int64_t lo = kMinChunkTiles;
    while (lo < T) {
      const int64_t mid = (lo + T) / 2;
      if (items_at(mid) <= slots) T = mid; else lo = mid + 1;
    }
  }
  w->chunk_tiles = (int32_t)std::min<int64_t>(T, INT32_MAX);
  w->max_chunks = splitting ? kMaxChunks : 1;
  w->slices = a->num_kv_heads % 8 == 0 ? 8 : 1;
  const int64_t hs = a->num_kv_heads / w->slices;
  // A request's biggest work item: key tiles of its longest chunk or whole
  // tile.  Not always from the last query tile: a tile just over the chunk
  // length is cut in two halves, while the tile before it may stay whole.
  for (int32_t b = 0; b < B; ++b) {
    const int64_t qb = qo[b + 1] - qo[b], L = kv[b + 1] - kv[b];
    int64_t big = 0;
    for (int64_t qt = 0; qt * BQ < qb; ++qt) {
      const int64_t nt = prefill_tile_keys(qt, BQ, qb, L, nc);
      const int64_t ns = std::min<int64_t>(w->max_chunks, ceil_div(nt, w->chunk_tiles));
      big = std::max(big, ceil_div(nt, ns));
    }
    biggest[b] = big;
  }
  // Requests whose items are biggest first, then by total work (an
  // approximately longest-first dispatch order; inside a request the items
  // already come biggest first).
  std::vector<int32_t> order(B);
  for (int32_t b = 0; b < B; ++b) order[b] = b;
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    return biggest[x] != biggest[y] ? biggest[x] > biggest[y] : work[x] > work[y];
  });
  int64_t first = 0, split_first = 0, split_tiles = 0;
  for (int32_t r = 0; r < B; ++r) {
    const int32_t b = order[r];
    const int64_t qb = qo[b + 1] - qo[b], L = kv[b + 1] - kv[b];
    int64_t n_g = 0, nsp_g = 0;
    for (int64_t qt = 0; qt * BQ < qb; ++qt) {
      const int64_t nt = prefill_tile_keys(qt, BQ, qb, L, nc);
      const int64_t ns = std::min<int64_t>(w->max_chunks, ceil_div(nt, w->chunk_tiles));
      n_g += ns;
      if (ns > 1) {
        nsp_g += ns;
        ++split_tiles;
      }
    }
    astr::PrefillWorkReq& q = w->req[r];
    q.b = b;
    q.first = (int32_t)first;
    q.split_first = (int32_t)split_first;
    q.q0 = qo[b];
    q.q_len = (int32_t)qb;
    q.kv0 = kv[b];
    q.seq_len = (int32_t)L;
    first += hs * n_g;
    split_first += hs * nsp_g;
  }
  w->req[B] = astr::PrefillWorkReq{0, (int32_t)first, (int32_t)split_first, 0, 0, 0, 0};
  w->num_reqs = B;
  const int64_t split_slots = w->slices * split_first;
  if (split_slots > astr::kCounterWords) {
    // More split tiles than the workspace's counter region holds: keep every tile whole.
    plan_prefill_impl(a, num_cus, false, w, out);
    return;
  }
  out->num_items = (int32_t)(w->slices * first);
  out->split_tiles = (int32_t)(split_tiles * a->num_kv_heads);
  out->chunk_tiles = w->chunk_tiles;
  out->max_chunks = w->max_chunks;
  out->partial_bytes = split_slots * astr::prefill_partial_bytes(a->head_dim);
  out->workspace_bytes = split_slots > 0 ? astr::kCounterBytes + out->partial_bytes : 0;
}

// Whether a prefill call can take the work-list path (automatic plan, batch
// within the kernel-argument list, item counts within int32).
bool prefill_work_list_ok(const astr_paged_args* a) {
  if (a->max_q_len != 0 || a->batch < 1 || a->batch > astr::kMaxWorkReqs) return false;
  const int64_t BQ = kPrefillRows / (a->num_qo_heads / a->num_kv_heads);
  int64_t items = 0;
  for (int32_t b = 0; b < a->batch; ++b)
    items += ceil_div((int64_t)a->qo_indptr_host[b + 1] - a->qo_indptr_host[b], BQ) * kMaxChunks;
  return items * a->num_kv_heads < (int64_t(1) << 30);
}

}  // namespace

extern "C" {

const char* astr_last_error(void) { return astr::last_error(); }

int astr_abi_version(void) { return ASTR_ABI_VERSION; }

size_t astr_workspace_size(int32_t batch, int32_t num_qo_heads, int32_t head_dim, int32_t max_splits) {
  if (batch < 1 || num_qo_heads < 1 || head_dim < 1 || max_splits < 0) return 0;
  const int64_t cap = max_splits == 0 ? ASTR_DEFAULT_MAX_SPLITS : max_splits;
  return (size_t)partial_bytes(batch, num_qo_heads, head_dim, cap);
}

int astr_plan_decode(const astr_paged_args* a, int32_t num_cus, astr_decode_plan* out) {
  if (out == nullptr) return fail(ASTR_ERR_INVALID_ARG, "plan output is NULL");
  if (a == nullptr) return fail(ASTR_ERR_INVALID_ARG, "args is NULL");
  int64_t total = 0;
  if (a->num_splits == 0) {
    // The automatic plan needs the host copy of kv_indptr.
    if (a->batch < 0) return fail(ASTR_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", a->batch);
    if (a->batch > 0 && a->kv_indptr_host == nullptr) return fail(ASTR_ERR_INVALID_ARG, "kv_indptr_host is NULL");
    if (a->batch > 0) total = a->kv_indptr_host[a->batch] - a->kv_indptr_host[0];
  }
  if (num_cus <= 0) {
    int st = device_cu_count(&num_cus);
    if (st != ASTR_OK) return st;
  }
  if (a->num_kv_heads < 1) return fail(ASTR_ERR_INVALID_ARG, "num_kv_heads must be >= 1");
  const int st = plan_decode_impl(a, total, num_cus, out);
  return st == ASTR_OK ? ok() : st;
}

}  // extern "C"

namespace {

// The new-token rows of an append: pointers, alignment and strides.
int validate_new_kv(const astr_new_kv* nkv) {
  if (nkv == nullptr) return fail(ASTR_ERR_INVALID_ARG, "new_kv is NULL");
  if (nkv->k_new == nullptr || nkv->v_new == nullptr) return fail(ASTR_ERR_INVALID_ARG, "k_new and v_new must be set");
  if (!aligned16(nkv->k_new) || !aligned16(nkv->v_new))
    return fail(ASTR_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  if (nkv->stride_tok <= 0 || nkv->stride_tok % 8 != 0 || nkv->stride_head <= 0 || nkv->stride_head % 8 != 0)
    return fail(ASTR_ERR_INVALID_ARG, "new_kv strides must be positive multiples of 8 elements (got %lld, %lld)",
                (long long)nkv->stride_tok, (long long)nkv->stride_head);
  return ASTR_OK;
}

}  // namespace

// Decode, optionally with the fused append of one new token per request.
int astr::decode_impl(const astr_paged_args* a, const astr_new_kv* nkv, void* workspace, size_t workspace_bytes,
                      void* stream, bool use_scratch) {
  int64_t total = 0;
  int st = validate_common(a, false, &total);
  if (st != ASTR_OK) return st;
  if (nkv != nullptr) {
    st = validate_new_kv(nkv);
    if (st != ASTR_OK) return st;
  }
  if (a->qo_indptr != nullptr || a->qo_indptr_host != nullptr)
    return fail(ASTR_ERR_INVALID_ARG, "decode takes no qo_indptr (one query row per request)");
  if (a->batch == 0) return ok();
  st = validate_mask(a, max_seq_len(a), 1);
  if (st != ASTR_OK) return st;
  int num_cus = 0;
  if (a->num_splits == 0) {
    st = device_cu_count(&num_cus);
    if (st != ASTR_OK) return st;
  }
  astr_decode_plan plan;
  st = plan_decode_impl(a, total, num_cus, &plan);
  if (st != ASTR_OK) return st;
  if (use_scratch) {
    if (plan.workspace_bytes > (int64_t)ASTR_NOALLOC_SCRATCH_BYTES)
      return fail(ASTR_ERR_WORKSPACE,
                  "the plan needs %lld bytes of split partials (batch %d, %d query heads, head_dim %d, %d work groups "
                  "per kv head), more than the %lld-byte scratch of the allocation-free entry point; call "
                  "astr_paged_decode with a caller workspace instead",
                  (long long)plan.workspace_bytes, a->batch, a->num_qo_heads, a->head_dim, plan.num_splits,
                  (long long)ASTR_NOALLOC_SCRATCH_BYTES);
    const hipError_t se = astr::scratch_buffer(&workspace, &workspace_bytes);
    if (se != hipSuccess) return fail(ASTR_ERR_HIP, "scratch address (hipGetSymbolAddress): %s", hipGetErrorString(se));
  }
  if (workspace == nullptr) return fail(ASTR_ERR_WORKSPACE, "decode needs a workspace of %lld bytes", (long long)plan.workspace_bytes);
  if (!aligned16(workspace)) return fail(ASTR_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  if ((int64_t)workspace_bytes < plan.workspace_bytes)
    return fail(ASTR_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %lld bytes the plan needs", workspace_bytes,
                (long long)plan.workspace_bytes);

  astr::DecodeLaunch p;
  p.batch = a->batch;
  p.num_qo_heads = a->num_qo_heads;
  p.num_kv_heads = a->num_kv_heads;
  p.head_dim = a->head_dim;
  p.group = a->num_qo_heads / a->num_kv_heads;
  p.sm_scale = a->sm_scale;
  p.q = static_cast<const uint16_t*>(a->q);
  p.q_stride_tok = a->q_stride_tok;
  p.q_stride_head = a->q_stride_head;
  p.o = static_cast<uint16_t*>(a->o);
  p.o_stride_tok = a->o_stride_tok;
  p.o_stride_head = a->o_stride_head;
  p.lse = a->lse;
  p.lse_stride_tok = a->lse_stride_tok;
  p.k_pool = static_cast<const uint16_t*>(a->k_pool);
  p.v_pool = static_cast<const uint16_t*>(a->v_pool);
  p.kv_stride_slot = a->kv_stride_slot;
  p.kv_stride_head = a->kv_stride_head;
  p.req_to_token = a->req_to_token;
  p.req_to_token_stride = a->req_to_token_stride;
  p.kv_indptr = a->kv_indptr;
  const int64_t range = pool_range_bytes(a);
  p.off32 = range <= kPoolRange32;
  p.pool_range = p.off32 ? (uint32_t)range : 0u;
  p.num_splits = plan.num_splits;
  p.num_partials = plan.num_partials;
  p.combine_groups = combine_groups(a, total, plan.num_splits);
  p.combine_head_blocks = combine_head_blocks(a, p.combine_groups);
  p.o_part = static_cast<float*>(workspace);
  p.ml_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       align256((int64_t)a->num_qo_heads * plan.num_partials * a->head_dim * 4));
  p.k_new = nkv != nullptr ? static_cast<const uint16_t*>(nkv->k_new) : nullptr;
  p.v_new = nkv != nullptr ? static_cast<const uint16_t*>(nkv->v_new) : nullptr;
  p.new_stride_tok = nkv != nullptr ? nkv->stride_tok : 0;
  p.new_stride_head = nkv != nullptr ? nkv->stride_head : 0;
  p.num_slots = a->num_slots;
  p.mask = a->mask;
  p.mask_stride_req = a->mask_stride_req;
  p.page_shift = page_shift_of(a->page_size);

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = astr::launch_decode_split(p, s, timing_pair(a->timing_events, 0));
  if (e != hipSuccess) return fail(ASTR_ERR_HIP, "split kernel launch: %s", hipGetErrorString(e));
  e = astr::launch_decode_combine(p, s, timing_pair(a->timing_events, 2));
  if (e != hipSuccess) return fail(ASTR_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
  return ok();
}

extern "C" {

int astr_paged_decode(const astr_paged_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  return astr::decode_impl(a, nullptr, workspace, workspace_bytes, stream);
}

int astr_paged_decode_noalloc(const astr_paged_args* a, void* stream) {
  return astr::decode_impl(a, nullptr, nullptr, 0, stream, true);
}

int astr_paged_decode_append(const astr_paged_args* a, const astr_new_kv* nkv, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (nkv == nullptr) return fail(ASTR_ERR_INVALID_ARG, "new_kv is NULL");
  return astr::decode_impl(a, nkv, workspace, workspace_bytes, stream);
}

int astr_kv_append(const astr_paged_args* a, const astr_new_kv* nkv, void* stream) {
  if (a == nullptr) return fail(ASTR_ERR_INVALID_ARG, "args is NULL");
  int st = validate_new_kv(nkv);
  if (st != ASTR_OK) return st;
  if (a->batch < 0) return fail(ASTR_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", a->batch);
  if (a->num_kv_heads < 1) return fail(ASTR_ERR_INVALID_ARG, "num_kv_heads must be >= 1 (got %d)", a->num_kv_heads);
  if (a->head_dim < 8 || a->head_dim % 8 != 0)
    return fail(ASTR_ERR_INVALID_ARG, "head_dim must be a positive multiple of 8 (got %d)", a->head_dim);
  if (a->batch > 65535) return fail(ASTR_ERR_INVALID_ARG, "batch (%d) must be <= 65535 (grid limit)", a->batch);
  if (a->max_q_len < 0) return fail(ASTR_ERR_INVALID_ARG, "max_q_len must be >= 0");
  if (a->batch == 0) return ok();
  struct { const void* p; const char* name; } req[] = {
      {a->k_pool, "k_pool"}, {a->v_pool, "v_pool"}, {a->req_to_token, "req_to_token"},
      {a->kv_indptr, "kv_indptr"}, {a->kv_indptr_host, "kv_indptr_host"}};
  for (auto& r : req)
    if (r.p == nullptr) return fail(ASTR_ERR_INVALID_ARG, "%s is NULL", r.name);
  if (!aligned16(a->k_pool) || !aligned16(a->v_pool)) return fail(ASTR_ERR_INVALID_ARG, "k_pool and v_pool must be 16-byte aligned");
  if (a->kv_stride_slot <= 0 || a->kv_stride_slot % 8 != 0 || a->kv_stride_head <= 0 || a->kv_stride_head % 8 != 0)
    return fail(ASTR_ERR_INVALID_ARG, "kv strides must be positive multiples of 8 elements");
  if (a->num_slots < 1 || a->num_slots > (int64_t)INT32_MAX + 1)
    return fail(ASTR_ERR_INVALID_ARG, "num_slots must be in [1, 2^31] (got %lld)", (long long)a->num_slots);
  if (a->req_to_token_stride < 0) return fail(ASTR_ERR_INVALID_ARG, "req_to_token_stride must be >= 0");
  if ((a->qo_indptr == nullptr) != (a->qo_indptr_host == nullptr))
    return fail(ASTR_ERR_INVALID_ARG, "qo_indptr and qo_indptr_host must both be set or both be NULL");
  int shift = 0;
  st = validate_pages(a, &shift);
  if (st != ASTR_OK) return st;
  const int32_t* kv = a->kv_indptr_host;
  const int32_t* qo = a->qo_indptr_host;
  if (kv[0] != 0) return fail(ASTR_ERR_INVALID_ARG, "kv_indptr[0] must be 0 (got %d)", kv[0]);
  if (qo != nullptr && qo[0] != 0) return fail(ASTR_ERR_INVALID_ARG, "qo_indptr[0] must be 0 (got %d)", qo[0]);
  int64_t max_new = 0;
  for (int b = 0; b < a->batch; ++b) {
    const int64_t L = (int64_t)kv[b + 1] - kv[b];
    const int64_t n = qo != nullptr ? (int64_t)qo[b + 1] - qo[b] : 1;
    if (n < 1 || n > L)
      return fail(ASTR_ERR_INVALID_ARG, "request %d: need 1 <= new tokens <= seq_len (new %lld, seq_len %lld)", b,
                  (long long)n, (long long)L);
    if (a->req_to_token_stride > 0 && row_entries(L, shift) > a->req_to_token_stride)
      return fail(ASTR_ERR_INVALID_ARG, "request %d: seq_len %lld needs %lld table entries, more than req_to_token_stride %lld",
                  b, (long long)L, (long long)row_entries(L, shift), (long long)a->req_to_token_stride);
    if (n > max_new) max_new = n;
  }
  if (a->max_q_len > 0) {
    if (max_new > a->max_q_len)
      return fail(ASTR_ERR_INVALID_ARG, "a request appends %lld tokens, more than max_q_len %d", (long long)max_new,
                  a->max_q_len);
    max_new = a->max_q_len;
  }
  if (max_new * a->num_kv_heads * (a->head_dim / 8) > (int64_t)INT32_MAX)
    return fail(ASTR_ERR_INVALID_ARG, "too many new tokens per request for one launch");

  astr::AppendLaunch p;
  p.batch = a->batch;
  p.num_kv_heads = a->num_kv_heads;
  p.head_dim = a->head_dim;
  p.max_new = (int32_t)max_new;
  p.k_new = static_cast<const uint16_t*>(nkv->k_new);
  p.v_new = static_cast<const uint16_t*>(nkv->v_new);
  p.new_stride_tok = nkv->stride_tok;
  p.new_stride_head = nkv->stride_head;
  p.k_pool = static_cast<uint16_t*>(const_cast<void*>(a->k_pool));
  p.v_pool = static_cast<uint16_t*>(const_cast<void*>(a->v_pool));
  p.kv_stride_slot = a->kv_stride_slot;
  p.kv_stride_head = a->kv_stride_head;
  p.num_slots = a->num_slots;
  p.req_to_token = a->req_to_token;
  p.req_to_token_stride = a->req_to_token_stride;
  p.kv_indptr = a->kv_indptr;
  p.qo_indptr = a->qo_indptr;
  p.page_shift = shift;
  const hipError_t e = astr::launch_kv_append(p, static_cast<hipStream_t>(stream), timing_pair(a->timing_events, 0));
  if (e != hipSuccess) return fail(ASTR_ERR_HIP, "append kernel launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Prefill validation (everything but the workspace); *max_q receives the grid's
// query length (max q_len, or max_q_len when fixed).
int validate_prefill(const astr_paged_args* a, int32_t* max_q_out) {
  int64_t total = 0;
  int st = validate_common(a, true, &total);
  if (st != ASTR_OK) return st;
  *max_q_out = 0;
  if (a->batch == 0) return ASTR_OK;
  if (a->qo_indptr == nullptr || a->qo_indptr_host == nullptr)
    return fail(ASTR_ERR_INVALID_ARG, "prefill needs qo_indptr and qo_indptr_host");
  if (a->max_q_len < 0) return fail(ASTR_ERR_INVALID_ARG, "max_q_len must be >= 0");
  const int32_t* qo = a->qo_indptr_host;
  const int32_t* kv = a->kv_indptr_host;
  if (qo[0] != 0) return fail(ASTR_ERR_INVALID_ARG, "qo_indptr[0] must be 0 (got %d)", qo[0]);
  int32_t max_q = 0;
  for (int b = 0; b < a->batch; ++b) {
    const int64_t ql = (int64_t)qo[b + 1] - qo[b];
    const int64_t L = (int64_t)kv[b + 1] - kv[b];
    if (ql < 1 || ql > L)
      return fail(ASTR_ERR_INVALID_ARG, "request %d: need 1 <= q_len <= seq_len (q_len %lld, seq_len %lld)", b, (long long)ql,
                  (long long)L);
    if (ql > max_q) max_q = (int32_t)ql;
  }
  st = validate_mask(a, max_seq_len(a), max_q);
  if (st != ASTR_OK) return st;
  if (a->max_q_len > 0) {
    if (max_q > a->max_q_len)
      return fail(ASTR_ERR_INVALID_ARG, "a q_len of %d exceeds max_q_len %d", max_q, a->max_q_len);
    max_q = a->max_q_len;
  }
  *max_q_out = max_q;
  return ASTR_OK;
}

}  // namespace

extern "C" {

int astr_plan_prefill(const astr_paged_args* a, int32_t num_cus, astr_prefill_plan* out) {
  if (out == nullptr) return fail(ASTR_ERR_INVALID_ARG, "plan output is NULL");
  memset(out, 0, sizeof(*out));
  int32_t max_q = 0;
  int st = validate_prefill(a, &max_q);
  if (st != ASTR_OK) return st;
  if (!prefill_work_list_ok(a)) return ok();
  if (num_cus <= 0) {
    st = device_cu_count(&num_cus);
    if (st != ASTR_OK) return st;
  }
  static thread_local astr::PrefillWork w;
  plan_prefill_impl(a, num_cus, true, &w, out);
  return ok();
}

int astr_paged_prefill(const astr_paged_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  int32_t max_q = 0;
  int st = validate_prefill(a, &max_q);
  if (st != ASTR_OK) return st;
  if (a->batch == 0) return ok();

  astr::PrefillLaunch p;
  memset(&p.work, 0, sizeof(p.work));
  p.part = nullptr;
  p.cnt = nullptr;
  p.part_bytes = 0;
  if (prefill_work_list_ok(a)) {
    int num_cus = 0;
    st = device_cu_count(&num_cus);
    if (st != ASTR_OK) return st;
    astr_prefill_plan plan;
    plan_prefill_impl(a, num_cus, workspace != nullptr, &p.work, &plan);
    if (plan.workspace_bytes > 0) {
      if (!aligned16(workspace)) return fail(ASTR_ERR_WORKSPACE, "workspace must be 16-byte aligned");
      if ((int64_t)workspace_bytes < plan.workspace_bytes)
        return fail(ASTR_ERR_WORKSPACE,
                    "prefill workspace of %zu bytes is smaller than the %lld bytes its split plan needs "
                    "(pass NULL to keep every query tile whole)",
                    workspace_bytes, (long long)plan.workspace_bytes);
      if (plan.partial_bytes > (int64_t)UINT32_MAX) {
        // Beyond one 32-bit buffer range: keep every tile whole.
        plan_prefill_impl(a, num_cus, false, &p.work, &plan);
      } else {
        p.cnt = static_cast<int32_t*>(workspace);
        p.part = static_cast<char*>(workspace) + astr::kCounterBytes;
        p.part_bytes = (uint32_t)plan.partial_bytes;
      }
    }
  }
  p.batch = a->batch;
  p.num_qo_heads = a->num_qo_heads;
  p.num_kv_heads = a->num_kv_heads;
  p.head_dim = a->head_dim;
  p.group = a->num_qo_heads / a->num_kv_heads;
  p.sm_scale = a->sm_scale;
  p.q = static_cast<const uint16_t*>(a->q);
  p.q_stride_tok = a->q_stride_tok;
  p.q_stride_head = a->q_stride_head;
  p.o = static_cast<uint16_t*>(a->o);
  p.o_stride_tok = a->o_stride_tok;
  p.o_stride_head = a->o_stride_head;
  p.lse = a->lse;
  p.lse_stride_tok = a->lse_stride_tok;
  p.k_pool = static_cast<const uint16_t*>(a->k_pool);
  p.v_pool = static_cast<const uint16_t*>(a->v_pool);
  p.kv_stride_slot = a->kv_stride_slot;
  p.kv_stride_head = a->kv_stride_head;
  p.req_to_token = a->req_to_token;
  p.req_to_token_stride = a->req_to_token_stride;
  p.kv_indptr = a->kv_indptr;
  p.qo_indptr = a->qo_indptr;
  p.max_q_len = max_q;
  p.non_causal = a->non_causal != 0;
  p.mask = a->mask;
  p.mask_stride_req = a->mask_stride_req;
  p.mask_stride_row = a->mask_stride_row;
  p.page_shift = page_shift_of(a->page_size);
  const int64_t range = pool_range_bytes(a);
  p.off32 = range <= kPoolRange32 && a->num_slots <= (int64_t(1) << 24) && a->kv_stride_slot * 2 < (int64_t(1) << 24);
  p.pool_range = p.off32 ? (uint32_t)range : 0u;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = astr::launch_prefill(p, s, timing_pair(a->timing_events, 0));
  if (e != hipSuccess) return fail(ASTR_ERR_HIP, "prefill kernel launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
