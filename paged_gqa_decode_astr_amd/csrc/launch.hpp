// Host-side launch descriptors shared by the C ABI layer and the HIP kernels.
// Plain structs: every field is already validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace astr {

// Arrival counters at the start of a prefill workspace, one per split query
// tile.  They must be zero before the first call on a workspace and every
// call leaves them zero; a fixed region, so that calls with different plans
// can share one workspace (a counter never lands on an earlier call's
// partials).  The chunk partials follow it.
constexpr int64_t kCounterWords = 8192;
constexpr int64_t kCounterBytes = kCounterWords * 4;

struct DecodeLaunch {
  int32_t batch, num_qo_heads, num_kv_heads, head_dim, group;
  float sm_scale;
  const uint16_t* q;
  int64_t q_stride_tok, q_stride_head;
  uint16_t* o;
  int64_t o_stride_tok, o_stride_head;
  float* lse;
  int64_t lse_stride_tok;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  int64_t kv_stride_slot, kv_stride_head;
  const int32_t* req_to_token;
  int64_t req_to_token_stride;
  const int32_t* kv_indptr;
  bool off32;            // every pool row of a kv head lies within pool_range bytes of its base
  uint32_t pool_range;   // off32: (num_slots - 1) * kv_stride_slot * 2 + head_dim * 2
  int32_t num_splits;    // Wh: work groups per kv head (grid.x)
  int32_t num_partials;  // P = Wh + B - 1 slots per query head
  int32_t combine_groups;  // thread groups of the combine kernel per head block (1..8)
  int32_t combine_head_blocks;  // head blocks per combine work group (groups x blocks <= 16)
  float* o_part;         // [Hq][P][D]
  float* ml_part;        // [Hq][P][2]
  // Fused KV append (decode_append): the new token of request b is its last
  // key; its rows come from k_new / v_new row b and are written to the pools.
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t new_stride_tok, new_stride_head;
  int64_t num_slots;
  // Optional uint8 mask (row 0 of each request's block): key t of request b
  // is hidden when mask[b * mask_stride_req + t] == 0.
  const uint8_t* mask;
  int64_t mask_stride_req;
  int32_t page_shift;    // log2 page size: slot = (req_to_token[row + t >> s] << s) + (t & (2^s - 1))
};

// KV append: n_b new tokens per request (1 when qo_indptr is null), written
// to pool slots req_to_token[row_b + L_b - n_b + i].
struct AppendLaunch {
  int32_t batch, num_kv_heads, head_dim;
  int32_t max_new;       // grid covers new tokens [0, max_new) of each request
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t new_stride_tok, new_stride_head;
  uint16_t* k_pool;
  uint16_t* v_pool;
  int64_t kv_stride_slot, kv_stride_head, num_slots;
  const int32_t* req_to_token;
  int64_t req_to_token_stride;
  const int32_t* kv_indptr;
  const int32_t* qo_indptr;   // null: one new token per request
  int32_t page_shift;         // log2 page size (see DecodeLaunch)
};

// Work list of an automatic prefill plan, passed by value in the kernel
// arguments (so a work group knows its request and key range without a
// round trip to memory).  A query tile's key range is cut into ns
// near-equal chunks, ns = min(max_chunks, ceil(key tiles / chunk_tiles));
// each chunk is one work item.  Items are laid out in `slices` interleaved
// sequences (8 when Hkv is a multiple of 8: block i runs on accelerator die
// i % 8 and slice i % 8 holds kv heads g = i % 8 + 8 k, so every item of one
// (request, kv head) group shares that die's L2; otherwise 1).  Inside a
// slice, requests follow req[0 .. num_reqs) and each request holds, for
// each of its kv heads in the slice, the group's items: query tiles from the
// last (most keys) down, chunks of a tile consecutive.  The tiles that are
// split come first in a group, and their chunks own the partial slots.
constexpr int kMaxWorkReqs = 96;
constexpr int kPrefillMaxChunks = 16;  // most key chunks per query tile
struct PrefillWorkReq {
  int32_t b;            // request index
  int32_t first;        // items of the slice before this request
  int32_t split_first;  // split-tile chunks of the slice before this request
  int32_t q0, q_len;    // qo_indptr[b], q_len_b
  int32_t kv0, seq_len; // kv_indptr[b], L_b
};
struct PrefillWork {
  int32_t num_reqs;     // 0: no work list (the kernel reads lengths from device memory)
  int32_t slices;       // 8 or 1
  int32_t chunk_tiles;  // T (key tiles of 64)
  int32_t max_chunks;   // 1 = no split
  PrefillWorkReq req[kMaxWorkReqs + 1];   // entry num_reqs holds the totals (first, split_first)
};

struct PrefillLaunch {
  int32_t batch, num_qo_heads, num_kv_heads, head_dim, group;
  float sm_scale;
  const uint16_t* q;
  int64_t q_stride_tok, q_stride_head;
  uint16_t* o;
  int64_t o_stride_tok, o_stride_head;
  float* lse;
  int64_t lse_stride_tok;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  int64_t kv_stride_slot, kv_stride_head;
  const int32_t* req_to_token;
  int64_t req_to_token_stride;
  const int32_t* kv_indptr;
  const int32_t* qo_indptr;
  int32_t max_q_len;     // grid covers query positions [0, max_q_len)
  bool non_causal;       // every row sees all L_b keys
  // Optional uint8 mask: key t hidden from row i of request b when
  // mask[b * mask_stride_req + i * mask_stride_row + t] == 0 (4-byte aligned).
  const uint8_t* mask;
  int64_t mask_stride_req, mask_stride_row;
  int32_t page_shift;    // log2 page size (see DecodeLaunch)
  bool off32;            // 32-bit buffer offsets: pool rows of a kv head within pool_range bytes, slot ids < 2^24
  uint32_t pool_range;   // off32: (num_slots - 1) * kv_stride_slot * 2 + head_dim * 2
  // Split tiles (work.max_chunks > 1): partial (acc, max, sum) of every chunk
  // in slot part[split slot] (prefill_partial_bytes(head_dim) each) and one
  // arrival counter per split tile in cnt[] (zero before the call; the chunk
  // that arrives last merges the tile and sets it back to zero).
  char* part;
  int32_t* cnt;
  uint32_t part_bytes;   // bytes of the partial area (buffer range)
  PrefillWork work;
};

// Bytes of one chunk's partial: per wavefront, row block and d block the
// lanes' fp32 accumulators, then per wavefront and row block the lanes'
// (reference max, row sum).  128 rows per work group.
constexpr int64_t prefill_partial_bytes(int head_dim) {
  return 4 * 2 * (head_dim / 16) * 64 * 16 + 4 * 2 * 64 * 8;
}

// Optional events stamped by the dispatch itself at the kernel's start and
// end (hipExtLaunchKernel), so their difference is the kernel's own duration.
struct Timing {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Each returns the launch status (hipGetLastError after the launch).
hipError_t launch_decode_split(const DecodeLaunch& p, hipStream_t stream, const Timing& t);
hipError_t launch_decode_combine(const DecodeLaunch& p, hipStream_t stream, const Timing& t);
hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream, const Timing& t);
hipError_t launch_kv_append(const AppendLaunch& p, hipStream_t stream, const Timing& t);

// Device address and size of the library's scratch array on the current
// device (astr_paged_decode_noalloc's partials); the address is taken once per
// device with hipGetSymbolAddress and cached.
hipError_t scratch_buffer(void** out, size_t* bytes);

// Whether a (head_dim, group) pair has a compiled kernel.
bool decode_supported(int head_dim, int group);
bool prefill_supported(int head_dim, int group);

}  // namespace astr
