// KV append for gfx950: writes the K/V rows of a step's new tokens into the
// token-slot pools before they are attended.
//
// Method (AstrAI commit-list pages): [attention_backend.py @47b3ed4], the
// commit that shares one write-then-gather K/V helper between backends;
// [extension @6f67ba8], the paged decode commit (position t of request b is
// pool slot req_to_token[row_b + t], page size one); [attention.py @c9ceca1],
// the batched torch path (a request's q_len new tokens are its last
// positions, stored in flat qo_indptr order).  kv_indptr already counts the
// new tokens.
//
// Grid (ceil(max_new * Hkv * D / 8 / 256), B): thread x of request b's
// column copies one 16-byte chunk of K and the same chunk of V of new token
// i = x / (Hkv * D / 8), kv head (x / (D / 8)) % Hkv.  Consecutive threads
// cover one contiguous 2*D-byte head row after another, so both the reads of
// the new rows and the writes of the pool rows are whole 64-byte segments.
// The work is a copy (HBM-bound: 8 * D * Hkv bytes per new token, its rows
// read once and written once, plus one slot id).  A decode step's append is
// a few hundred kilobytes and runs at launch latency, which is why decode
// also has a fused form.
#include "device_common.hpp"
#include "kernel_launch.hpp"

namespace astr {
namespace {

constexpr int kAppendThreads = 256;

__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(const AppendLaunch p) {
  const int b = blockIdx.y;
  const int chunks_per_head = p.head_dim / 8;
  const int chunks_per_tok = p.num_kv_heads * chunks_per_head;
  const int64_t x = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
  const int i = (int)(x / chunks_per_tok);
  const int c = (int)(x % chunks_per_tok);
  const int g = c / chunks_per_head;
  const int dc = c % chunks_per_head;
  const int64_t kv0 = p.kv_indptr[b];
  const int64_t L = (int64_t)p.kv_indptr[b + 1] - kv0;
  const int64_t row0 = p.qo_indptr != nullptr ? (int64_t)p.qo_indptr[b] : (int64_t)b;
  const int64_t n = p.qo_indptr != nullptr ? (int64_t)p.qo_indptr[b + 1] - row0 : 1;
  if (i >= n) return;
  const int64_t rowb = p.req_to_token_stride > 0 ? (int64_t)b * p.req_to_token_stride : kv0;
  const int64_t pos = L - n + i;
  const int32_t slot = (p.req_to_token[rowb + (pos >> p.page_shift)] << p.page_shift) +
                       (int32_t)(pos & ((1 << p.page_shift) - 1));
  if (slot < 0 || (int64_t)slot >= p.num_slots) return;   // outside the pool: nothing is written
  const int64_t src = (row0 + i) * p.new_stride_tok + (int64_t)g * p.new_stride_head + 8 * dc;
  const int64_t dst = (int64_t)slot * p.kv_stride_slot + (int64_t)g * p.kv_stride_head + 8 * dc;
  const uint4 kv = *reinterpret_cast<const uint4*>(p.k_new + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(p.v_new + src);
  *reinterpret_cast<uint4*>(p.k_pool + dst) = kv;
  *reinterpret_cast<uint4*>(p.v_pool + dst) = vv;
}

}  // namespace

hipError_t launch_kv_append(const AppendLaunch& p, hipStream_t s, const Timing& t) {
  const int64_t chunks = (int64_t)p.max_new * p.num_kv_heads * (p.head_dim / 8);
  const dim3 grid((unsigned)((chunks + kAppendThreads - 1) / kAppendThreads), (unsigned)p.batch, 1);
  return launch_kernel(kv_append_kernel, grid, dim3(kAppendThreads), s, t, p);
}

}  // namespace astr
