// Ragged paged GQA prefill for gfx950 on the matrix cores.
//
// Method (AstrAI commit-list pages): [attention.py @c9ceca1], the commit that
// batches the torch path: query row i of request b sits at absolute position
// c_b + i with c_b = seq_len_b - q_len_b and sees keys 0 .. c_b + i; masked
// keys weigh exactly zero; rows are read and written in flat qo_indptr order.
// [extension @6f67ba8]: K/V come through req_to_token with page size one; the
// prefill kernel tiles over queries and uses matrix instructions for QK^T and
// PV; query head h reads kv head h / G.
//
// Work group = (query tile, kv head g, request b) on a 1-D grid laid out
// for the per-XCD L2s (see the work-item mapping below).  The G query heads
// that share kv head g are stacked with the positions into 128 rows (row
// R = position * G + head), so each K/V tile staged in LDS serves all of
// them.  Up to head_dim 128 a work group is 4 wavefronts and wavefront w owns
// rows 32 w .. 32 w + 31 as two 16-row blocks; at head_dim 256 it is 8
// wavefronts of one 16-row block each (see prefill_row_blocks).
// Per 64-key tile:
//   * K and V rows are gathered through req_to_token straight into LDS
//     (global_load_lds, 16 bytes per lane) one tile ahead, slot ids one more
//     tile ahead, into the other of two stage buffers, so a single wait and
//     barrier per tile separates producers and consumers.  Rows are D
//     elements, unpadded; the 16-byte chunk c of row r sits at chunk
//     c ^ swz(r) (swz = 2 (r % 8) for D = 128), which keeps both the K operand
//     reads and the transposing V reads free of bank conflicts;
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = Q^T
//     held in registers): lane l gets the logits of keys 4*(l/16)..+3 of each
//     16-key block for row l % 16, so a row's max needs two cross-lane steps;
//   * softmax in base 2 against a lazily raised per-row reference (the
//     accumulators are rescaled only when a logit exceeds it by more than
//     kTau), weights rounded to bf16; the row sums of the rounded weights come
//     from one more MFMA per 32 keys with an all-ones A operand, so the output
//     is an exact convex combination of the bf16-weighted rows;
//   * O^T += V^T P^T on v_mfma_f32_16x16x32_bf16: P^T is already in the
//     B-operand layout (k = 8*(l/16) + e covers keys 4*(l/16) + e of two
//     adjacent 16-key blocks), and V^T is read from the V tile with
//     two transposing LDS reads (ds_read_b64_tr_b16) that follow the same key
//     order.
// Output rows are normalised by the row sum and written as bf16 (round to
// nearest even); lse = reference + log2(sum), returned in natural-log units.
//
// Split key ranges (automatic plan with a workspace): the query tiles with the
// most keys bound the kernel's time (every work group of a batch like
// prefill_b8 is resident at once, and the tiles of long cached prefixes see
// up to ~6x the keys of the short ones), so the host cuts each tile's key
// tiles into ns near-equal chunks of about chunk_tiles and runs each chunk as
// its own work group.  A chunk leaves its unnormalised accumulators, reference
// max and row sums in a workspace slot (written, then released at agent
// scope) and counts itself on the tile's arrival counter; the chunk that
// arrives last reads the other chunks' slots with agent-coherent loads,
// merges them with its own registers by the log-sum-exp rule and writes the
// tile's rows.  Nothing waits on another work group.  The host passes the
// work list (request order, per-request item prefixes and lengths) in the
// kernel arguments, so a work group knows its request, tile and key range
// before its first memory access.
#include "device_common.hpp"
#include "kernel_launch.hpp"

#include <type_traits>

namespace astr {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

// Optional phase stamps (built only with ASTR_PHASE_STAMPS=1, into a
// separate library; the library as shipped has none of this code): every
// wavefront of the first kStampWgs work groups adds up, per phase of the tile
// loop, the shader-clock cycles (s_memtime) it spends -- issuing the next
// tile's gather, S = K Q^T with the softmax, P.V, waiting for the gather, the
// barrier -- and counts its tiles.
#ifndef ASTR_PHASE_STAMPS
#define ASTR_PHASE_STAMPS 0
#endif
constexpr bool kStamps = ASTR_PHASE_STAMPS != 0;
constexpr int kStampWgs = 4096;
constexpr int kStampPhases = 6;   // gather issue, S + softmax, P.V, gather wait, barrier, tiles
#if ASTR_PHASE_STAMPS
__device__ unsigned long long g_prefill_stamps[kStampWgs][8][kStampPhases];
#endif

constexpr int kRows = 128;       // (position, head) rows per work group
// 16-row blocks per wavefront: two up to head_dim 128 (each K and V operand
// read from LDS feeds two MFMAs), one at 256, where two blocks' accumulators
// and operands overflowed the registers of the one wavefront per SIMD that
// fit; with one block the work group has 8 wavefronts, two per SIMD.
template <int D>
constexpr int prefill_row_blocks() { return D == 256 ? 1 : 2; }
template <int D>
constexpr int prefill_waves() { return kRows / (16 * prefill_row_blocks<D>()); }   // per work group
template <int D>
constexpr int prefill_threads() { return prefill_waves<D>() * kWave; }
constexpr int KT = 64;           // keys per tile
constexpr float kTau = 8.0f;     // log2 headroom before the accumulators are rescaled
constexpr int kXcds = 8;         // accelerator dies a launch is dealt across

__device__ __forceinline__ uint4 load16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ f32x4 mfma32k(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D>
struct PShape {
  static constexpr int kSteps = D / 32;                        // k-steps of S^T = K Q^T
  static constexpr int kDBlocks = D / 16;                      // 16-wide d blocks of O^T
};

typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
// Cache-policy operand of a buffer access: sc1 = coherent at agent scope
// (the loads see what other work groups released at agent scope, on any XCD).
constexpr int kScopeAgent = 16;

// Waves per SIMD the kernel is built for: two (two 4-wavefront work groups
// per CU up to head_dim 128; one 8-wavefront work group at 256, whose K/V
// stages take 128 KB of LDS).
template <int D>
constexpr int prefill_waves_per_simd() { return 2; }

// The (query tile, chunk) a work group runs and its key tiles [it_lo, it_hi).
struct PrefillItem {
  int b, g, qt;
  int q0, qb, kv0, L;
  int s, ns;             // chunk s of ns (ns == 1: the whole tile)
  int it_lo, it_hi;
  int slot, tile_slot;   // split tiles: this chunk's partial slot, the tile's counter (its chunk 0's slot)
};

// Key tiles of query tile qt (all rows of it) and their chunk count.
__device__ __forceinline__ int tile_key_tiles(int qt, int BQ, int qb, int L, bool non_causal) {
  const int kv_end = non_causal ? L : L - qb + min(BQ * (qt + 1), qb);
  return (kv_end + KT - 1) / KT;
}
__device__ __forceinline__ int tile_chunks(int nt, const PrefillWork& w) {
  return min(w.max_chunks, (nt + w.chunk_tiles - 1) / w.chunk_tiles);
}

template <int D, int G, bool OFF32, bool MASK, bool WORK>
__global__ __launch_bounds__(prefill_threads<D>()) __attribute__((amdgpu_waves_per_eu(prefill_waves_per_simd<D>()))) void prefill_kernel(const PrefillLaunch p) {
  using S = PShape<D>;
  constexpr int BQ = kRows / G;   // query positions per work group
  constexpr int NS = S::kSteps;
  constexpr int NB = S::kDBlocks;
  constexpr int kRB = prefill_row_blocks<D>();
  constexpr int kWavesWg = prefill_waves<D>();
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // Two stages, each its own array, so that the compiler can tell the LDS
  // DMA into one stage from the reads of the other.
  __shared__ __align__(16) uint16_t sK0[KT * D];
  __shared__ __align__(16) uint16_t sK1[KT * D];
  __shared__ __align__(16) uint16_t sV0[KT * D];
  __shared__ __align__(16) uint16_t sV1[KT * D];

  PrefillItem it;
  if constexpr (WORK) {
    // Work list in the kernel arguments: slice x = blockIdx % slices, position
    // j = blockIdx / slices in it; the request holding j is the number of
    // requests after the first whose item prefix is <= j (a ballot over the
    // prefixes, two per lane).
    const PrefillWork& w = p.work;
    const int S_ = w.slices;
    const int x = blockIdx.x % S_;
    const int j = blockIdx.x / S_;
    static_assert(kMaxWorkReqs <= 2 * kWave, "two prefixes per lane");
    int cnt = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 1 + lane + kWave * h;
      const int f = w.req[min(i, kMaxWorkReqs)].first;   // in bounds for every lane
      cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(i < w.num_reqs && f <= j));
    }
    const int r = __builtin_amdgcn_readfirstlane(cnt);
    const PrefillWorkReq rq = w.req[r];
    const int hs = p.num_kv_heads / S_;                           // kv heads of the request in this slice
    const int n_g = (w.req[r + 1].first - rq.first) / hs;         // items of one (request, kv head) group
    const int nsp_g = (w.req[r + 1].split_first - rq.split_first) / hs;   // of which chunks of split tiles
    const int local = j - rq.first;
    const int gi = local / n_g;
    const int k = local - gi * n_g;
    it.b = rq.b;
    it.g = x + S_ * gi;
    it.q0 = rq.q0;
    it.qb = rq.q_len;
    it.kv0 = rq.kv0;
    it.L = rq.seq_len;
    // Walk the group's tiles from the last one down to the k-th item.
    int qt = (it.qb + BQ - 1) / BQ - 1;
    int before = 0, nt = 0, ns = 1;
    for (;; --qt) {
      nt = tile_key_tiles(qt, BQ, it.qb, it.L, p.non_causal);
      ns = tile_chunks(nt, w);
      if (k < before + ns || qt == 0) break;
      before += ns;
    }
    it.qt = qt;
    it.s = k - before;
    it.ns = ns;
    it.it_lo = nt * it.s / ns;
    it.it_hi = nt * (it.s + 1) / ns;
    const int split_base = rq.split_first + gi * nsp_g;
    it.slot = (split_base + k) * S_ + x;
    it.tile_slot = (split_base + before) * S_ + x;
  } else {
    // Fixed grid (lengths from device memory).  Consecutive work groups are
    // dealt to the 8 XCDs in turn, and each XCD has its own L2, so the linear
    // id is remapped to keep every query tile of one (kv head, request) group
    // on one XCD: the group's K/V tiles then come from HBM once and from that
    // L2 for the other query tiles.  Groups are spread over the XCDs round
    // robin, and within a group the tiles with the most keys start first.
    const int nq = p.max_q_len > 0 ? (p.max_q_len + BQ - 1) / BQ : 0;
    const int ngroups = p.num_kv_heads * p.batch;
    if (nq == 0) return;
    const int xcd = blockIdx.x % kXcds;
    const int j = blockIdx.x / kXcds;
    const int grp = xcd + kXcds * (j / nq);
    if (grp >= ngroups) return;  // padding of the last round; uniform
    it.qt = nq - 1 - j % nq;
    it.g = grp % p.num_kv_heads;
    it.b = grp / p.num_kv_heads;
    it.q0 = p.qo_indptr[it.b];
    it.qb = p.qo_indptr[it.b + 1] - it.q0;
    if (it.qt * BQ >= it.qb) return;  // uniform over the work group
    it.kv0 = p.kv_indptr[it.b];
    it.L = p.kv_indptr[it.b + 1] - it.kv0;
    it.s = 0;
    it.ns = 1;
    it.it_lo = 0;
    it.it_hi = tile_key_tiles(it.qt, BQ, it.qb, it.L, p.non_causal);
    it.slot = it.tile_slot = 0;
  }
  const int b = it.b, g = it.g, qt = it.qt, q0 = it.q0, qb = it.qb, L = it.L;
  const int p0 = qt * BQ;
  const int cofs = L - qb;              // absolute position of query row 0
  const int npos = min(BQ, qb - p0);    // valid positions in this tile
  // Keys [0, kv_end) are visible to some row (all L keys when non-causal).
  const int kv_end = p.non_causal ? L : cofs + p0 + npos;
  const int it_lo = it.it_lo, it_hi = it.it_hi;
  const int32_t* ids = p.req_to_token + (p.req_to_token_stride > 0 ? (int64_t)b * p.req_to_token_stride : (int64_t)it.kv0);

  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l16 = lane & 15;
  const int kb = lane >> 4;

  // Gather: each tile row (key) is D bf16 in LDS, split into CPR 16-byte
  // chunks stored XOR-swizzled (chunk c of row r at position c ^ swz(r)) so
  // that the MFMA operand reads and the transposing V reads hit distinct
  // banks.  Load instruction i of wavefront wv fills the 1 KB block of rows
  // RPI (NI wv + i) .. + RPI - 1 straight from HBM (global_load_lds: lane l
  // lands at block + 16 l), so lane l fetches row RPI (NI wv + i) + l / CPR,
  // global chunk (l % CPR) ^ swz(row).  Keys past kv_end re-read key
  // kv_end - 1 (finite data; every row masks them).
  // OFF32: buffer loads over the kv head's rows (and the request's slot ids)
  // with 32-bit offsets, one 24-bit multiply-add per key; otherwise 64-bit
  // global addresses.
  constexpr int CPR = D / 8;
  constexpr int RPI = kWave / CPR;
  constexpr int NT = KT / RPI;                                   // load instructions per K (or V) tile
  constexpr int NI = NT >= kWavesWg ? NT / kWavesWg : 1;          // per wavefront
  static_assert(NT % NI == 0 && NT / NI <= kWavesWg, "tile rows split evenly over the loading wavefronts");
  // When a tile is fewer load instructions than there are wavefronts, only
  // the first NT / NI wavefronts gather (uniform per wavefront); otherwise
  // the test is compiled out (a branch there cost the head_dim 128 kernel 7%).
  [[maybe_unused]] const bool loader = NI * wv < NT;
  constexpr bool kSomeIdle = NT < kWavesWg;
  // The swizzle stays below the row's chunk count: at D = 32 a row has only
  // 4 chunks, and an XOR value of 4 or more would address the next row.
  auto swz = [](int r) { return D >= 128 ? 2 * (r & 7) : (D == 64 ? 2 * ((r >> 1) & 3) : (r >> 1) & 3); };
  const int grow0 = RPI * NI * wv + lane / CPR;
  int gchunk[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) gchunk[i] = (lane % CPR) ^ swz(grow0 + RPI * i);
  const int64_t head_off = (int64_t)g * p.kv_stride_head;
  __amdgpu_buffer_rsrc_t krs, vrs, irs;
  uint32_t row_bytes = 0;
  if constexpr (OFF32) {
    krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.k_pool + head_off), (short)0, (int)p.pool_range, 0x00020000);
    vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.v_pool + head_off), (short)0, (int)p.pool_range, 0x00020000);
    irs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(ids), (short)0,
                                            4 * (((kv_end - 1) >> p.page_shift) + 1), 0x00020000);
    row_bytes = (uint32_t)(p.kv_stride_slot * 2);
  }
  int id_next[NI];
  auto load_ids = [&](int t0) {
    if constexpr (kSomeIdle) {
      if (!loader) return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = min(t0 + grow0 + RPI * i, kv_end - 1);
      // The table entry only; gather adds the page arithmetic where the slot is used.
      if constexpr (OFF32) id_next[i] = __builtin_amdgcn_raw_buffer_load_b32(irs, 4 * (t >> p.page_shift), 0, 0);
      else id_next[i] = ids[t >> p.page_shift];
    }
  };
  // Tile starting at key t0: slot of row i's key from its table entry.
  auto gather = [&](uint16_t* kdst, uint16_t* vdst, int t0) {
    if constexpr (kSomeIdle) {
      if (!loader) return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row0 = RPI * (NI * wv + i);
      const int slot = (id_next[i] << p.page_shift) +
                       (min(t0 + grow0 + RPI * i, kv_end - 1) & ((1 << p.page_shift) - 1));
      if constexpr (OFF32) {
        const uint32_t voff = __umul24((uint32_t)slot, row_bytes) + 16u * gchunk[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kdst + row0 * D), 16, voff, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(vdst + row0 * D), 16, voff, 0, 0, 0);
      } else {
        const int64_t off = (int64_t)slot * p.kv_stride_slot + head_off + 8 * gchunk[i];
        __builtin_amdgcn_global_load_lds(p.k_pool + off, (lds_void*)(kdst + row0 * D), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(p.v_pool + off, (lds_void*)(vdst + row0 * D), 16, 0, 0);
      }
    }
  };
  // Every wavefront waits for its own loads of a stage, then the barrier
  // makes the whole tile visible.
  auto stage_ready = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // The first tile of the range into stage 0, the next tile's slot ids behind it.
  load_ids(it_lo * KT);
  gather(sK0, sV0, it_lo * KT);
  load_ids((it_lo + 1) * KT);

  // B operand of S^T = K Q^T: lane (r + 16 kb) holds Q[row r][32 ks + 8 kb .. +7] of each row block.
  bf16x8 qop[kRB][NS];
  int lim[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int R = 16 * (kRB * wv + rb) + l16;
    const int posl = R / G;
    const int head = g * G + R % G;
    lim[rb] = p.non_causal ? L - 1 : cofs + p0 + posl;  // last key this row may see
    const bool ok = posl < npos;
#pragma unroll
    for (int ks = 0; ks < NS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ok) v = load16(p.q + (int64_t)(q0 + p0 + posl) * p.q_stride_tok + (int64_t)head * p.q_stride_head + 32 * ks + 8 * kb);
      qop[rb][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // MASK: lane (l16, kb) needs, for each row block rb, the mask bytes of its
  // row (query p0 + (16 (kRB wv + rb) + l16) / G of the request) at keys
  // t0 + 16 tb + 4 kb .. +3:
  // one dword per (rb, tb), loaded one tile ahead through a buffer resource
  // over the request's mask block, whose range check returns 0 (hidden) for
  // anything past it.  A 2-D mask has row stride 0.
  [[maybe_unused]] uint32_t mcur[kRB][4], mnext[kRB][4];
  [[maybe_unused]] uint32_t mrow[kRB];
  [[maybe_unused]] __amdgpu_buffer_rsrc_t mrs;
  auto load_mask = [&](int t0, uint32_t (&dst)[kRB][4]) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        dst[rb][tb] = __builtin_amdgcn_raw_buffer_load_b32(mrs, mrow[rb] + (uint32_t)(t0 + 16 * tb + 4 * kb), 0, 0);
  };
  if constexpr (MASK) {
    mrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.mask + (int64_t)b * p.mask_stride_req), (short)0,
                                            (int)p.mask_stride_req, 0x00020000);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) mrow[rb] = (uint32_t)((p0 + (16 * (kRB * wv + rb) + l16) / G) * p.mask_stride_row);
    load_mask(it_lo * KT, mcur);
  }
  const float qk_scale = p.sm_scale * kLog2e;
  const int lim_min = p.non_causal ? L - 1 : cofs + p0;   // smallest row limit of the work group
  f32x4 acc[kRB][NB];
  f32x4 lacc[kRB];     // row sums of the weights (all four entries of a lane equal)
  float mref[kRB];
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    mref[rb] = -INFINITY;
    lacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < NB; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  stage_ready();

  // Tiles wholly below the first row's causal limit run without mask code,
  // the remaining (diagonal) tiles with it.
  [[maybe_unused]] unsigned long long ph[kStampPhases] = {0, 0, 0, 0, 0, 0};
  auto stamp = [&]() __attribute__((always_inline)) -> unsigned long long {
    if constexpr (kStamps) {
      __builtin_amdgcn_sched_barrier(0);
      const unsigned long long t = __builtin_amdgcn_s_memtime();
      __builtin_amdgcn_sched_barrier(0);
      return t;
    } else {
      return 0;
    }
  };
  auto tile = [&](auto masked, auto stage, int it) __attribute__((always_inline)) {
    {
      [[maybe_unused]] const unsigned long long T0 = stamp();
      const int t0 = it * KT;
      const bool more = it + 1 < it_hi;   // uniform
      if (more) {
        if constexpr (decltype(stage)::value == 0) gather(sK1, sV1, t0 + KT); else gather(sK0, sV0, t0 + KT);
        load_ids(t0 + 2 * KT);
        if constexpr (MASK) load_mask(t0 + KT, mnext);
      }
      [[maybe_unused]] const unsigned long long T1 = stamp();
      const uint16_t* kt = decltype(stage)::value == 0 ? sK0 : sK1;
      const uint16_t* vt = decltype(stage)::value == 0 ? sV0 : sV1;
      const int swk = swz(l16);                               // K operand rows 16 tb + l16
      const int swv = swz(4 * kb + (l16 >> 2));               // V^T rows 32 k2 (+16) + 4 kb + l16 / 4

      // S^T blocks: st[rb][tb][q] = S^T[t0 + 16 tb + 4 kb + q][row 16 rb + l16].
      // The K operands of key block tb + 1 are read from LDS while block tb's
      // MFMAs run; the scheduling fences keep the compiler from pulling the
      // reads back next to their first use, where each pair would wait out a
      // full LDS latency.
      f32x4 st[kRB][4];
      // At head_dim 256 one block's K operands are 32 registers and the
      // wavefront's other state fills the register file, so the next block's
      // are not read ahead there (reading them ahead spilled to scratch).
      constexpr int KBUF = D == 256 ? 1 : 2;
      bf16x8 ka[KBUF][NS];
  #pragma unroll
      for (int ks = 0; ks < NS; ++ks) ka[0][ks] = *reinterpret_cast<const bf16x8*>(&kt[l16 * D + 8 * ((4 * ks + kb) ^ swk)]);
  #pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        if (KBUF == 1 && tb > 0) {
  #pragma unroll
          for (int ks = 0; ks < NS; ++ks)
            ka[0][ks] = *reinterpret_cast<const bf16x8*>(&kt[(16 * tb + l16) * D + 8 * ((4 * ks + kb) ^ swk)]);
        }
        if (KBUF == 2 && tb < 3) {
  #pragma unroll
          for (int ks = 0; ks < NS; ++ks)
            ka[(tb + 1) % KBUF][ks] = *reinterpret_cast<const bf16x8*>(&kt[(16 * (tb + 1) + l16) * D + 8 * ((4 * ks + kb) ^ swk)]);
        }
        if constexpr (KBUF == 2) __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int rb = 0; rb < kRB; ++rb) st[rb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int ks = 0; ks < NS; ++ks)
  #pragma unroll
          for (int rb = 0; rb < kRB; ++rb) st[rb][tb] = mfma32k(ka[tb % KBUF][ks], qop[rb][ks], st[rb][tb]);
      }

      // Causal mask (only tiles that reach past the first row's limit need
      // it), and the boolean mask (every tile of a MASK work group).
      if constexpr (decltype(masked)::value) {
  #pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          const int thr = lim[rb] - t0 - 4 * kb;   // key 16 tb + q of this lane is visible iff <= thr
  #pragma unroll
          for (int tb = 0; tb < 4; ++tb)
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              bool hide = 16 * tb + q > thr;
              if constexpr (MASK) hide = hide || ((mcur[rb][tb] >> (8 * q)) & 0xffu) == 0u;
              if (hide) st[rb][tb][q] = -INFINITY;
            }
        }
      }
      bf16x8 pop[kRB][2];
  #pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        // Exponents against the current reference: x = s - mref (base 2).  The
        // common case needs only this lane's maximum: if no x exceeds kTau the
        // reference stands and no cross-lane step is taken.  A NaN maximum
        // (mref == -inf before the row's first visible key) also raises.
        float x[16];
        const float moff = -mref[rb];
  #pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = fmaf(st[rb][i / 4][i % 4], qk_scale, moff);
        float lmax = x[0];
  #pragma unroll
        for (int i = 1; i < 15; i += 2) lmax = fmaxf(lmax, fmaxf(x[i], x[i + 1]));
        lmax = fmaxf(lmax, x[15]);
        const bool raise = !(lmax <= kTau);
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {   // uniform over the wavefront
          // Raise the reference of every row of the block to its running max.
          float tmax = st[rb][0][0];
  #pragma unroll
          for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, st[rb][i / 4][i % 4]);
          tmax = xor_max<16, kWave>(tmax) * qk_scale;
          const float mnew = fmaxf(mref[rb], tmax);
          // mref == -inf before the row's first visible key: alpha is 0 (or,
          // MASK, 1 while the row still has none: exp2(-inf - -inf) would be
          // NaN, and NaN * 0 is not 0).
          float alpha = exp2f(mref[rb] - mnew);
          if constexpr (MASK) alpha = mnew == -INFINITY ? 1.f : alpha;
          mref[rb] = mnew;
          lacc[rb] *= alpha;
  #pragma unroll
          for (int db = 0; db < NB; ++db) acc[rb][db] *= alpha;
          const float moff2 = mnew == -INFINITY ? 0.f : -mnew;   // no visible key yet: every weight 0
  #pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = fmaf(st[rb][i / 4][i % 4], qk_scale, moff2);
        }
  #pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          bf16x8 v;
  #pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (__bf16)__builtin_amdgcn_exp2f(x[8 * k2 + e]);
          pop[rb][k2] = v;
          // Row sums of the rounded weights on the matrix core: every row of the
          // all-ones A operand yields the column sums of P^T.
          lacc[rb] = mfma32k(ones, v, lacc[rb]);
        }
      }

      // O^T += V^T P^T: A = V^T[16 db + l16][keys], keys in the same order as
      // P^T's k slots; the operands of d block db + 1 are read while block
      // db's MFMAs run (same fencing as for K).
      auto vread = [&](int db, bf16x8 (&dst)[2]) {
  #pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int vcol = 8 * ((2 * db + ((l16 & 3) >> 1)) ^ swv) + 4 * (l16 & 1);
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vt + (32 * k2 + 4 * kb + (l16 >> 2)) * D + vcol));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vt + (32 * k2 + 16 + 4 * kb + (l16 >> 2)) * D + vcol));
          const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          dst[k2] = __builtin_bit_cast(bf16x8, both);
        }
      };
      [[maybe_unused]] const unsigned long long T2 = stamp();
      bf16x8 va[2][2];
      vread(0, va[0]);
  #pragma unroll
      for (int db = 0; db < NB; ++db) {
        if (db + 1 < NB) vread(db + 1, va[(db + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
  #pragma unroll
          for (int rb = 0; rb < kRB; ++rb) acc[rb][db] = mfma32k(va[db & 1][k2], pop[rb][k2], acc[rb][db]);
      }

      if constexpr (kStamps) {
        const unsigned long long T3 = stamp();
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const unsigned long long T4 = stamp();
        stage_ready();
        const unsigned long long T5 = stamp();
        ph[0] += T1 - T0;
        ph[1] += T2 - T1;
        ph[2] += T3 - T2;
        ph[3] += T4 - T3;
        ph[4] += T5 - T4;
        ph[5] += 1;
      } else {
        stage_ready();   // the next stage is loaded; this one may be overwritten
      }
      if constexpr (MASK) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) mcur[rb][tb] = mnext[rb][tb];
      }
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // Tile it lives in stage (it - it_lo) % 2.
  auto run_tiles = [&](auto masked, int it_begin, int it_end) {
    int it = it_begin;
    if (it < it_end && ((it - it_lo) & 1)) tile(masked, S1{}, it++);
    for (; it + 1 < it_end; it += 2) {
      tile(masked, S0{}, it);
      tile(masked, S1{}, it + 1);
    }
    if (it < it_end) tile(masked, S0{}, it);
  };
  const int it_plain = MASK ? it_lo : max(it_lo, min(it_hi, (lim_min + 1) / KT));
  run_tiles(std::false_type{}, it_lo, it_plain);
  run_tiles(std::true_type{}, it_plain, it_hi);

#if ASTR_PHASE_STAMPS
  if (lane == 0 && blockIdx.x < kStampWgs) {
    for (int i = 0; i < kStampPhases; ++i) g_prefill_stamps[blockIdx.x][wv][i] = ph[i];
  }
#endif
  // acc[rb][db][q] = O^T[d = 16 db + 4 kb + q][row 16 rb + l16], relative to mref.
  float ltot[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) ltot[rb] = lacc[rb][0];
  if (WORK && it.ns > 1) {
    // Split tile: leave this chunk's state in its slot (lane-major, so every
    // access is one contiguous 1 KB per instruction) with agent-coherent
    // (sc1, write-through) stores, wait until every one has completed, then
    // count the chunk on the tile's counter.  (An agent-scope release fence
    // would also write back the whole L2 of the XCD, which measured 2x slower
    // for the kernel; the stores that must be seen are all coherent already.)
    const uint32_t slot_off = (uint32_t)it.slot * (uint32_t)prefill_partial_bytes(D);
    const uint32_t ml_off = (uint32_t)(kRows / 16) * NB * kWave * 16u;   // after the (wavefront, row block) accumulators
    __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(p.part, (short)0, (int)p.part_bytes, 0x00020000);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
      for (int db = 0; db < NB; ++db)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[rb][db]), prs,
                                               slot_off + 16u * (((wv * kRB + rb) * NB + db) * kWave + lane), 0,
                                               kScopeAgent);
      const float2 ml = make_float2(mref[rb], ltot[rb]);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ml), prs,
                                            slot_off + ml_off + 8u * ((wv * kRB + rb) * kWave + lane), 0, kScopeAgent);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wavefront's slot stores have completed
    // The arrival count is broadcast through the first word of a K stage,
    // free since the last tile's barrier (a separate __shared__ word would
    // take the work group past 64 KB of LDS, and two of them would then no
    // longer fit on one CU: measured one work group per CU).
    int* s_arrival = reinterpret_cast<int*>(sK0);
    __syncthreads();
    if (tid == 0) *s_arrival = __hip_atomic_fetch_add(p.cnt + it.tile_slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*s_arrival != it.ns - 1) return;   // uniform: another chunk of the tile arrives later and merges
    // The last chunk: every chunk's slot is complete (its own too).  Read
    // them with agent-scope (sc1) loads and fold them in chunk order by the
    // log-sum-exp rule, so the result does not depend on which chunk arrived
    // last; then reset the counter for the next call.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      mref[rb] = -INFINITY;
      ltot[rb] = 0.f;
#pragma unroll
      for (int db = 0; db < NB; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int s2 = 0; s2 < it.ns; ++s2) {
      const uint32_t o2 = (uint32_t)(it.tile_slot + s2 * p.work.slices) * (uint32_t)prefill_partial_bytes(D);
      float2 ml2[kRB];
      f32x4 a2[kRB][NB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        ml2[rb] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(
                                                 prs, o2 + ml_off + 8u * ((wv * kRB + rb) * kWave + lane), 0, kScopeAgent));
#pragma unroll
        for (int db = 0; db < NB; ++db)
          a2[rb][db] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     prs, o2 + 16u * (((wv * kRB + rb) * NB + db) * kWave + lane), 0, kScopeAgent));
      }
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        // A chunk with no visible key for the row has max -inf and sum 0.
        const float mnew = fmaxf(mref[rb], ml2[rb].x);
        const float c1 = mref[rb] == -INFINITY ? 0.f : exp2f(mref[rb] - mnew);
        const float c2 = ml2[rb].x == -INFINITY ? 0.f : exp2f(ml2[rb].x - mnew);
        ltot[rb] = ltot[rb] * c1 + ml2[rb].y * c2;
#pragma unroll
        for (int db = 0; db < NB; ++db) acc[rb][db] = acc[rb][db] * c1 + a2[rb][db] * c2;
        mref[rb] = mnew;
      }
    }
    if (tid == 0) __hip_atomic_store(p.cnt + it.tile_slot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int R = 16 * (kRB * wv + rb) + l16;
    const int posl = R / G;
    if (posl >= npos) continue;
    const int row = q0 + p0 + posl;
    const int head = g * G + R % G;
    // A row with no visible key (only possible with a mask) is written as
    // zeros with lse = -inf.
    const float inv = ltot[rb] > 0.f ? 1.f / ltot[rb] : 0.f;
    uint16_t* orow = p.o + (int64_t)row * p.o_stride_tok + (int64_t)head * p.o_stride_head;
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      const uint32_t w0 = (uint32_t)f32_to_bf16_rne(acc[rb][db][0] * inv) | ((uint32_t)f32_to_bf16_rne(acc[rb][db][1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16_rne(acc[rb][db][2] * inv) | ((uint32_t)f32_to_bf16_rne(acc[rb][db][3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * db + 4 * kb) = make_uint2(w0, w1);
    }
    if (p.lse != nullptr && kb == 0)
      p.lse[(int64_t)row * p.lse_stride_tok + head] = ltot[rb] > 0.f ? (mref[rb] + log2f(ltot[rb])) * kLn2 : -INFINITY;
  }
}

template <int D, int G, bool WORK>
hipError_t launch_w(const PrefillLaunch& p, dim3 grid, hipStream_t s, const Timing& t) {
  if (p.mask != nullptr) {
    if (p.off32) return launch_kernel(prefill_kernel<D, G, true, true, WORK>, grid, dim3(prefill_threads<D>()), s, t, p);
    return launch_kernel(prefill_kernel<D, G, false, true, WORK>, grid, dim3(prefill_threads<D>()), s, t, p);
  }
  if (p.off32) return launch_kernel(prefill_kernel<D, G, true, false, WORK>, grid, dim3(prefill_threads<D>()), s, t, p);
  return launch_kernel(prefill_kernel<D, G, false, false, WORK>, grid, dim3(prefill_threads<D>()), s, t, p);
}

template <int D, int G>
hipError_t launch_t(const PrefillLaunch& p, hipStream_t s, const Timing& t) {
  if (p.work.num_reqs > 0) {
    // One work group per item of the work list.
    const int64_t blocks = (int64_t)p.work.slices * p.work.req[p.work.num_reqs].first;
    if (blocks < 1 || blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    return launch_w<D, G, true>(p, dim3((unsigned)blocks, 1, 1), s, t);
  }
  constexpr int BQ = kRows / G;
  const int64_t nq = (p.max_q_len + BQ - 1) / BQ;
  const int64_t groups = (int64_t)p.num_kv_heads * p.batch;
  const int64_t blocks = kXcds * ((groups + kXcds - 1) / kXcds) * nq;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  return launch_w<D, G, false>(p, dim3((unsigned)blocks, 1, 1), s, t);
}

}  // namespace

bool prefill_supported(int head_dim, int group) {
  return (head_dim == 32 || head_dim == 64 || head_dim == 128 || head_dim == 256) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t s, const Timing& t) {
  switch (p.head_dim * 100 + p.group) {
    case 3201: return launch_t<32, 1>(p, s, t);
    case 3202: return launch_t<32, 2>(p, s, t);
    case 3204: return launch_t<32, 4>(p, s, t);
    case 3208: return launch_t<32, 8>(p, s, t);
    case 6401: return launch_t<64, 1>(p, s, t);
    case 6402: return launch_t<64, 2>(p, s, t);
    case 6404: return launch_t<64, 4>(p, s, t);
    case 6408: return launch_t<64, 8>(p, s, t);
    case 12801: return launch_t<128, 1>(p, s, t);
    case 12802: return launch_t<128, 2>(p, s, t);
    case 12804: return launch_t<128, 4>(p, s, t);
    case 12808: return launch_t<128, 8>(p, s, t);
    case 25601: return launch_t<256, 1>(p, s, t);
    case 25602: return launch_t<256, 2>(p, s, t);
    case 25604: return launch_t<256, 4>(p, s, t);
    case 25608: return launch_t<256, 8>(p, s, t);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace astr

#if ASTR_PHASE_STAMPS
// Phase-stamp builds only: copy out or clear the per-wavefront phase cycles
// ([kStampWgs][8][6] unsigned 64-bit: gather issue, S + softmax, P.V, gather
// wait, barrier, tiles).
extern "C" int astr_debug_prefill_stamps(void* host, size_t bytes) {
  if (bytes < sizeof(astr::g_prefill_stamps)) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(astr::g_prefill_stamps), sizeof(astr::g_prefill_stamps));
}
extern "C" int astr_debug_prefill_stamps_clear(void) {
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(astr::g_prefill_stamps));
  if (e != hipSuccess) return (int)e;
  return (int)hipMemset(ptr, 0, sizeof(astr::g_prefill_stamps));
}
#endif
