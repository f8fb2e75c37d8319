// Paged GQA decode for gfx950: split-KV kernel and log-sum-exp combine kernel.
//
// Method (AstrAI commit-list pages): [extension @6f67ba8], the commits that
// (a) read K/V through req_to_token as a page table with page size one,
// (b) turn decode into split-KV with o_part / ml_part partials merged by a
// separate combine kernel, (c) load both K and V of a tile up front instead of
// looking up KV addresses per element in the softmax loop, (d) keep several
// tile loads in flight while the current tile is computed, and (e) drop the
// partial memset because each split writes every slot it owns.
//
// Work partition (this library's split planner): the keys of one kv head are
// laid end to end in request order (N = kv_indptr[B] keys) and cut into
// W = min(Wh, N) near-equal contiguous ranges, one per work group
// (blockIdx.x = w, blockIdx.y = kv head g).  Where a range crosses request
// boundaries it is processed as one piece per request; piece (w, b) writes
// partial slot w + b.  Ranges are computed on the device from kv_indptr, so a
// fixed grid stays valid when sequence lengths change.
//
// Inside a work group, the tiles of the pieces (16 keys each, in pairs) are
// laid end to end and cut into 4 contiguous blocks of near-equal length, one
// per wavefront, so every wavefront loads about the same number of tiles
// whatever the piece lengths.
// Per tile and wavefront both products run on the matrix cores:
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A is the K tile as loaded
//    (lane l holds 8 bf16 of key l % 16; four lanes cover 64 contiguous bytes
//    of a row per load), B holds the group's q rows (column j is query head
//    j % G), so every column of S^T is one head of the GQA group and each
//    K/V row is read from HBM once for all G heads.  Lane l receives the
//    logits of keys 4*(l/16)..+3 for head l % 16.
//  * O^T += V^T P^T with v_mfma_f32_16x16x16_bf16: the weights, split into a
//    bf16 high part and a bf16 remainder (two MFMAs, near-fp32 weights), are
//    already in the B-operand layout; V^T comes from a wavefront-private LDS
//    copy of the V tile through the transposing LDS read ds_read_b64_tr_b16
//    (lane j of each 16-lane group addresses row 4*(l/16) + j/4, columns
//    4*(j%4).. of a 16-column block and receives column j of rows
//    4*(l/16)..+3).
//  * K and V rows of a key share one slot id; the next tile's loads and the
//    ids one tile further are issued before the current tile is computed.
//  * Softmax runs in base 2 against a lazily raised reference max: the
//    accumulators are rescaled only when a logit exceeds the reference by more
//    than kTau (so weights stay <= 2^kTau); the exact running max is tracked
//    alongside and the written (m, l) pair uses it.  Keys past the piece end
//    weigh exactly zero; their loads re-read a valid key of the same request.
// A piece inside one block is finished by its wavefront, which writes the
// normalised partial (o, m, l) per query head; a piece crossing block
// boundaries is merged through LDS once every wavefront is done.
//
// Fused KV append (APPEND; [attention_backend.py @47b3ed4], the commit sharing
// one write-then-gather K/V helper): the new token of request b is its last
// key L_b - 1, and the work group whose range holds that key (for its kv head)
// is the only one that reads it.  Before its first tile load, that work group
// copies the token's K/V row from k_new / v_new into the pools; a work-group
// barrier orders those stores before its own tile loads, which then read the
// new rows like any other key.  The tile loop is the plain decode's; the
// arithmetic sees the values a separate append followed by a decode would
// read, so both give the same bits.
#include "device_common.hpp"
#include "kernel_launch.hpp"

namespace astr {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

// Optional timeline stamps (built only with ASTR_PHASE_STAMPS=1, into a
// separate library; the library as shipped has none of this code): thread 0
// of each of the first kStampWgs split work groups records the constant
// 100 MHz clock (s_memrealtime) at its start, once kv_indptr is staged, when
// its first tile's loads are issued and at its end, its hardware CU and XCD
// ids and its piece count.
#ifndef ASTR_PHASE_STAMPS
#define ASTR_PHASE_STAMPS 0
#endif
constexpr bool kStamps = ASTR_PHASE_STAMPS != 0;
constexpr int kStampWgs = 4096;
#if ASTR_PHASE_STAMPS
__device__ unsigned long long g_decode_stamps[kStampWgs][8];
#endif

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTile = 16;       // keys per wavefront per tile (one MFMA column block)
constexpr int kQBatchRows = 32;  // q rows (pieces x group heads) staged in LDS at a time
constexpr float kTau = 8.0f;    // log2 headroom before the accumulators are rescaled

__device__ __forceinline__ uint4 load16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Number of request ends kv_indptr[1..B] that are <= x, i.e. the request
// holding flat position x.  Uses the whole work group.
__device__ __forceinline__ int request_of(const int32_t* kv_indptr, int B, int64_t x) {
  int count = 0;
  for (int base = 1; base <= B; base += kThreads) {
    const int idx = base + (int)threadIdx.x;
    const int pred = (idx <= B) && ((int64_t)kv_indptr[idx] <= x);
    count += __syncthreads_count(pred);
  }
  return count;
}

template <int D>
struct Shape {
  static constexpr int kSteps = D / 32;    // 16-byte K (and V) loads per lane per tile; QK^T k-steps
  static constexpr int kDBlocks = D / 16;  // 16-wide d blocks of O^T (PV MFMAs per tile)
  static constexpr int kVRow = D + 16;     // LDS row stride of the V tile (elements), padded
};

// K and V of one 16-key tile in the MFMA A-operand layout: lane l holds the
// 16-byte chunks 8*(l/16) + 32*s of key l % 16.
template <int D>
struct Tile {
  uint4 k[Shape<D>::kSteps];
  uint4 v[Shape<D>::kSteps];
  uint64_t vis;   // MASK: bit j set when key j of the tile is not hidden by the mask (wavefront-uniform)
};

// Pool rows are addressed from a per-kv-head base (wavefront-uniform, so it
// lives in scalar registers) plus a per-lane byte offset.
//
// When every row of the head's range lies within kPoolRange32 bytes of the
// base (OFF32), the loads are raw buffer loads over a resource covering
// exactly that range, with 32-bit offsets.  A key past the end of its piece
// (the tail of the last tile, pad tiles, tiles beyond the work group's last
// piece) gets the offset kOob, which the range check turns into zeros with no
// memory access.  Every load is still issued unconditionally: a branch around
// a load would keep the compiler from counting outstanding loads, and it would
// then wait for the prefetched tile before computing the current one.
//
// Larger pools take 64-bit global addresses; there keys past the piece end
// re-read the piece's last key (the data is never used).
constexpr uint32_t kOob = 0xFFFFF000u;
constexpr int64_t kPoolRange32 = kOob;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct PoolView {
  __amdgpu_buffer_rsrc_t k_rsrc, v_rsrc;   // OFF32: buffer resources over the head's rows
  const char* kbase;                        // otherwise: global base pointers of the head
  const char* vbase;
  int64_t row_bytes;
};

template <int D, bool OFF32>
__device__ __forceinline__ void load_tile(Tile<D>& t, const PoolView& pv, int id, int lane) {
  const int kb = lane >> 4;
  if constexpr (OFF32) {
    const uint32_t base = id >= 0 ? (uint32_t)id * (uint32_t)pv.row_bytes + 16u * kb : kOob;
#pragma unroll
    for (int s = 0; s < Shape<D>::kSteps; ++s) {
      t.k[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pv.k_rsrc, base + 64 * s, 0, 0));
      t.v[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pv.v_rsrc, base + 64 * s, 0, 0));
    }
  } else {
    const int64_t base = (int64_t)id * pv.row_bytes + 16 * kb;
#pragma unroll
    for (int s = 0; s < Shape<D>::kSteps; ++s) {
      t.k[s] = *reinterpret_cast<const uint4*>(pv.kbase + base + 64 * s);
      t.v[s] = *reinterpret_cast<const uint4*>(pv.vbase + base + 64 * s);
    }
  }
}

// The pieces of a work group (requests its key range touches).  kv_indptr is
// staged in LDS in windows of kKvStage entries (normally the whole array, in
// one round trip); pieces are processed in windows of at most one q batch
// (kQBatchRows / G pieces) inside it.  Piece j of a window is request b0 + j;
// its keys inside the range are positions [t_begin(j), t_end(j)) of that
// request.
constexpr int kKvStage = 1024;

struct PieceTable {
  const int32_t* kv;   // LDS copy of kv_indptr[b0 .. b0 + n]
  int e0, e1;          // the work group's flat key range (kv_indptr values are int32)
  int b0, n;
  __device__ __forceinline__ int t_begin(int j) const { return max(e0, kv[j]) - kv[j]; }
  __device__ __forceinline__ int t_end(int j) const { return min(e1, kv[j + 1]) - kv[j]; }
};

// Work inside a window of pieces.  Piece j is cut into 32-key pairs of
// tiles, P_j = ceil(len_j / 32) of them (the last pair may hold masked keys
// and a fully masked pad tile), and the window's pairs, laid end to end in
// piece order, are cut into kWaves contiguous blocks of near-equal length:
// wavefront wv takes pairs [q0, q1) = [Ptot wv / kWaves, Ptot (wv + 1) /
// kWaves).  Every wavefront therefore loads about the same number of tiles,
// whatever the piece lengths.  A piece inside one block is finished by its
// wavefront, which writes the partial; a piece crossing a block boundary is
// merged through LDS at the end of the window.
//
// Per-wavefront piece table in LDS, entry j = {first pair of piece j,
// t_begin, t_end, kv_indptr[b0 + j]}; entry n holds the pair total.
struct PieceEntry {
  int pf, tb, te, kv;
};

// A wavefront's position in its sequence of tiles: piece j, first key t of
// the tile, end of the wavefront's keys in the piece (stop, a multiple of 32
// past the segment start), the piece's key end te and the table row of its
// request.  j == n marks the end of the sequence; te and row then keep the
// values of a valid piece, so the addresses made from them stay valid.
struct Cursor {
  int j, t, stop, te;
  int jr;     // piece whose request addresses the keys (j, or the last one past the end)
  int ridx;   // its req_to_token row: request index (2-D table) or kv_indptr entry (flat table)
};

// Waves per SIMD the split kernel is built for: three 4-wavefront work groups
// per CU up to head_dim 128; at head_dim 256 the two K/V tiles, the
// accumulators and the q operands need the whole register file of one wave
// (accumulators in AGPRs), so one work group per CU.
template <int D>
constexpr int split_waves_per_simd() { return D == 256 ? 1 : 3; }

template <int D, int G, bool OFF32, bool APPEND, bool MASK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(split_waves_per_simd<D>()))) void decode_split_kernel(const DecodeLaunch p) {
  using S = Shape<D>;
  constexpr int NS = S::kSteps;
  constexpr int NB = S::kDBlocks;
  constexpr int QSTR = D + 8;   // padded q row (spreads LDS banks)
  __shared__ __align__(16) float sm_acc[kWaves][G][D];   // slot A of each wavefront (shared first piece)
  __shared__ float4 sm_ml[2][kWaves][G];         // (mref, max, l) of slots A and B
  __shared__ int4 sm_lead[kWaves];               // merge led by each wavefront: (piece or -1, slot A?, last wavefront)
  __shared__ PieceEntry sm_tab[kWaves][kQBatchRows + 1];
  constexpr int QB = kQBatchRows / G;   // pieces whose q rows are staged at a time
  __shared__ __align__(16) uint16_t sm_q[QB][G][QSTR];           // q rows of the staged pieces
  __shared__ __align__(16) uint16_t sm_v[kWaves][kTile][S::kVRow];  // per-wavefront V tile
  static_assert(G * D * sizeof(float) <= sizeof(sm_v[0]), "slot B (G x D floats) must fit a wavefront's V tile area");
  __shared__ int32_t sm_kv[kKvStage];                              // window of kv_indptr starting at kv_base

  [[maybe_unused]] const unsigned long long stamp_start = kStamps ? __builtin_amdgcn_s_memrealtime() : 0;
  const int w = blockIdx.x;
  const int g = blockIdx.y;
  const int B = p.batch;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);   // wavefront-uniform
  const int l16 = lane & 15;
  const int kb = lane >> 4;
  const int hcol = l16 % G;     // query head of this lane's S^T / O^T column
  const float qscale = p.sm_scale * kLog2e;
  PoolView pv;
  pv.kbase = reinterpret_cast<const char*>(p.k_pool + (int64_t)g * p.kv_stride_head);
  pv.vbase = reinterpret_cast<const char*>(p.v_pool + (int64_t)g * p.kv_stride_head);
  pv.row_bytes = p.kv_stride_slot * 2;
  if constexpr (OFF32) {
    pv.k_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(pv.kbase), (short)0, (int)p.pool_range, 0x00020000);
    pv.v_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(pv.vbase), (short)0, (int)p.pool_range, 0x00020000);
  }

  // kv_indptr[0 .. min(B, kKvStage - 1)] -> LDS in one round trip.
  int kv_base = 0;
  const int staged = min(B, kKvStage - 1);
  for (int t = tid; t <= staged; t += kThreads) sm_kv[t] = p.kv_indptr[t];
  const int64_t N_glob = B > staged ? (int64_t)p.kv_indptr[B] : 0;
  __syncthreads();
  // Values read from LDS are the same in every lane; readfirstlane lets the
  // compiler keep them (and what depends on them) in scalar registers.
  const int64_t N = B > staged ? N_glob : (int64_t)__builtin_amdgcn_readfirstlane(sm_kv[B]);
  const int64_t W = min((int64_t)p.num_splits, N);
  if (w >= W) return;  // uniform over the work group

  [[maybe_unused]] const unsigned long long stamp_staged = kStamps ? __builtin_amdgcn_s_memrealtime() : 0;
  [[maybe_unused]] unsigned long long stamp_first = 0;
  PieceTable pt;
  pt.e0 = (int)(((int64_t)w * N) / W);
  pt.e1 = (int)(((int64_t)(w + 1) * N) / W);
  int bnext;
  if (B <= staged) {
    // Largest b < B with kv_indptr[b] <= e0 (binary search in LDS).
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)sm_kv[mid] <= pt.e0) lo = mid; else hi = mid - 1;
    }
    bnext = __builtin_amdgcn_readfirstlane(lo);
  } else {
    bnext = request_of(p.kv_indptr, B, pt.e0);
  }
  [[maybe_unused]] const int stamp_b0 = bnext;

  // APPEND: requests bnext .. bnext + n_last - 1 have their last key in this
  // range (those with kv_indptr[b + 1] <= e1; the request holding e0 ends
  // after e0).  Task t copies 16 bytes of the K (wk = 0) or V (wk = 1) row of
  // kv head g of request bnext + t / (D / 4).  Every task is copied here,
  // before the window's set-up (holding the loaded rows across it would
  // spill them); a barrier before the first tile load orders the stores
  // before the loads that read them.
  [[maybe_unused]] int n_last = 0;
  auto kvp = [&](int b) -> int64_t { return b <= staged ? (int64_t)sm_kv[b] : (int64_t)p.kv_indptr[b]; };
  auto append_load = [&](int t, int32_t& slot, uint4& val) {
    const int b = bnext + t / (2 * (D / 8));
    const int64_t kb0 = kvp(b);
    const int64_t L = kvp(b + 1) - kb0;
    const int32_t* row = p.req_to_token + (p.req_to_token_stride > 0 ? (int64_t)b * p.req_to_token_stride : kb0);
    slot = (row[(L - 1) >> p.page_shift] << p.page_shift) + (int)((L - 1) & ((1 << p.page_shift) - 1));
    val = load16((((t / (D / 8)) & 1) ? p.v_new : p.k_new) + (int64_t)b * p.new_stride_tok +
                 (int64_t)g * p.new_stride_head + 8 * (t % (D / 8)));
  };
  auto append_store = [&](int t, int32_t slot, const uint4& val) {
    if (slot < 0 || (int64_t)slot >= p.num_slots) return;   // outside the pool: nothing is written
    *reinterpret_cast<uint4*>(const_cast<uint16_t*>(((t / (D / 8)) & 1) ? p.v_pool : p.k_pool) +
                              (int64_t)slot * p.kv_stride_slot + (int64_t)g * p.kv_stride_head + 8 * (t % (D / 8))) = val;
  };
  if constexpr (APPEND) {
    // The requests ending in the range form a prefix of bnext, bnext + 1, ...:
    // each lane tests one, a ballot counts them (64 per step; every
    // wavefront finds the same count).
    for (int base = bnext;; base += kWave) {
      const int b = base + lane;
      const uint64_t m = __builtin_amdgcn_ballot_w64(b < B && kvp(b + 1) <= pt.e1);
      n_last += __builtin_popcountll(m);
      if (m != ~0ull) break;
    }
    for (int t = tid; t < n_last * 2 * (D / 8); t += kThreads) {
      int32_t slot;
      uint4 val;
      append_load(t, slot, val);
      append_store(t, slot, val);
    }
  }
  bool first_window = true;

  for (;;) {
    // Keep the window holding kv_indptr[bnext] and at least one entry after it.
    if (bnext - kv_base + 1 >= kKvStage) {
      __syncthreads();
      kv_base = bnext;
      for (int t = tid; t < kKvStage; t += kThreads) sm_kv[t] = p.kv_indptr[min(kv_base + t, B)];
      __syncthreads();
    }
    if (bnext >= B || __builtin_amdgcn_readfirstlane(sm_kv[bnext - kv_base]) >= pt.e1) break;
    pt.b0 = bnext;
    pt.kv = sm_kv + (bnext - kv_base);
    const int room = min(kKvStage - 1 - (bnext - kv_base), QB);
    int n = 0;
    while (n < room && pt.b0 + n < B && __builtin_amdgcn_readfirstlane(pt.kv[n]) < pt.e1) ++n;
    pt.n = n;
    bnext = pt.b0 + n;

    // Piece table of the window (lane j < n computes entry j; an inclusive
    // scan over the lanes gives the pair offsets; lane n holds the total).
    PieceEntry* tab = sm_tab[wv];
    int incl;
    {
      const int jc = min(lane, n - 1);
      const int tb = pt.t_begin(jc), te = pt.t_end(jc);
      const int pairs = lane < n ? (te - tb + 2 * kTile - 1) / (2 * kTile) : 0;
      // Inclusive scan over the lanes.  The lane id passes through an empty
      // asm so that the source-lane addresses are formed here, per window,
      // instead of being hoisted out of the loop as six live registers.
      int x = pairs;
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __builtin_amdgcn_ds_bpermute((ln - o) << 2, x);
        if (ln >= o) x += y;
      }
      incl = x;
      if (lane <= n) tab[lane] = PieceEntry{x - pairs, tb, te, pt.kv[jc]};
    }
    const int Ptot = __builtin_amdgcn_readlane(incl, n);
    const int q0 = Ptot * wv / kWaves;
    const int q1 = Ptot * (wv + 1) / kWaves;
    // First piece of the block: the number of pieces that end at or before pair q0.
    const int jfirst = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < n && incl <= q0));
    auto entry = [&](int j) -> PieceEntry {   // wavefront-uniform read of the table
      const PieceEntry e = tab[j];
      return PieceEntry{__builtin_amdgcn_readfirstlane(e.pf), __builtin_amdgcn_readfirstlane(e.tb),
                        __builtin_amdgcn_readfirstlane(e.te), __builtin_amdgcn_readfirstlane(e.kv)};
    };
    auto ridx_of = [&](int j, int kvj) -> int { return p.req_to_token_stride > 0 ? pt.b0 + j : kvj; };
    auto row_of = [&](const Cursor& cu) -> int64_t {
      return p.req_to_token_stride > 0 ? (int64_t)cu.ridx * p.req_to_token_stride : (int64_t)cu.ridx;
    };
    // The cursor cu entering piece j (at the start of this wavefront's pairs
    // in it), or ended if the block holds none of it.
    auto enter = [&](Cursor cu, int j) -> Cursor {
      Cursor r = cu;
      r.j = n;
      r.t = cu.te;
      if (j < n) {
        const PieceEntry e = entry(j);
        const int pf_next = __builtin_amdgcn_readfirstlane(tab[j + 1].pf);
        const int lo = max(q0, e.pf), hi = min(q1, pf_next);
        if (lo < hi) {
          r.j = j;
          r.jr = j;
          r.t = e.tb + 2 * kTile * (lo - e.pf);
          r.stop = e.tb + 2 * kTile * (hi - e.pf);
          r.te = e.te;
          r.ridx = ridx_of(j, e.kv);
        }
      }
      return r;
    };
    // The next tile of the wavefront's sequence after cu.
    auto next = [&](Cursor cu) -> Cursor {
      if (cu.j >= n) return cu;
      cu.t += kTile;
      if (cu.t < cu.stop) return cu;
      return enter(cu, cu.j + 1);
    };

    // Slot id of this lane's key in the tile at cursor cu; -1 (OFF32) or the
    // piece's last key (64-bit path) for a key past the piece end, and for
    // every key of a past-the-end cursor.  The id itself is always read from
    // a valid req_to_token entry.
    // The table entry is loaded here, one tile ahead; slot_at turns it into
    // the slot when the tile is loaded, so nothing waits for the entry early.
    auto id_at = [&](const Cursor& cu) -> int {
      const int t = cu.t + l16;
      return p.req_to_token[row_of(cu) + (min(t, cu.te - 1) >> p.page_shift)];
    };
    // Slot of this lane's key at cursor cu from its table entry e (page size
    // 2^page_shift: entry << page_shift plus the position inside the page).
    auto slot_at = [&](const Cursor& cu, int e) -> int {
      const int t = cu.t + l16;
      const int id = (e << p.page_shift) + (min(t, cu.te - 1) & ((1 << p.page_shift) - 1));
      if constexpr (OFF32) return t < cu.te ? id : -1;
      return id;
    };
    // MASK: the mask byte of this lane's key at cursor cu (read for the
    // clamped key, like the slot id, so it stays inside the request's row).
    auto mask_at = [&](const Cursor& cu) -> int {
      if constexpr (!MASK) return 1;
      const int t = min(cu.t + l16, cu.te - 1);
      return p.mask[(int64_t)(pt.b0 + cu.jr) * p.mask_stride_req + t];
    };
    // q rows of pieces [j0, j0 + nb) -> sm_q[0 .. nb).  The caller brackets
    // this with barriers.
    auto stage_q = [&](int j0, int nb) {
      for (int t = tid; t < nb * G * (D / 8); t += kThreads) {
        const int jj = t / (G * (D / 8));
        const int hh = (t / (D / 8)) % G;
        const int dc = t % (D / 8);
        *reinterpret_cast<uint4*>(&sm_q[jj][hh][8 * dc]) =
            load16(p.q + (int64_t)(pt.b0 + j0 + jj) * p.q_stride_tok + (int64_t)(g * G + hh) * p.q_stride_head + 8 * dc);
      }
    };

    // Ping-pong pipeline over the wavefront's tile sequence c0, c1, c2, ...
    // (which runs across piece boundaries).  While tile k is computed from
    // one register buffer, tile k+1 is in flight into the other; right after,
    // the first buffer is refilled with tile k+2.  Slot ids run one tile
    // further ahead and are always issued before the data loads that must
    // stay in flight while they are used: vmcnt retires loads in issue order,
    // so an id load issued after a data load could only be waited for
    // together with it.  A wavefront's tiles in a piece come in pairs, so
    // buffer A always holds even tiles and B odd ones and no register copy
    // (which would wait for its load) is ever needed.
    // The q rows of the window's pieces are staged before any tile load, so
    // waiting for them waits for nothing else.
    stage_q(0, n);
    if constexpr (APPEND) {
      // The new rows are in the pools before any wavefront loads a tile
      // (a work-group barrier orders the stores before the loads).
      if (first_window && n_last > 0) __syncthreads();   // uniform over the work group
      first_window = false;
    }
    if constexpr (kStamps) {
      if (stamp_first == 0) stamp_first = __builtin_amdgcn_s_memrealtime();
    }
    Cursor c0;
    {
      const PieceEntry e0 = entry(0);
      c0.jr = 0;
      c0.te = e0.te;
      c0.ridx = ridx_of(0, e0.kv);
      c0.j = n;
      c0.t = c0.stop = c0.te;
      if (q0 < q1) c0 = enter(c0, jfirst);
    }
    Cursor c1 = next(c0);
    Cursor c2 = next(c1);
    Cursor c3 = next(c2);
    int iA = id_at(c0);
    int iB = id_at(c1);
    int mA = mask_at(c0);
    int mB = mask_at(c1);
    Tile<D> A, Bt;
    load_tile<D, OFF32>(A, pv, slot_at(c0, iA), lane);
    if constexpr (MASK) A.vis = __builtin_amdgcn_ballot_w64(mA != 0);
    iA = id_at(c2);
    mA = mask_at(c2);
    load_tile<D, OFF32>(Bt, pv, slot_at(c1, iB), lane);
    if constexpr (MASK) Bt.vis = __builtin_amdgcn_ballot_w64(mB != 0);
    // No merge led by this wavefront yet (only .x is read before a merge
    // record overwrites all fields; a one-register constant, so the compiler
    // does not keep a four-register tuple live across the window).
    if (lane == 0) sm_lead[wv].x = -1;
    __syncthreads();

    float mref = -INFINITY, mx = -INFINITY, lsum = 0.f;
    f32x4 acc[NB];
    int t_end = 0;
    bf16x8 qop[NS];
    uint16_t* vt = &sm_v[wv][0][0];

    // Logits, softmax weights and P.V for the tile in buffer X (cursor c0).
    auto compute = [&](const Tile<D>& X) {
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s)
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, X.k[s]), qop[s], st, 0, 0, 0);
      // st[r] = S^T[key 4 kb + r][head hcol]; V tile -> LDS meanwhile.
#pragma unroll
      for (int s = 0; s < NS; ++s) *reinterpret_cast<uint4*>(vt + l16 * S::kVRow + 32 * s + 8 * kb) = X.v[s];
      float sc[4];
      float tmax = -INFINITY;
      bool raise = false;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bool vis = c0.t + 4 * kb + r < t_end;
        if constexpr (MASK) vis = vis && ((X.vis >> (4 * kb + r)) & 1);
        sc[r] = vis ? st[r] * qscale : -INFINITY;
        tmax = fmaxf(tmax, sc[r]);
        raise |= sc[r] > mref + kTau;
      }
      mx = fmaxf(mx, tmax);
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {   // uniform over the wavefront
        const float mnew = fmaxf(mref, xor_max<16, kWave>(tmax));
        const float alpha = exp2f(mref - mnew);
        mref = mnew;
        lsum *= alpha;
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] *= alpha;
      }
      // Weights as a bf16 high part plus a bf16 remainder for two P.V MFMAs
      // (about 16 significant bits); the sum uses the fp32 weights.
      bf16x4 phi, plo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // MASK: a tile can start a piece with every key hidden (mref still
        // -inf); hidden keys weigh exactly 0.
        const float pr = (MASK && sc[r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[r] - mref);
        lsum += pr;
        phi[r] = (__bf16)pr;
        plo[r] = (__bf16)(pr - (float)phi[r]);
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const s16x4 av = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(vt + (4 * kb + (l16 >> 2)) * S::kVRow + 16 * b + 4 * (l16 & 3)));
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4, phi), acc[b], 0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4, plo), acc[b], 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
    };
    // One pipeline step: X holds tile c0, the other buffer holds c1 (in
    // flight), iX holds the id of c2; iY is free and receives the id of c3.
    auto step = [&](Tile<D>& X, int& iX, int& iY, int& mX, int& mY) {
      compute(X);
      iY = id_at(c3);
      mY = mask_at(c3);
      load_tile<D, OFF32>(X, pv, slot_at(c2, iX), lane);
      if constexpr (MASK) X.vis = __builtin_amdgcn_ballot_w64(mX != 0);
      c0 = c1;
      c1 = c2;
      c2 = c3;
      c3 = next(c3);
    };

    // The wavefront's pieces, in order.
    while (c0.j < n) {
      const int j = c0.j;   // uniform
      const PieceEntry e = entry(j);
      const int pf_next = __builtin_amdgcn_readfirstlane(tab[j + 1].pf);
      const bool owned = e.pf >= q0 && pf_next <= q1;   // the whole piece is in this block
#pragma unroll
      for (int s = 0; s < NS; ++s) qop[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sm_q[j][hcol][32 * s + 8 * kb]));
      mref = -INFINITY;
      mx = -INFINITY;
      lsum = 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      t_end = c0.te;
      while (c0.j == j) {
        step(A, iA, iB, mA, mB);
        step(Bt, iB, iA, mB, mA);
      }
      // Wavefront totals over the four key groups of each column.
      const float l_tot = xor_sum<16, kWave>(lsum);
      const float mx_tot = xor_max<16, kWave>(mx);
      // The lane's column and key group, opaque to the compiler, so that the
      // addresses below are formed here instead of being hoisted out of the
      // tile loop (where they would hold registers the pipeline needs).
      int col = l16, kg = kb;
      asm volatile("" : "+v"(col), "+v"(kg));
      if (owned) {
        // The wavefront writes the partial: o = acc / l, and (m, l) against
        // the exact running max.
        if (col < G) {
          const int64_t pidx = (int64_t)(g * G + col) * p.num_partials + w + pt.b0 + j;
          const float inv = 1.f / l_tot;
#pragma unroll
          for (int b = 0; b < NB; ++b)
            *reinterpret_cast<float4*>(&p.o_part[pidx * D + 16 * b + 4 * kg]) =
                make_float4(acc[b][0] * inv, acc[b][1] * inv, acc[b][2] * inv, acc[b][3] * inv);
          if (kg == 0) {
            p.ml_part[pidx * 2 + 0] = mx_tot * kLn2;
            p.ml_part[pidx * 2 + 1] = l_tot * exp2f(mref - mx_tot);
          }
        }
        continue;
      }
      // A piece shared with other wavefronts: its state goes to slot A (the
      // block's first piece: sm_acc) or slot B (its last piece, which starts
      // inside the block: the wavefront's own V tile area, no longer used).
      const bool slot_a = e.pf <= q0;
      float* dst = slot_a ? &sm_acc[wv][0][0] : reinterpret_cast<float*>(vt);
      if (col < G) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[col * D + 16 * b + 4 * kg + r] = acc[b][r];
        if (kg == 0) {
          sm_ml[slot_a ? 0 : 1][wv][col] = float4{mref, mx_tot, l_tot, 0.f};
        }
      }
      if (e.pf >= q0 && lane == 0) {
        // This wavefront holds the first pairs of the piece: it records the
        // merge (piece, its slot, the last wavefront holding pairs of it).
        int wl = kWaves - 1;
        while (Ptot * wl / kWaves > pf_next - 1) --wl;
        sm_lead[wv] = int4{j, slot_a ? 1 : 0, wl, 0};
      }
    }

    // Merge the pieces that cross block boundaries: piece j led by
    // wavefront lw is held by wavefronts lw .. wl, in slot A except the
    // leader's slot B when the piece starts inside its block.
    __syncthreads();
    int tid_m = tid;   // opaque copy: the merge's addresses are formed here
    asm volatile("" : "+v"(tid_m));
    for (int lw = 0; lw < kWaves - 1; ++lw) {
      const int4 rec = sm_lead[lw];
      const int j = __builtin_amdgcn_readfirstlane(rec.x);
      if (j < 0) continue;
      const bool lead_a = __builtin_amdgcn_readfirstlane(rec.y) != 0;
      const int wl = __builtin_amdgcn_readfirstlane(rec.z);
      const int slot = w + pt.b0 + j;
      // Wavefronts with an empty block (fewer pairs than wavefronts) hold nothing.
      bool part[kWaves];
#pragma unroll
      for (int k = 0; k < kWaves; ++k) part[k] = k >= lw && k <= wl && Ptot * k / kWaves != Ptot * (k + 1) / kWaves;
      // Thread task: two consecutive d of one head (G * D / 2 tasks).
      for (int task = tid_m; task < G * D / 2; task += kThreads) {
        const int hh = task / (D / 2);
        const int d = 2 * (task % (D / 2));
        // Every wavefront's state is read at once (one LDS round trip); the
        // ones not holding the piece are then ignored.
        float4 ml[kWaves];
        float2 a[kWaves];
#pragma unroll
        for (int k = 0; k < kWaves; ++k) {
          const bool in_b = k == lw && !lead_a;
          ml[k] = sm_ml[in_b ? 1 : 0][k][hh];
          const float* src = in_b ? reinterpret_cast<const float*>(&sm_v[k][0][0]) : &sm_acc[k][0][0];
          a[k] = *reinterpret_cast<const float2*>(&src[hh * D + d]);
        }
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < kWaves; ++k)
          if (part[k]) M = fmaxf(M, ml[k].y);
        float num0 = 0.f, num1 = 0.f, den = 0.f;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) {
          if (!part[k] || ml[k].x == -INFINITY) continue;  // no visible key of this piece in that wavefront
          const float sc = exp2f(ml[k].x - M);
          num0 = fmaf(a[k].x, sc, num0);
          num1 = fmaf(a[k].y, sc, num1);
          den = fmaf(ml[k].z, sc, den);
        }
        const int64_t pidx = (int64_t)(g * G + hh) * p.num_partials + slot;
        *reinterpret_cast<float2*>(&p.o_part[pidx * D + d]) = make_float2(num0 / den, num1 / den);
        if (d == 0) *reinterpret_cast<float2*>(&p.ml_part[pidx * 2]) = make_float2(M * kLn2, den);
      }
    }
    __syncthreads();
  }
#if ASTR_PHASE_STAMPS
  if (tid == 0) {
    const int id = blockIdx.y * gridDim.x + blockIdx.x;
    if (id < kStampWgs) {
      unsigned long long* d = g_decode_stamps[id];
      d[0] = stamp_start;
      d[1] = stamp_staged;
      d[2] = stamp_first;
      d[3] = __builtin_amdgcn_s_memrealtime();
      d[4] = __builtin_amdgcn_s_getreg(4 | (31 << 11));    // HW_ID: CU, shader array and engine of the wave
      d[5] = __builtin_amdgcn_s_getreg(20 | (31 << 11));   // XCC_ID: the accelerator die
      d[6] = (unsigned long long)(bnext - stamp_b0);      // pieces
      d[7] = 1;
    }
  }
#endif
}

// One work group per (request, combine_head_blocks blocks of kHeads query
// heads), each block with combine_groups groups of 64 threads (the host picks
// the group count from the longest request's piece count, and merges up to 4
// head blocks into one work group only for large grids, which launch faster
// as fewer, larger work groups; any group count gives the same result up to
// rounding order, the head-block count does not change it at all).  Thread t of a group owns four consecutive
// output elements of one head (float4 loads) and folds pieces r, r + groups,
// ... of the request, w_first..w_last (r = its group), into (M, den, num)
// with an online log-sum-exp merge, kBatch pieces at a time so that their
// loads are in flight together.  The groups of a block then merge through
// LDS in group order, and group 0 writes O (bf16, round to nearest even) and
// lse = M + ln(den).
constexpr int kBatch = 8;
constexpr int kMaxCombineGroups = 8;
constexpr int kCombineGroupThreads = kWave;
constexpr int kMaxCombineThreads = 1024;
// LDS slots for the groups r > 0 of all head blocks: groups x blocks <= 16.
constexpr int kCombineSlots = kMaxCombineThreads / kCombineGroupThreads - 1;

template <int D>
struct CombineShape {
  static constexpr int kHeads = kCombineGroupThreads * 4 / D;   // query heads per head block
};

template <int D, int G>
__global__ __launch_bounds__(kMaxCombineThreads) void decode_combine_kernel(const DecodeLaunch p) {
  constexpr int HP = CombineShape<D>::kHeads;
  __shared__ float4 s_num[kCombineSlots][kCombineGroupThreads];
  __shared__ float s_m[kCombineSlots][kCombineGroupThreads];
  __shared__ float s_den[kCombineSlots][kCombineGroupThreads];
  const int b = blockIdx.x;
  const int t = threadIdx.x % kCombineGroupThreads;
  const int ngrp = p.combine_groups;
  const int grp = (threadIdx.x / kCombineGroupThreads) % ngrp;
  const int hb = threadIdx.x / (kCombineGroupThreads * ngrp);
  const int h = (blockIdx.y * p.combine_head_blocks + hb) * HP + t / (D / 4);
  const int d4 = 4 * (t % (D / 4));
  const bool live = h < p.num_qo_heads;
  const int hc = live ? h : p.num_qo_heads - 1;   // idle threads read a valid row
  const int64_t N = p.kv_indptr[p.batch];
  const int64_t x0 = p.kv_indptr[b];
  const int64_t x1 = (int64_t)p.kv_indptr[b + 1] - 1;
  const int64_t W = min((int64_t)p.num_splits, N);
  const int wf = (int)(((x0 + 1) * W + N - 1) / N - 1);
  const int wl = (int)(((x1 + 1) * W + N - 1) / N - 1);
  const int n = wl - wf + 1;
  const int64_t base = (int64_t)hc * p.num_partials + b + wf;
  const float* ml = p.ml_part + base * 2;
  const float* op = p.o_part + base * D + d4;
  float M = -INFINITY, den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = grp; i0 < n; i0 += kBatch * ngrp) {
    float m[kBatch], l[kBatch];
    float4 o[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int pi = min(i0 + i * ngrp, n - 1);
      const float2 mlv = *reinterpret_cast<const float2*>(ml + 2 * pi);
      m[i] = mlv.x;
      l[i] = mlv.y;
      o[i] = *reinterpret_cast<const float4*>(op + (int64_t)pi * D);
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (i0 + i * ngrp < n) Mb = fmaxf(Mb, m[i]);
    // M == -inf before the first piece with a visible key: num and den are 0
    // and stay so (no 0 * inf).
    const float sc = M == Mb ? 1.f : expf(M - Mb);
    den *= sc;
    num.x *= sc; num.y *= sc; num.z *= sc; num.w *= sc;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      // A piece whose keys are all hidden by the mask has m = -inf and no
      // defined o or l: it adds nothing.
      if (i0 + i * ngrp >= n || m[i] == -INFINITY) continue;
      const float wgt = l[i] * expf(m[i] - Mb);
      den += wgt;
      num.x = fmaf(wgt, o[i].x, num.x);
      num.y = fmaf(wgt, o[i].y, num.y);
      num.z = fmaf(wgt, o[i].z, num.z);
      num.w = fmaf(wgt, o[i].w, num.w);
    }
    M = Mb;
  }
  if (ngrp > 1) {
    const int slot0 = hb * (ngrp - 1) - 1;   // slot of group r of this head block: slot0 + r
    if (grp > 0) {
      s_num[slot0 + grp][t] = num;
      s_m[slot0 + grp][t] = M;
      s_den[slot0 + grp][t] = den;
    }
    __syncthreads();
    if (grp > 0) return;
    for (int k = 1; k < ngrp; ++k) {
      const float mk = s_m[slot0 + k][t];
      if (mk == -INFINITY) continue;   // group had no piece
      const float Mn = fmaxf(M, mk);
      const float a = M == -INFINITY ? 0.f : expf(M - Mn), c = expf(mk - Mn);   // M = -inf: group 0 saw no visible key
      const float4 nk = s_num[slot0 + k][t];
      den = den * a + s_den[slot0 + k][t] * c;
      num.x = num.x * a + nk.x * c;
      num.y = num.y * a + nk.y * c;
      num.z = num.z * a + nk.z * c;
      num.w = num.w * a + nk.w * c;
      M = Mn;
    }
  }
  if (!live) return;
  // No visible key in the whole request (possible only with a mask): O = 0, lse = -inf.
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const uint32_t w0 = (uint32_t)f32_to_bf16_rne(num.x * inv) | ((uint32_t)f32_to_bf16_rne(num.y * inv) << 16);
  const uint32_t w1 = (uint32_t)f32_to_bf16_rne(num.z * inv) | ((uint32_t)f32_to_bf16_rne(num.w * inv) << 16);
  *reinterpret_cast<uint2*>(p.o + (int64_t)b * p.o_stride_tok + (int64_t)h * p.o_stride_head + d4) = make_uint2(w0, w1);
  if (p.lse != nullptr && d4 == 0) p.lse[(int64_t)b * p.lse_stride_tok + h] = den > 0.f ? M + logf(den) : -INFINITY;
}

template <int D, int G>
hipError_t launch_split_t(const DecodeLaunch& p, hipStream_t s, const Timing& t) {
  const dim3 grid(p.num_splits, p.num_kv_heads, 1);
  const int variant = (p.off32 ? 4 : 0) + (p.k_new != nullptr ? 2 : 0) + (p.mask != nullptr ? 1 : 0);
  switch (variant) {
    case 0: return launch_kernel(decode_split_kernel<D, G, false, false, false>, grid, dim3(kThreads), s, t, p);
    case 1: return launch_kernel(decode_split_kernel<D, G, false, false, true>, grid, dim3(kThreads), s, t, p);
    case 2: return launch_kernel(decode_split_kernel<D, G, false, true, false>, grid, dim3(kThreads), s, t, p);
    case 3: return launch_kernel(decode_split_kernel<D, G, false, true, true>, grid, dim3(kThreads), s, t, p);
    case 4: return launch_kernel(decode_split_kernel<D, G, true, false, false>, grid, dim3(kThreads), s, t, p);
    case 5: return launch_kernel(decode_split_kernel<D, G, true, false, true>, grid, dim3(kThreads), s, t, p);
    case 6: return launch_kernel(decode_split_kernel<D, G, true, true, false>, grid, dim3(kThreads), s, t, p);
    default: return launch_kernel(decode_split_kernel<D, G, true, true, true>, grid, dim3(kThreads), s, t, p);
  }
}

template <int D, int G>
hipError_t launch_combine_t(const DecodeLaunch& p, hipStream_t s, const Timing& t) {
  constexpr int HP = CombineShape<D>::kHeads;
  const int blocks = (p.num_qo_heads + HP - 1) / HP;
  const int nhb = p.combine_head_blocks;
  if (p.combine_groups < 1 || p.combine_groups > kMaxCombineGroups || nhb < 1 ||
      p.combine_groups * nhb * kCombineGroupThreads > kMaxCombineThreads)
    return hipErrorInvalidConfiguration;
  const dim3 grid(p.batch, (blocks + nhb - 1) / nhb, 1);
  return launch_kernel(decode_combine_kernel<D, G>, grid, dim3(kCombineGroupThreads * p.combine_groups * nhb), s, t, p);
}

#define ASTR_DECODE_CASES(FN)                       \
  switch (p.head_dim * 100 + p.group) {             \
    case 3201: return FN<32, 1>(p, s, t);              \
    case 3202: return FN<32, 2>(p, s, t);              \
    case 3204: return FN<32, 4>(p, s, t);              \
    case 3208: return FN<32, 8>(p, s, t);              \
    case 6401: return FN<64, 1>(p, s, t);              \
    case 6402: return FN<64, 2>(p, s, t);              \
    case 6404: return FN<64, 4>(p, s, t);              \
    case 6408: return FN<64, 8>(p, s, t);              \
    case 12801: return FN<128, 1>(p, s, t);            \
    case 12802: return FN<128, 2>(p, s, t);            \
    case 12804: return FN<128, 4>(p, s, t);            \
    case 12808: return FN<128, 8>(p, s, t);            \
    case 25601: return FN<256, 1>(p, s, t);            \
    case 25602: return FN<256, 2>(p, s, t);            \
    case 25604: return FN<256, 4>(p, s, t);            \
    case 25608: return FN<256, 8>(p, s, t);            \
    default: return hipErrorInvalidValue;           \
  }

}  // namespace

bool decode_supported(int head_dim, int group) {
  return (head_dim == 32 || head_dim == 64 || head_dim == 128 || head_dim == 256) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_decode_split(const DecodeLaunch& p, hipStream_t s, const Timing& t) { ASTR_DECODE_CASES(launch_split_t) }

hipError_t launch_decode_combine(const DecodeLaunch& p, hipStream_t s, const Timing& t) { ASTR_DECODE_CASES(launch_combine_t) }

}  // namespace astr

#if ASTR_PHASE_STAMPS
// Timeline-stamp builds only: copy out or clear the split work groups'
// records ([kStampWgs][8] unsigned 64-bit, work group id = y * grid_x + x:
// start, kv_indptr staged, first tile issued, end (100 MHz clock), HW_ID,
// XCC_ID, pieces, 1 when written).
extern "C" int astr_debug_decode_stamps(void* host, size_t bytes) {
  if (bytes < sizeof(astr::g_decode_stamps)) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(astr::g_decode_stamps), sizeof(astr::g_decode_stamps));
}
extern "C" int astr_debug_decode_stamps_clear(void) {
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(astr::g_decode_stamps));
  if (e != hipSuccess) return (int)e;
  return (int)hipMemset(ptr, 0, sizeof(astr::g_decode_stamps));
}
#endif
