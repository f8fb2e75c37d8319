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
// Inside a work group, 4 wavefronts take interleaved 16-key tiles of a piece.
// Per tile and wavefront:
//  * K is fetched in the B-operand layout of v_mfma_f32_16x16x32_bf16 (lane
//    l holds 8 bf16 of key l % 16; four lanes cover 64 contiguous bytes of a
//    row per load), and the logits of all G query heads of the GQA group come
//    out of D/32 MFMAs whose A operand repeats the group's q rows, so every
//    lane receives the G logits of its own key.  Each K/V row is read from HBM
//    once for all G heads.
//  * V is fetched row-wise (D/8 lanes per 2D-byte row) and P.V runs on the
//    VALU in fp32; the softmax weights cross from the MFMA layout to the row
//    layout through a small wavefront-private LDS buffer.
//  * The next tile's K/V loads and the slot ids two tiles ahead are issued
//    before the current tile is computed (register double buffering).
//  * Softmax runs in base 2 against a lazily raised reference max: the
//    accumulators are rescaled only when a logit exceeds the reference by more
//    than kTau (so weights stay <= 2^kTau); the exact running max is tracked
//    alongside and the written (m, l) pair uses it.  Keys past the piece end
//    are never read and weigh exactly zero.
// At the end of a piece the 4 wavefronts merge through LDS and one normalised
// partial (o, m, l) per query head is written.
#include "device_common.hpp"
#include "launch.hpp"

namespace astr {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTile = 16;       // keys per wavefront per tile (one MFMA column block)
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

template <int D, int G>
struct Shape {
  static constexpr int kSteps = D / 32;            // MFMA k-steps over the head dim
  static constexpr int kPasses = (G + 3) / 4;      // MFMAs per k-step (4 heads per pass)
  static constexpr int kLanesPerRow = D / 8;       // V row layout: lanes per head row
  static constexpr int kRowsPerLoad = kWave / kLanesPerRow;
  static constexpr int kVLoads = kTile / kRowsPerLoad;
};

template <int D, int G>
struct Tile {
  uint4 k[Shape<D, G>::kSteps];
  uint4 v[Shape<D, G>::kVLoads];
};

template <int D, int G>
__device__ __forceinline__ void load_tile(Tile<D, G>& t, const DecodeLaunch& p, int id_k, int t0, int t_end,
                                          int64_t head_off, int lane) {
  using S = Shape<D, G>;
  const int l16 = lane & 15;
  const int kb = lane >> 4;
  const int r = lane / S::kLanesPerRow;
  const int c = lane % S::kLanesPerRow;
  const bool kvalid = t0 + l16 < t_end;
  const int64_t kbase = (int64_t)id_k * p.kv_stride_slot + head_off;
#pragma unroll
  for (int s = 0; s < S::kSteps; ++s)
    t.k[s] = kvalid ? load16(p.k_pool + kbase + 32 * s + 8 * kb) : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < S::kVLoads; ++i) {
    const int tok = r + S::kRowsPerLoad * i;                 // key within the tile
    const int id_v = __shfl(id_k, tok, kWave);               // lane `tok` holds that key's slot
    const bool vvalid = t0 + tok < t_end;
    t.v[i] = vvalid ? load16(p.v_pool + (int64_t)id_v * p.kv_stride_slot + head_off + 8 * c) : make_uint4(0, 0, 0, 0);
  }
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(const DecodeLaunch p) {
  using S = Shape<D, G>;
  constexpr int LPR = S::kLanesPerRow;
  constexpr int RPL = S::kRowsPerLoad;
  constexpr int GP = (G + 3) / 4 * 4;   // p row padded to whole 16-byte vectors
  __shared__ float sm_acc[kWaves][G][D];
  __shared__ float sm_mref[kWaves][G];
  __shared__ float sm_mx[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  __shared__ __align__(16) float sm_p[kWaves][kTile][GP];

  const int w = blockIdx.x;
  const int g = blockIdx.y;
  const int B = p.batch;
  const int64_t N = p.kv_indptr[B];
  const int64_t W = min((int64_t)p.num_splits, N);
  if (w >= W) return;  // uniform over the work group
  const int64_t e0 = ((int64_t)w * N) / W;
  const int64_t e1 = ((int64_t)(w + 1) * N) / W;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int l16 = lane & 15;
  const int kb = lane >> 4;
  const int r = lane / LPR;
  const int c = lane % LPR;
  const float qscale = p.sm_scale * kLog2e;
  const int64_t head_off = (int64_t)g * p.kv_stride_head;
  constexpr int kStep = kWaves * kTile;   // keys between a wavefront's consecutive tiles

  int b = request_of(p.kv_indptr, B, e0);
  for (; b < B; ++b) {
    const int64_t kb0 = p.kv_indptr[b];
    const int64_t kb1 = p.kv_indptr[b + 1];
    if (kb0 >= e1) break;
    const int t_begin = (int)(max(e0, kb0) - kb0);
    const int t_end = (int)(min(e1, kb1) - kb0);
    const int32_t* ids = p.req_to_token + (p.req_to_token_stride > 0 ? (int64_t)b * p.req_to_token_stride : kb0);

    // Slot ids (MFMA layout: lane l <-> key l % 16) and K/V of the first tile.
    int tile0 = t_begin + wv * kTile;
    int id_cur = (tile0 + l16 < t_end) ? ids[tile0 + l16] : 0;
    int id_next = (tile0 + kStep + l16 < t_end) ? ids[tile0 + kStep + l16] : 0;
    Tile<D, G> cur, nxt;
    if (tile0 < t_end) load_tile<D, G>(cur, p, id_cur, tile0, t_end, head_off, lane);

    // A operand: row i of pass ps is query head (4 ps + i % 4) % G of the group.
    bf16x8 qa[S::kPasses][S::kSteps];
#pragma unroll
    for (int ps = 0; ps < S::kPasses; ++ps) {
      const int hh = (4 * ps + (l16 & 3)) % G;
      const uint16_t* qrow = p.q + (int64_t)b * p.q_stride_tok + (int64_t)(g * G + hh) * p.q_stride_head;
#pragma unroll
      for (int s = 0; s < S::kSteps; ++s) qa[ps][s] = __builtin_bit_cast(bf16x8, load16(qrow + 32 * s + 8 * kb));
    }

    float mref[G], mx[G], lsum[G], acc[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      mref[hh] = -INFINITY;
      mx[hh] = -INFINITY;
      lsum[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
    }

    for (; tile0 < t_end; tile0 += kStep) {
      const int tnext = tile0 + kStep;
      if (tnext < t_end) load_tile<D, G>(nxt, p, id_next, tnext, t_end, head_off, lane);
      const int tnn = tnext + kStep;
      const int id_nn = (tnn + l16 < t_end) ? ids[tnn + l16] : 0;

      // Logits of key l16 for every head of the group, in log2 units.
      float sc[G];
#pragma unroll
      for (int ps = 0; ps < S::kPasses; ++ps) {
        f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < S::kSteps; ++s) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ps][s], __builtin_bit_cast(bf16x8, cur.k[s]), st, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (4 * ps + q < G) sc[4 * ps + q] = st[q] * qscale;
      }
      const bool kvalid = tile0 + l16 < t_end;
      bool raise = false;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        if (!kvalid) sc[hh] = -INFINITY;
        mx[hh] = fmaxf(mx[hh], sc[hh]);
        raise |= sc[hh] > mref[hh] + kTau;
      }
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {   // uniform over the wavefront
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float tmax = xor_max<1, 16>(sc[hh]);
          const float mnew = fmaxf(mref[hh], tmax);
          const float alpha = exp2f(mref[hh] - mnew);
          mref[hh] = mnew;
          lsum[hh] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha;
        }
      }
      // Weights to the row layout through LDS (wavefront-private buffer).
      if (lane < kTile) {
        float pw[GP];
#pragma unroll
        for (int hh = 0; hh < GP; ++hh) pw[hh] = hh < G ? exp2f(sc[hh] - mref[hh]) : 0.f;
#pragma unroll
        for (int v4 = 0; v4 < GP / 4; ++v4)
          *reinterpret_cast<float4*>(&sm_p[wv][lane][4 * v4]) = make_float4(pw[4 * v4], pw[4 * v4 + 1], pw[4 * v4 + 2], pw[4 * v4 + 3]);
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < S::kVLoads; ++i) {
        const int tok = r + RPL * i;
        float pw[GP];
#pragma unroll
        for (int v4 = 0; v4 < GP / 4; ++v4) {
          const float4 x = *reinterpret_cast<const float4*>(&sm_p[wv][tok][4 * v4]);
          pw[4 * v4] = x.x; pw[4 * v4 + 1] = x.y; pw[4 * v4 + 2] = x.z; pw[4 * v4 + 3] = x.w;
        }
        float vf[8];
        unpack8(cur.v[i], vf);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          lsum[hh] += pw[hh];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pw[hh], vf[e], acc[hh][e]);
        }
      }
      __builtin_amdgcn_wave_barrier();
      cur = nxt;
      id_next = id_nn;
    }

    // Wavefront totals: rows of the V layout, and the exact max over keys.
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      lsum[hh] = xor_sum<LPR, kWave>(lsum[hh]);
      mx[hh] = xor_max<1, 16>(mx[hh]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = xor_sum<LPR, kWave>(acc[hh][e]);
    }
    if (r == 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) sm_acc[wv][hh][c * 8 + e] = acc[hh][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        sm_mref[wv][hh] = mref[hh];
        sm_mx[wv][hh] = mx[hh];
        sm_l[wv][hh] = lsum[hh];
      }
    }
    __syncthreads();
    const int slot = w + b;
    for (int idx = tid; idx < G * D; idx += kThreads) {
      const int hh = idx / D;
      const int d = idx % D;
      float M = -INFINITY;
#pragma unroll
      for (int k = 0; k < kWaves; ++k) M = fmaxf(M, sm_mx[k][hh]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int k = 0; k < kWaves; ++k) {
        if (sm_mref[k][hh] == -INFINITY) continue;  // wavefront had no key of this piece
        const float sc = exp2f(sm_mref[k][hh] - M);
        num = fmaf(sm_acc[k][hh][d], sc, num);
        den = fmaf(sm_l[k][hh], sc, den);
      }
      const int64_t pidx = (int64_t)(g * G + hh) * p.num_partials + slot;
      p.o_part[pidx * D + d] = num / den;
      if (d == 0) {
        p.ml_part[pidx * 2 + 0] = M * kLn2;
        p.ml_part[pidx * 2 + 1] = den;
      }
    }
    __syncthreads();
  }
}

// One work group per (request, kv head): merges the pieces w_first..w_last
// of the request for the G query heads of kv head g.  Pass 1: one wavefront
// per head reduces the max logit M and the total weight sum_s l_s e^(m_s - M).
// Pass 2: the weights of up to kChunk pieces are staged in LDS and every
// thread accumulates its (head, d) outputs with independent loads.
constexpr int kChunk = 64;

template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(const DecodeLaunch p) {
  constexpr int kPer = (G * D + kThreads - 1) / kThreads;   // outputs per thread
  __shared__ float s_w[G][kChunk];
  __shared__ float s_M[G];
  __shared__ float s_den[G];
  const int b = blockIdx.x;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int64_t N = p.kv_indptr[p.batch];
  const int64_t W = min((int64_t)p.num_splits, N);
  const int64_t x0 = p.kv_indptr[b];
  const int64_t x1 = (int64_t)p.kv_indptr[b + 1] - 1;
  const int wf = (int)(((x0 + 1) * W + N - 1) / N - 1);
  const int wl = (int)(((x1 + 1) * W + N - 1) / N - 1);
  const int n = wl - wf + 1;

  for (int hh = wv; hh < G; hh += kWaves) {
    const float* ml = p.ml_part + ((int64_t)(g * G + hh) * p.num_partials + b + wf) * 2;
    float M = -INFINITY;
    for (int i = lane; i < n; i += kWave) M = fmaxf(M, ml[2 * i]);
    M = xor_max<1, kWave>(M);
    float den = 0.f;
    for (int i = lane; i < n; i += kWave) den += ml[2 * i + 1] * expf(ml[2 * i] - M);
    den = xor_sum<1, kWave>(den);
    if (lane == 0) {
      s_M[hh] = M;
      s_den[hh] = den;
    }
  }
  __syncthreads();

  float num[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) num[j] = 0.f;
  for (int c0 = 0; c0 < n; c0 += kChunk) {
    const int cn = min(kChunk, n - c0);
    for (int idx = tid; idx < G * kChunk; idx += kThreads) {
      const int hh = idx / kChunk, i = idx % kChunk;
      if (i < cn) {
        const float* ml = p.ml_part + ((int64_t)(g * G + hh) * p.num_partials + b + wf + c0 + i) * 2;
        s_w[hh][i] = ml[1] * expf(ml[0] - s_M[hh]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = tid + j * kThreads;
      if (idx < G * D) {
        const int hh = idx / D, d = idx % D;
        const float* op = p.o_part + ((int64_t)(g * G + hh) * p.num_partials + b + wf + c0) * D + d;
        float a = num[j];
        for (int i = 0; i < cn; ++i) a = fmaf(s_w[hh][i], op[(int64_t)i * D], a);
        num[j] = a;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int idx = tid + j * kThreads;
    if (idx < G * D) {
      const int hh = idx / D, d = idx % D;
      const int h = g * G + hh;
      p.o[(int64_t)b * p.o_stride_tok + (int64_t)h * p.o_stride_head + d] = f32_to_bf16_rne(num[j] / s_den[hh]);
      if (p.lse != nullptr && d == 0) p.lse[(int64_t)b * p.lse_stride_tok + h] = s_M[hh] + logf(s_den[hh]);
    }
  }
}

template <int D, int G>
hipError_t launch_split_t(const DecodeLaunch& p, hipStream_t s) {
  hipLaunchKernelGGL((decode_split_kernel<D, G>), dim3(p.num_splits, p.num_kv_heads, 1), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_combine_t(const DecodeLaunch& p, hipStream_t s) {
  hipLaunchKernelGGL((decode_combine_kernel<D, G>), dim3(p.batch, p.num_kv_heads, 1), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

#define ASTR_DECODE_CASES(FN)                       \
  switch (p.head_dim * 100 + p.group) {             \
    case 6401: return FN<64, 1>(p, s);              \
    case 6402: return FN<64, 2>(p, s);              \
    case 6404: return FN<64, 4>(p, s);              \
    case 6408: return FN<64, 8>(p, s);              \
    case 12801: return FN<128, 1>(p, s);            \
    case 12802: return FN<128, 2>(p, s);            \
    case 12804: return FN<128, 4>(p, s);            \
    case 12808: return FN<128, 8>(p, s);            \
    default: return hipErrorInvalidValue;           \
  }

}  // namespace

bool decode_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_decode_split(const DecodeLaunch& p, hipStream_t s) { ASTR_DECODE_CASES(launch_split_t) }

hipError_t launch_decode_combine(const DecodeLaunch& p, hipStream_t s) { ASTR_DECODE_CASES(launch_combine_t) }

}  // namespace astr
