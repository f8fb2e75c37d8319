// Paged GQA decode for gfx950: split-KV kernel and log-sum-exp combine kernel.
//
// Method (AstrAI commit-list pages): [extension @6f67ba8], the commits that
// (a) read K/V through req_to_token as a page table with page size one,
// (b) turn decode into split-KV with o_part / ml_part partials merged by a
// separate combine kernel, (c) preload both K and V of a tile instead of
// looking up KV addresses per element in the softmax loop, and (d) drop the
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
// Inside a work group: 4 wavefronts take interleaved tiles of the piece.  A
// head row of D bf16 is covered by D/8 lanes with one 16-byte load each, so a
// wavefront-wide load fetches 64*16/(2*D) whole rows; each lane issues 4 K and
// 4 V loads per tile, all of them before any arithmetic.  The GQA group's G
// query heads share every K/V row fetched (one HBM read per row for G heads).
// Scores are reduced across the row's lanes with butterfly shuffles; softmax
// runs in base 2 with the scale folded into q; masked lanes (past the piece
// end) get exactly zero weight and their K/V are never read.  At the end of a
// piece the 4 wavefronts' (m, l, acc) states are merged through LDS and one
// normalised partial is written.
#include "device_common.hpp"
#include "launch.hpp"

namespace astr {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kLoads = 4;  // 16-byte K loads (and V loads) per lane per tile

template <int D>
struct RowMap {
  static constexpr int kLanesPerRow = D / 8;
  static constexpr int kRowsPerLoad = kWave / kLanesPerRow;
  static constexpr int kTile = kRowsPerLoad * kLoads;  // keys per wavefront per tile
};

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

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
__global__ __launch_bounds__(kThreads) void decode_split_kernel(const DecodeLaunch p) {
  constexpr int LPR = RowMap<D>::kLanesPerRow;
  constexpr int RPL = RowMap<D>::kRowsPerLoad;
  constexpr int TILE = RowMap<D>::kTile;
  __shared__ float sm_acc[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];

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
  const int r = lane / LPR;  // row within a load
  const int c = lane % LPR;  // 8-element chunk of the head row
  const float qscale = p.sm_scale * kLog2e;
  const int64_t kv_head_off = (int64_t)g * p.kv_stride_head + c * 8;

  int b = request_of(p.kv_indptr, B, e0);
  for (; b < B; ++b) {
    const int64_t kb0 = p.kv_indptr[b];
    const int64_t kb1 = p.kv_indptr[b + 1];
    if (kb0 >= e1) break;
    const int t_begin = (int)(max(e0, kb0) - kb0);
    const int t_end = (int)(min(e1, kb1) - kb0);
    const int32_t* ids = p.req_to_token + (p.req_to_token_stride > 0 ? (int64_t)b * p.req_to_token_stride : kb0);

    float qf[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint4 qv = load16(p.q + (int64_t)b * p.q_stride_tok + (int64_t)(g * G + hh) * p.q_stride_head + c * 8);
      unpack8(qv, qf[hh]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[hh][e] *= qscale;
    }
    float m[G], lsum[G], acc[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      m[hh] = -INFINITY;
      lsum[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
    }

    for (int tile0 = t_begin + wv * TILE; tile0 < t_end; tile0 += kWaves * TILE) {
      uint4 kr[kLoads], vr[kLoads];
      bool valid[kLoads];
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int t = tile0 + r + RPL * i;
        valid[i] = t < t_end;
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
        if (valid[i]) {
          const int64_t off = (int64_t)ids[t] * p.kv_stride_slot + kv_head_off;
          kr[i] = load16(p.k_pool + off);
          vr[i] = load16(p.v_pool + off);
        }
      }
      float s[kLoads][G];
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        float kf[8];
        unpack8(kr[i], kf);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) part = fmaf(qf[hh][e], kf[e], part);
          part = xor_sum<1, LPR>(part);
          s[i][hh] = valid[i] ? part : -INFINITY;
        }
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float tmax = s[0][hh];
#pragma unroll
        for (int i = 1; i < kLoads; ++i) tmax = fmaxf(tmax, s[i][hh]);
        tmax = xor_max<LPR, kWave>(tmax);
        const float mnew = fmaxf(m[hh], tmax);
        const float alpha = exp2f(m[hh] - mnew);
        m[hh] = mnew;
        lsum[hh] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha;
      }
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        float vf[8];
        unpack8(vr[i], vf);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float pr = exp2f(s[i][hh] - m[hh]);
          lsum[hh] += pr;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pr, vf[e], acc[hh][e]);
        }
      }
    }

    // Wavefront totals: sum over the rows held by different lane groups.
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      lsum[hh] = xor_sum<LPR, kWave>(lsum[hh]);
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
        sm_m[wv][hh] = m[hh];
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
      for (int k = 0; k < kWaves; ++k) M = fmaxf(M, sm_m[k][hh]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int k = 0; k < kWaves; ++k) {
        if (sm_m[k][hh] == -INFINITY) continue;  // wavefront had no key of this piece
        const float sc = exp2f(sm_m[k][hh] - M);
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
// of the request for the G query heads of kv head g.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(const DecodeLaunch p) {
  const int b = blockIdx.x;
  const int g = blockIdx.y;
  const int64_t N = p.kv_indptr[p.batch];
  const int64_t W = min((int64_t)p.num_splits, N);
  const int64_t x0 = p.kv_indptr[b];
  const int64_t x1 = (int64_t)p.kv_indptr[b + 1] - 1;
  const int wf = (int)(((x0 + 1) * W + N - 1) / N - 1);
  const int wl = (int)(((x1 + 1) * W + N - 1) / N - 1);
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int hh = idx / D;
    const int d = idx % D;
    const int h = g * G + hh;
    const int64_t base = (int64_t)h * p.num_partials + b;  // slot of piece w is w + b
    float M = -INFINITY;
    for (int w = wf; w <= wl; ++w) M = fmaxf(M, p.ml_part[(base + w) * 2]);
    float num = 0.f, den = 0.f;
    for (int w = wf; w <= wl; ++w) {
      const float wt = p.ml_part[(base + w) * 2 + 1] * expf(p.ml_part[(base + w) * 2] - M);
      den += wt;
      num = fmaf(wt, p.o_part[(base + w) * D + d], num);
    }
    p.o[(int64_t)b * p.o_stride_tok + (int64_t)h * p.o_stride_head + d] = f32_to_bf16_rne(num / den);
    if (p.lse != nullptr && d == 0) p.lse[(int64_t)b * p.lse_stride_tok + h] = M + logf(den);
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
