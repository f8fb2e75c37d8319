// Ragged paged GQA prefill for gfx950 with bf16 MFMA (v_mfma_f32_16x16x32_bf16).
//
// Method (AstrAI commit-list pages): [attention.py @c9ceca1], the commit that
// batches the torch path: query row i of request b sits at absolute position
// c_b + i with c_b = seq_len_b - q_len_b and sees keys 0 .. c_b + i; masked
// keys weigh exactly zero; rows are read and written in flat qo_indptr order.
// [extension @6f67ba8]: K/V come through req_to_token with page size one; the
// prefill kernel tiles over queries and uses matrix instructions for QK^T and
// PV; query head h reads kv head h / G.
//
// Work group = (query tile, kv head g, request b), 4 wavefronts.  The G query
// heads that share kv head g are stacked with the positions into 128 rows
// (row R = position * G + head), so each K/V tile staged in LDS serves all
// of them.  Per 64-key tile:
//   * K rows are staged row-major and V rows transposed (V^T[d][t]) in LDS;
//   * each wavefront computes S^T = K Q^T for its 32 rows (A = K from LDS,
//     B = Q^T held in registers), which leaves every lane with 16 logits of one
//     row, so the row max / sum need only two cross-lane steps;
//   * P^T is rounded to bf16 and fed straight back as the B operand of
//     O^T += V^T P^T (A = V^T read from LDS), with the key order inside each
//     32-key step permuted identically in both operands.
// Output rows are normalised by the row sum of the same bf16-rounded weights.
#include "device_common.hpp"
#include "kernel_launch.hpp"

namespace astr {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kThreads = 256;
constexpr int kRows = 128;  // (position, head) rows per work group
constexpr int KT = 64;      // keys per tile

__device__ __forceinline__ uint4 load16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void prefill_kernel(const PrefillLaunch p) {
  constexpr int BQ = kRows / G;     // query positions per work group
  constexpr int KSTR = D + 8;       // LDS row stride of K (elements)
  constexpr int VSTR = KT + 8;      // LDS row stride of V^T (elements)
  constexpr int DSTEPS = D / 32;    // k-steps of S^T = K Q^T
  constexpr int DBLK = D / 16;      // 16-wide d blocks of O^T
  constexpr int CPR = D / 8;        // 16-byte chunks per head row
  constexpr int RPP = kThreads / CPR;
  constexpr int PASSES = KT / RPP;
  __shared__ __align__(16) uint16_t sK[KT * KSTR];
  __shared__ __align__(16) uint16_t sVt[D * VSTR];

  const int qt = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int q0 = p.qo_indptr[b];
  const int qb = p.qo_indptr[b + 1] - q0;
  const int p0 = qt * BQ;
  if (p0 >= qb) return;  // uniform over the work group
  const int kv0 = p.kv_indptr[b];
  const int L = p.kv_indptr[b + 1] - kv0;
  const int cofs = L - qb;             // absolute position of query row 0
  const int npos = min(BQ, qb - p0);   // valid positions in this tile
  const int kv_end = cofs + p0 + npos; // keys [0, kv_end) are visible to some row
  const int32_t* ids = p.req_to_token + (p.req_to_token_stride > 0 ? (int64_t)b * p.req_to_token_stride : (int64_t)kv0);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int l16 = lane & 15;
  const int kb = lane >> 4;

  // B operand of S^T = K Q^T: lane (r + 16 kb) holds Q[row r][32 ks + 8 kb .. +7].
  bf16x8 qop[2][DSTEPS];
  int lim[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int R = 32 * wv + 16 * rb + l16;
    const int posl = R / G;
    const int head = g * G + R % G;
    lim[rb] = cofs + p0 + posl;  // last key this row may see
    const bool ok = posl < npos;
#pragma unroll
    for (int ks = 0; ks < DSTEPS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ok) v = load16(p.q + (int64_t)(q0 + p0 + posl) * p.q_stride_tok + (int64_t)head * p.q_stride_head + 32 * ks + 8 * kb);
      qop[rb][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const float qk_scale = p.sm_scale * kLog2e;
  f32x4 acc[2][DBLK];
  float m[2], lsum[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    m[rb] = -INFINITY;
    lsum[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int tl0 = tid / CPR;
  const int ch = tid % CPR;
  const int64_t head_off = (int64_t)g * p.kv_stride_head + ch * 8;

  for (int t0 = 0; t0 < kv_end; t0 += KT) {
    uint4 kreg[PASSES], vreg[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int t = t0 + tl0 + RPP * i;
      kreg[i] = make_uint4(0, 0, 0, 0);
      vreg[i] = make_uint4(0, 0, 0, 0);
      if (t < kv_end) {
        const int64_t off = (int64_t)ids[t] * p.kv_stride_slot + head_off;
        kreg[i] = load16(p.k_pool + off);
        vreg[i] = load16(p.v_pool + off);
      }
    }
    __syncthreads();  // the previous tile's LDS reads are complete
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int tl = tl0 + RPP * i;
      *reinterpret_cast<uint4*>(&sK[tl * KSTR + ch * 8]) = kreg[i];
      const uint32_t w4[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sVt[(ch * 8 + 2 * e) * VSTR + tl] = (uint16_t)(w4[e] & 0xffffu);
        sVt[(ch * 8 + 2 * e + 1) * VSTR + tl] = (uint16_t)(w4[e] >> 16);
      }
    }
    __syncthreads();

    const bool need_mask = (t0 + KT - 1) > (cofs + p0);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      // S^T blocks: st[tb][q] = S^T[t0 + 16 tb + 4 kb + q][row 16 rb + l16]
      f32x4 st[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        st[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DSTEPS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sK[(16 * tb + l16) * KSTR + 32 * ks + 8 * kb]);
          st[tb] = mfma16(a, qop[rb][ks], st[tb]);
        }
      }
      float sv[4][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float s = st[tb][q] * qk_scale;
          if (need_mask && (t0 + 16 * tb + 4 * kb + q) > lim[rb]) s = -INFINITY;
          sv[tb][q] = s;
          tmax = fmaxf(tmax, s);
        }
      tmax = xor_max<16, kWave>(tmax);
      const float mnew = fmaxf(m[rb], tmax);
      const float alpha = exp2f(m[rb] - mnew);
      m[rb] = mnew;
      lsum[rb] *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) acc[rb][db] *= alpha;

      uint32_t pk[4][2];
      float psum = 0.f;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const uint16_t lo = f32_to_bf16_rne(exp2f(sv[tb][2 * h2] - mnew));
          const uint16_t hi = f32_to_bf16_rne(exp2f(sv[tb][2 * h2 + 1] - mnew));
          psum += __uint_as_float((uint32_t)lo << 16) + __uint_as_float((uint32_t)hi << 16);
          pk[tb][h2] = (uint32_t)lo | ((uint32_t)hi << 16);
        }
      lsum[rb] += psum;

#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        // k-slot 8 kb + e holds key 32 k2 + 4 kb + e (e < 4) or 32 k2 + 16 + 4 kb + (e - 4).
        const bf16x8 bop = __builtin_bit_cast(bf16x8, make_uint4(pk[2 * k2][0], pk[2 * k2][1], pk[2 * k2 + 1][0], pk[2 * k2 + 1][1]));
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const uint16_t* vrow = &sVt[(16 * db + l16) * VSTR + 32 * k2 + 4 * kb];
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
          const bf16x8 aop = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
          acc[rb][db] = mfma16(aop, bop, acc[rb][db]);
        }
      }
    }
  }

  // acc[rb][db][q] = O^T[d = 16 db + 4 kb + q][row 16 rb + l16] (unnormalised)
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float ltot = xor_sum<16, kWave>(lsum[rb]);
    const int R = 32 * wv + 16 * rb + l16;
    const int posl = R / G;
    if (posl >= npos) continue;
    const int row = q0 + p0 + posl;
    const int head = g * G + R % G;
    const float inv = 1.f / ltot;
    uint16_t* orow = p.o + (int64_t)row * p.o_stride_tok + (int64_t)head * p.o_stride_head;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const uint32_t w0 = (uint32_t)f32_to_bf16_rne(acc[rb][db][0] * inv) | ((uint32_t)f32_to_bf16_rne(acc[rb][db][1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16_rne(acc[rb][db][2] * inv) | ((uint32_t)f32_to_bf16_rne(acc[rb][db][3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * db + 4 * kb) = make_uint2(w0, w1);
    }
    if (p.lse != nullptr && kb == 0) p.lse[(int64_t)row * p.lse_stride_tok + head] = (m[rb] + log2f(ltot)) * kLn2;
  }
}

template <int D, int G>
hipError_t launch_t(const PrefillLaunch& p, hipStream_t s, const Timing& t) {
  constexpr int BQ = kRows / G;
  const int qtiles = (p.max_q_len + BQ - 1) / BQ;
  return launch_kernel(prefill_kernel<D, G>, dim3(qtiles, p.num_kv_heads, p.batch), dim3(kThreads), s, t, p);
}

}  // namespace

bool prefill_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t s, const Timing& t) {
  switch (p.head_dim * 100 + p.group) {
    case 6401: return launch_t<64, 1>(p, s, t);
    case 6402: return launch_t<64, 2>(p, s, t);
    case 6404: return launch_t<64, 4>(p, s, t);
    case 6408: return launch_t<64, 8>(p, s, t);
    case 12801: return launch_t<128, 1>(p, s, t);
    case 12802: return launch_t<128, 2>(p, s, t);
    case 12804: return launch_t<128, 4>(p, s, t);
    case 12808: return launch_t<128, 8>(p, s, t);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace astr
