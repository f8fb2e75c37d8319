// Matrix cores against the vector ALU for the decode logits and P.V.
//
// Runs, on the same device buffers and the same split count, two decode
// paths of the decode microbench shape (32 requests with one query row each,
// GQA 32 / 8 heads, head_dim 128, seq_len ~ U{200..2000}, a 2^17-slot bf16
// pool read through a random-permutation token table):
//   * valu: the split + combine kernels this library first shipped, before
//     its decode moved to the matrix cores.  Per lane: one 16-byte chunk of a
//     key row; the logit of a (key, head) pair is an fp32 dot product of that
//     chunk with the query, summed over the 16 lanes of the row by
//     butterfly shuffles; online softmax per head; P.V as per-lane fp32
//     multiply-adds; the four wavefronts of a work group merge through LDS;
//     a combine kernel merges the splits by the log-sum-exp rule.
//   * mfma: astr_paged_decode, this library's current decode (logits and P.V
//     on v_mfma_f32_16x16x*_bf16, see csrc/decode.hip).
// Cold: each call uses the next of 4 input sets (2 GiB of pools in all, past
// the 256 MB Infinity Cache).  Prints per-call times from stream events and
// the largest output difference between the two paths; under
// `rocprofv3 --kernel-trace --stats` the per-kernel durations come out too.
// Usage: decode_valu [calls]   (default 200)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <random>
#include <vector>

#include "astr_attn.h"

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
      std::exit(1);                                                               \
    }                                                                             \
  } while (0)
#define CHECK_ASTR(x)                                                             \
  do {                                                                            \
    int s_ = (x);                                                                 \
    if (s_ != 0) {                                                                \
      std::fprintf(stderr, "%s failed: %s\n", #x, astr_last_error());            \
      std::exit(1);                                                               \
    }                                                                             \
  } while (0)

namespace {

constexpr int kB = 32, kHq = 32, kHkv = 8, kD = 128, kG = kHq / kHkv;
constexpr int kSlots = 1 << 17;
constexpr int kSets = 4;
constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kLoads = 4;                      // 16-byte K (and V) loads per lane per tile
constexpr int kLanesPerRow = kD / 8;           // 16 lanes hold one key row
constexpr int kRowsPerLoad = kWave / kLanesPerRow;
constexpr int kTile = kRowsPerLoad * kLoads;   // keys per wavefront per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct ValuArgs {
  int batch, num_splits, num_partials;
  float sm_scale;
  const uint16_t* q;
  uint16_t* o;
  float* lse;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* slots;      // flat token table, indexed from kv_indptr[b]
  const int32_t* kv_indptr;
  float* o_part;             // [Hq][P][D]
  float* ml_part;            // [Hq][P][2]
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ void widen8(const uint4& v, float (&f)[8]) {
  f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
template <int FROM, int TO>
__device__ __forceinline__ float bfly_sum(float v) {
#pragma unroll
  for (int m = FROM; m < TO; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
template <int FROM, int TO>
__device__ __forceinline__ float bfly_max(float v) {
#pragma unroll
  for (int m = FROM; m < TO; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// Work group (w, g): keys [w N / W, (w + 1) N / W) of kv head g, one piece
// per request the range touches; piece (w, b) writes partial slot w + b.
__global__ __launch_bounds__(kThreads) void valu_split(const ValuArgs p) {
  __shared__ float sm_acc[kWaves][kG][kD];
  __shared__ float sm_m[kWaves][kG];
  __shared__ float sm_l[kWaves][kG];
  const int w = blockIdx.x, g = blockIdx.y, B = p.batch;
  const int64_t N = p.kv_indptr[B];
  const int64_t W = min((int64_t)p.num_splits, N);
  if (w >= W) return;
  const int64_t e0 = (int64_t)w * N / W, e1 = (int64_t)(w + 1) * N / W;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int r = lane / kLanesPerRow, c = lane % kLanesPerRow;
  const float qscale = p.sm_scale * kLog2e;
  // First request whose range holds e0.
  int b = 0;
  for (int base = 1; base <= B; base += kThreads) {
    const int idx = base + tid;
    b += __syncthreads_count(idx <= B && (int64_t)p.kv_indptr[idx] <= e0);
  }
  for (; b < B; ++b) {
    const int64_t kb0 = p.kv_indptr[b], kb1 = p.kv_indptr[b + 1];
    if (kb0 >= e1) break;
    const int t_begin = (int)(max(e0, kb0) - kb0), t_end = (int)(min(e1, kb1) - kb0);
    const int32_t* ids = p.slots + kb0;
    float qf[kG][8];
#pragma unroll
    for (int hh = 0; hh < kG; ++hh) {
      widen8(*reinterpret_cast<const uint4*>(p.q + ((int64_t)b * kHq + g * kG + hh) * kD + c * 8), qf[hh]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[hh][e] *= qscale;
    }
    float m[kG], lsum[kG], acc[kG][8];
#pragma unroll
    for (int hh = 0; hh < kG; ++hh) {
      m[hh] = -INFINITY;
      lsum[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
    }
    for (int tile0 = t_begin + wv * kTile; tile0 < t_end; tile0 += kWaves * kTile) {
      uint4 kr[kLoads], vr[kLoads];
      bool valid[kLoads];
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int t = tile0 + r + kRowsPerLoad * i;
        valid[i] = t < t_end;
        kr[i] = vr[i] = make_uint4(0, 0, 0, 0);
        if (valid[i]) {
          const int64_t off = ((int64_t)ids[t] * kHkv + g) * kD + c * 8;
          kr[i] = *reinterpret_cast<const uint4*>(p.k_pool + off);
          vr[i] = *reinterpret_cast<const uint4*>(p.v_pool + off);
        }
      }
      float s[kLoads][kG];
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        float kf[8];
        widen8(kr[i], kf);
#pragma unroll
        for (int hh = 0; hh < kG; ++hh) {
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) part = fmaf(qf[hh][e], kf[e], part);
          part = bfly_sum<1, kLanesPerRow>(part);
          s[i][hh] = valid[i] ? part : -INFINITY;
        }
      }
#pragma unroll
      for (int hh = 0; hh < kG; ++hh) {
        float tmax = s[0][hh];
#pragma unroll
        for (int i = 1; i < kLoads; ++i) tmax = fmaxf(tmax, s[i][hh]);
        tmax = bfly_max<kLanesPerRow, kWave>(tmax);
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
        widen8(vr[i], vf);
#pragma unroll
        for (int hh = 0; hh < kG; ++hh) {
          const float pr = exp2f(s[i][hh] - m[hh]);
          lsum[hh] += pr;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pr, vf[e], acc[hh][e]);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < kG; ++hh) {
      lsum[hh] = bfly_sum<kLanesPerRow, kWave>(lsum[hh]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = bfly_sum<kLanesPerRow, kWave>(acc[hh][e]);
    }
    if (r == 0) {
#pragma unroll
      for (int hh = 0; hh < kG; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) sm_acc[wv][hh][c * 8 + e] = acc[hh][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int hh = 0; hh < kG; ++hh) {
        sm_m[wv][hh] = m[hh];
        sm_l[wv][hh] = lsum[hh];
      }
    }
    __syncthreads();
    for (int idx = tid; idx < kG * kD; idx += kThreads) {
      const int hh = idx / kD, d = idx % kD;
      float M = -INFINITY;
#pragma unroll
      for (int k = 0; k < kWaves; ++k) M = fmaxf(M, sm_m[k][hh]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int k = 0; k < kWaves; ++k) {
        if (sm_m[k][hh] == -INFINITY) continue;
        const float sc = exp2f(sm_m[k][hh] - M);
        num = fmaf(sm_acc[k][hh][d], sc, num);
        den = fmaf(sm_l[k][hh], sc, den);
      }
      const int64_t pidx = (int64_t)(g * kG + hh) * p.num_partials + w + b;
      p.o_part[pidx * kD + d] = num / den;
      if (d == 0) {
        p.ml_part[pidx * 2 + 0] = M * kLn2;
        p.ml_part[pidx * 2 + 1] = den;
      }
    }
    __syncthreads();
  }
}

// Work group (b, g): merges the pieces of request b for the heads of kv head g.
__global__ __launch_bounds__(kThreads) void valu_combine(const ValuArgs p) {
  const int b = blockIdx.x, g = blockIdx.y;
  const int64_t N = p.kv_indptr[p.batch];
  const int64_t W = min((int64_t)p.num_splits, N);
  const int64_t x0 = p.kv_indptr[b], x1 = (int64_t)p.kv_indptr[b + 1] - 1;
  const int wf = (int)(((x0 + 1) * W + N - 1) / N - 1), wl = (int)(((x1 + 1) * W + N - 1) / N - 1);
  for (int idx = threadIdx.x; idx < kG * kD; idx += kThreads) {
    const int hh = idx / kD, d = idx % kD, h = g * kG + hh;
    const int64_t base = (int64_t)h * p.num_partials + b;
    float M = -INFINITY;
    for (int w = wf; w <= wl; ++w) M = fmaxf(M, p.ml_part[(base + w) * 2]);
    float num = 0.f, den = 0.f;
    for (int w = wf; w <= wl; ++w) {
      const float wt = p.ml_part[(base + w) * 2 + 1] * expf(p.ml_part[(base + w) * 2] - M);
      den += wt;
      num = fmaf(wt, p.o_part[(base + w) * kD + d], num);
    }
    p.o[((int64_t)b * kHq + h) * kD + d] = to_bf16(num / den);
    if (d == 0) p.lse[(int64_t)b * kHq + h] = M + logf(den);
  }
}

// Pool and query contents: bf16 values of a hash of the element index, in
// about [-1, 1) (no arithmetic of the method; only bytes to read).
__global__ void fill_bf16(uint16_t* dst, int64_t n, uint32_t seed) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    uint32_t x = (uint32_t)i * 2654435761u ^ seed;
    x ^= x >> 15; x *= 2246822519u; x ^= x >> 13;
    const float f = (float)(x & 0xffffu) / 32768.f - 1.f;
    dst[i] = (uint16_t)(__float_as_uint(f) >> 16);
  }
}

float bf16_to_f32(uint16_t v) {
  uint32_t u = (uint32_t)v << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

struct Set {
  uint16_t *q, *k, *v, *o_valu, *o_mfma;
  float *lse_valu, *lse_mfma;
  int32_t *slots, *kv_indptr;
  std::vector<int32_t> kv_host;
  void* ws;
  size_t ws_bytes;
};

}  // namespace

int main(int argc, char** argv) {
  const int calls = argc > 1 ? std::atoi(argv[1]) : 200;
  if (calls < 1) return 2;
  const int64_t pool_elems = (int64_t)kSlots * kHkv * kD;
  std::vector<Set> sets(kSets);
  for (int s = 0; s < kSets; ++s) {
    Set& S = sets[s];
    std::mt19937 rng(20260500 + s);
    std::uniform_int_distribution<int> len(200, 2000);
    S.kv_host.assign(kB + 1, 0);
    for (int b = 0; b < kB; ++b) S.kv_host[b + 1] = S.kv_host[b] + len(rng);
    const int N = S.kv_host[kB];
    std::vector<int32_t> perm(kSlots);
    std::iota(perm.begin(), perm.end(), 0);
    std::shuffle(perm.begin(), perm.end(), rng);
    CHECK(hipMalloc(&S.q, (size_t)kB * kHq * kD * 2));
    CHECK(hipMalloc(&S.k, (size_t)pool_elems * 2));
    CHECK(hipMalloc(&S.v, (size_t)pool_elems * 2));
    CHECK(hipMalloc(&S.o_valu, (size_t)kB * kHq * kD * 2));
    CHECK(hipMalloc(&S.o_mfma, (size_t)kB * kHq * kD * 2));
    CHECK(hipMalloc(&S.lse_valu, (size_t)kB * kHq * 4));
    CHECK(hipMalloc(&S.lse_mfma, (size_t)kB * kHq * 4));
    CHECK(hipMalloc(&S.slots, (size_t)N * 4));
    CHECK(hipMalloc(&S.kv_indptr, (size_t)(kB + 1) * 4));
    CHECK(hipMemcpy(S.slots, perm.data(), (size_t)N * 4, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(S.kv_indptr, S.kv_host.data(), (size_t)(kB + 1) * 4, hipMemcpyHostToDevice));
    hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, S.q, (int64_t)kB * kHq * kD, 0x1000u + s);
    hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, S.k, pool_elems, 0x2000u + s);
    hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, S.v, pool_elems, 0x3000u + s);
    CHECK(hipGetLastError());
  }
  auto args_of = [&](Set& S, uint16_t* o, float* lse) {
    astr_paged_args a;
    std::memset(&a, 0, sizeof(a));
    a.batch = kB; a.num_qo_heads = kHq; a.num_kv_heads = kHkv; a.head_dim = kD;
    a.sm_scale = 1.f / std::sqrt((float)kD);
    a.q = S.q; a.q_stride_tok = kHq * kD; a.q_stride_head = kD;
    a.o = o; a.o_stride_tok = kHq * kD; a.o_stride_head = kD;
    a.lse = lse; a.lse_stride_tok = kHq;
    a.k_pool = S.k; a.v_pool = S.v; a.kv_stride_slot = kHkv * kD; a.kv_stride_head = kD; a.num_slots = kSlots;
    a.req_to_token = S.slots; a.req_to_token_stride = 0;
    a.kv_indptr = S.kv_indptr; a.kv_indptr_host = S.kv_host.data();
    return a;
  };
  // One plan (split count) for both paths: the library's for set 0.
  astr_decode_plan plan;
  {
    astr_paged_args a = args_of(sets[0], sets[0].o_mfma, sets[0].lse_mfma);
    CHECK_ASTR(astr_plan_decode(&a, 0, &plan));
  }
  for (Set& S : sets) {
    S.ws_bytes = astr_workspace_size(kB, kHq, kD, plan.num_splits);
    CHECK(hipMalloc(&S.ws, S.ws_bytes));
  }
  auto run_valu = [&](Set& S) {
    ValuArgs p;
    p.batch = kB; p.num_splits = plan.num_splits; p.num_partials = plan.num_splits + kB - 1;
    p.sm_scale = 1.f / std::sqrt((float)kD);
    p.q = S.q; p.o = S.o_valu; p.lse = S.lse_valu; p.k_pool = S.k; p.v_pool = S.v;
    p.slots = S.slots; p.kv_indptr = S.kv_indptr;
    p.o_part = static_cast<float*>(S.ws);
    const size_t opart = ((size_t)kHq * p.num_partials * kD * 4 + 255) / 256 * 256;
    p.ml_part = reinterpret_cast<float*>(static_cast<char*>(S.ws) + opart);
    hipLaunchKernelGGL(valu_split, dim3(plan.num_splits, kHkv), dim3(kThreads), 0, 0, p);
    hipLaunchKernelGGL(valu_combine, dim3(kB, kHkv), dim3(kThreads), 0, 0, p);
  };
  auto run_mfma = [&](Set& S) {
    astr_paged_args a = args_of(S, S.o_mfma, S.lse_mfma);
    a.num_splits = plan.num_splits;
    CHECK_ASTR(astr_paged_decode(&a, S.ws, S.ws_bytes, nullptr));
  };
  // Outputs of both paths on every set, then the largest difference.
  float max_diff = 0.f;
  for (Set& S : sets) {
    run_valu(S);
    run_mfma(S);
    CHECK(hipDeviceSynchronize());
    std::vector<uint16_t> ov((size_t)kB * kHq * kD), om(ov.size());
    CHECK(hipMemcpy(ov.data(), S.o_valu, ov.size() * 2, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(om.data(), S.o_mfma, om.size() * 2, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < ov.size(); ++i) max_diff = std::max(max_diff, std::fabs(bf16_to_f32(ov[i]) - bf16_to_f32(om[i])));
  }
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  auto time_us = [&](auto run) {
    for (int k = 0; k < 20; ++k) run(sets[k % kSets]);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    for (int k = 0; k < calls; ++k) run(sets[k % kSets]);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    return ms * 1e3 / calls;
  };
  const double us_valu = time_us(run_valu);
  const double us_mfma = time_us(run_mfma);
  std::printf("| decode path | us per call (cold, %d calls over %d sets) |\n|---|---|\n", calls, kSets);
  std::printf("| valu: per-lane fp32 dot products + shuffles, split + combine | %.2f |\n", us_valu);
  std::printf("| mfma: astr_paged_decode (v_mfma logits and P.V), split + combine | %.2f |\n", us_mfma);
  std::printf("\nB=%d Hq=%d Hkv=%d D=%d, %d work groups per kv head; max |O_valu - O_mfma| = %.3g\n", kB, kHq,
              kHkv, kD, plan.num_splits, max_diff);
  for (Set& S : sets) {
    CHECK(hipFree(S.q)); CHECK(hipFree(S.k)); CHECK(hipFree(S.v));
    CHECK(hipFree(S.o_valu)); CHECK(hipFree(S.o_mfma)); CHECK(hipFree(S.lse_valu)); CHECK(hipFree(S.lse_mfma));
    CHECK(hipFree(S.slots)); CHECK(hipFree(S.kv_indptr)); CHECK(hipFree(S.ws));
  }
  return 0;
}
