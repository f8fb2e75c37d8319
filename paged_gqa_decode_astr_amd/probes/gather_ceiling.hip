// Bandwidth ceilings for the paged decode access pattern on one GPU.
//
// Measures, with no attention arithmetic, how fast the K/V bytes of a decode
// batch can be brought in:
//   * gather: work group (w, g) of a (96, 8) grid reads the 256-byte K and V
//     segments of kv head g for its share of the request keys, whose pool
//     slots are a random permutation (page size one), 16 bytes per lane, one
//     load instruction covering 4 keys x 256 bytes;
//   * gather16: the same grid and bytes with the decode split kernel's load
//     shape, one instruction covering 16 keys x 64 bytes (4 lanes per key);
//   * gather_row: a 1-D grid of 768 work groups, each reading the whole
//     2 KB slot rows (all 8 kv heads) of K and V for its share of the keys;
//   * stream: the same number of bytes read contiguously;
//   * copy: a device-to-device copy of that many bytes (read + write).
// "cold" rotates over 4 independent pool pairs (2 GiB, well beyond the
// Infinity Cache); "warm" re-reads one pair with the same slots.
// Usage: gather_ceiling [keys]   (default 35200 keys, 8 kv heads, head_dim 128)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
      std::exit(1);                                                               \
    }                                                                             \
  } while (0)

namespace {

constexpr int kHeads = 8;
constexpr int kDim = 128;
constexpr int kRowElems = kHeads * kDim;   // bf16 elements per pool slot
constexpr int kSlots = 1 << 17;
constexpr int kSets = 4;

__global__ void gather(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
                       const int* __restrict__ slots, int n, uint32_t* sink) {
  const int W = gridDim.x, w = blockIdx.x, g = blockIdx.y;
  const int lo = (int)((long long)w * n / W), hi = (int)((long long)(w + 1) * n / W);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t acc = 0;
  for (int base = lo + wv * 16; base < hi; base += 64) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = min(base + u * 4 + lane / 16, hi - 1);
      const long long off = (long long)slots[i] * kRowElems + g * kDim + (lane % 16) * 8;
      v[u] = *reinterpret_cast<const uint4*>(kp + off);
      v[u + 4] = *reinterpret_cast<const uint4*>(vp + off);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;   // keeps the loads; practically never true
}

__global__ void gather16(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
                         const int* __restrict__ slots, int n, uint32_t* sink) {
  const int W = gridDim.x, w = blockIdx.x, g = blockIdx.y;
  const int lo = (int)((long long)w * n / W), hi = (int)((long long)(w + 1) * n / W);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t acc = 0;
  for (int base = lo + wv * 16; base < hi; base += 64) {
    const int i = min(base + lane / 4, hi - 1);
    const long long row = (long long)slots[i] * kRowElems + g * kDim + (lane % 4) * 8;
    uint4 v[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v[s] = *reinterpret_cast<const uint4*>(kp + row + 32 * s);
      v[s + 4] = *reinterpret_cast<const uint4*>(vp + row + 32 * s);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

__global__ void gather_row(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
                           const int* __restrict__ slots, int n, uint32_t* sink) {
  const int W = gridDim.x, w = blockIdx.x;
  const int lo = (int)((long long)w * n / W), hi = (int)((long long)(w + 1) * n / W);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t acc = 0;
  // Each wavefront takes 2 keys per step; one instruction reads half a 2 KB row.
  for (int base = lo + wv * 2; base < hi; base += 8) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = min(base + u, hi - 1);
      const long long row = (long long)slots[i] * kRowElems + lane * 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v[4 * u + h] = *reinterpret_cast<const uint4*>(kp + row + 512 * h);
        v[4 * u + 2 + h] = *reinterpret_cast<const uint4*>(vp + row + 512 * h);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

__global__ void stream(const uint4* __restrict__ a, long long n16, uint32_t* sink) {
  uint32_t acc = 0;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n16; i += (long long)gridDim.x * blockDim.x) {
    const uint4 v = a[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

template <typename F>
double time_us(F launch, int reps) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  for (int r = 0; r < 8; ++r) launch(r);
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(a));
  for (int r = 0; r < reps; ++r) launch(r);
  CHECK(hipEventRecord(b));
  CHECK(hipEventSynchronize(b));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, a, b));
  CHECK(hipEventDestroy(a));
  CHECK(hipEventDestroy(b));
  return ms * 1e3 / reps;
}

}  // namespace

int main(int argc, char** argv) {
  const int n = argc > 1 ? std::atoi(argv[1]) : 35200;
  if (n <= 0 || n > kSlots) {
    std::fprintf(stderr, "keys must be in [1, %d]\n", kSlots);
    return 2;
  }
  const size_t pool_bytes = (size_t)kSlots * kRowElems * 2;
  uint16_t* kp[kSets];
  uint16_t* vp[kSets];
  int* slots[kSets];
  uint32_t* sink;
  CHECK(hipMalloc(&sink, 64));
  std::mt19937 rng(20260101);
  for (int s = 0; s < kSets; ++s) {
    CHECK(hipMalloc(&kp[s], pool_bytes));
    CHECK(hipMalloc(&vp[s], pool_bytes));
    CHECK(hipMemset(kp[s], 1, pool_bytes));
    CHECK(hipMemset(vp[s], 2, pool_bytes));
    std::vector<int> perm(kSlots);
    for (int i = 0; i < kSlots; ++i) perm[i] = i;
    std::shuffle(perm.begin(), perm.end(), rng);
    CHECK(hipMalloc(&slots[s], n * sizeof(int)));
    CHECK(hipMemcpy(slots[s], perm.data(), n * sizeof(int), hipMemcpyHostToDevice));
  }
  const double bytes = (double)n * kHeads * kDim * 2 * 2;   // K + V segments
  const long long n16 = (long long)(bytes / 16);
  const int reps = 40;
  std::printf("| pattern | cache | us per pass | GB/s |\n|---|---|---|---|\n");
  for (int cold = 1; cold >= 0; --cold) {
    const double us = time_us([&](int r) {
      const int s = cold ? r % kSets : 0;
      hipLaunchKernelGGL(gather, dim3(96, kHeads), dim3(256), 0, 0, kp[s], vp[s], slots[s], n, sink);
    }, reps);
    std::printf("| gather: 256-byte K and V segments per (key, kv head), random slots | %s | %.2f | %.1f |\n",
                cold ? "cold (4 rotating pool pairs)" : "warm (one pool pair, same slots)", us, bytes / us * 1e-3);
  }
  for (int cold = 1; cold >= 0; --cold) {
    const double us = time_us([&](int r) {
      const int s = cold ? r % kSets : 0;
      hipLaunchKernelGGL(gather16, dim3(96, kHeads), dim3(256), 0, 0, kp[s], vp[s], slots[s], n, sink);
    }, reps);
    std::printf("| gather16: the same segments, 16 keys x 64 bytes per load instruction (the split kernel's shape) | %s | %.2f | %.1f |\n",
                cold ? "cold (4 rotating pool pairs)" : "warm (one pool pair, same slots)", us, bytes / us * 1e-3);
  }
  for (int cold = 1; cold >= 0; --cold) {
    const double us = time_us([&](int r) {
      const int s = cold ? r % kSets : 0;
      hipLaunchKernelGGL(gather_row, dim3(96 * kHeads), dim3(256), 0, 0, kp[s], vp[s], slots[s], n, sink);
    }, reps);
    std::printf("| gather_row: whole 2 KB K and V slot rows (all 8 kv heads) per key, random slots | %s | %.2f | %.1f |\n",
                cold ? "cold (4 rotating pool pairs)" : "warm (one pool pair, same slots)", us, bytes / us * 1e-3);
  }
  for (int cold = 1; cold >= 0; --cold) {
    const double us = time_us([&](int r) {
      const int s = cold ? r % kSets : 0;
      hipLaunchKernelGGL(stream, dim3(2048), dim3(256), 0, 0, reinterpret_cast<const uint4*>(kp[s]), n16, sink);
    }, reps);
    std::printf("| stream: the same byte count read contiguously | %s | %.2f | %.1f |\n",
                cold ? "cold (4 rotating buffers)" : "warm (one buffer)", us, bytes / us * 1e-3);
  }
  for (int cold = 1; cold >= 0; --cold) {
    const double us = time_us([&](int r) {
      const int s = cold ? r % kSets : 0;
      CHECK(hipMemcpyAsync(vp[(s + 1) % kSets], kp[s], (size_t)bytes, hipMemcpyDeviceToDevice, 0));
    }, reps);
    std::printf("| copy: device-to-device copy of the same byte count (read + write counted) | %s | %.2f | %.1f |\n",
                cold ? "cold (4 rotating buffers)" : "warm (one buffer)", us, 2 * bytes / us * 1e-3);
  }
  std::printf("\nkeys %d, kv heads %d, head_dim %d: %.1f MB of K and V per pass\n", n, kHeads, kDim, bytes / 1e6);
  for (int s = 0; s < kSets; ++s) {
    CHECK(hipFree(kp[s]));
    CHECK(hipFree(vp[s]));
    CHECK(hipFree(slots[s]));
  }
  CHECK(hipFree(sink));
  return 0;
}
