// LDS access patterns of the prefill kernel's tile loop, one kernel each.
//
// Each kernel repeats one pattern many times over a 64-row bf16 tile (head
// dim 128) held in LDS with a given row stride; run it under
//   rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS
// to see the bank-conflict cycles of each pattern, or alone for the time per
// instruction.  Patterns:
//   k_read<S>:   MFMA A-operand reads of the K tile (lane l: row l % 16 of a
//                16-row block, 16-byte chunk 4 ks + l / 16), ds_read_b128;
//   v_tr<S>:     transposing reads of the V tile (ds_read_b64_tr_b16), lane
//                j of a 16-lane group at row 4 (l / 16) + j / 4, columns
//                4 (j % 4) .. of a 16-column block;
//   store<S, M>: 16-byte stores of a gathered tile; M = 0: thread t stores
//                key t / 4 at chunks 4 (t % 4) + i (quarters of a row per
//                thread); M = 1: threads 8u + j store keys 4 (u / 2) + u % 2
//                and two rows further, chunks 4 i + j % 4;
//   k_read_swz, v_tr_swz: the same reads from unpadded rows (stride D)
//                whose 16-byte chunk c of row r sits at chunk c ^ 2 (r % 8),
//                the layout the direct global-to-LDS gather writes.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
      std::exit(1);                                                               \
    }                                                                             \
  } while (0)

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
constexpr int kD = 128, kKeys = 64, kIters = 2000;

template <int S>
__global__ void k_read(uint32_t* out) {
  __shared__ __align__(16) uint16_t t[kKeys * S];
  const int tid = threadIdx.x, l16 = tid & 15, kb = (tid & 63) >> 4;
  for (int i = tid; i < kKeys * S / 8; i += 256) reinterpret_cast<uint4*>(t)[i] = make_uint4(i, i, i, i);
  __syncthreads();
  uint32_t acc = 0;
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(&t[(16 * tb + l16) * S + ((32 * ks + 8 * kb) ^ ((it & 1) << 3))]);
        acc += a.x ^ a.y ^ a.z ^ a.w;
      }
    asm volatile("" ::: "memory");
  }
  out[blockIdx.x * 256 + tid] = acc;
}

template <int S>
__global__ void v_tr(uint32_t* out) {
  __shared__ __align__(16) uint16_t t[kKeys * S];
  const int tid = threadIdx.x, l16 = tid & 15, kb = (tid & 63) >> 4;
  for (int i = tid; i < kKeys * S / 8; i += 256) reinterpret_cast<uint4*>(t)[i] = make_uint4(i, i, i, i);
  __syncthreads();
  uint32_t acc = 0;
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (32 * k2 + 4 * kb + (l16 >> 2)) * S + 16 * db + 4 * (l16 & 3)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (32 * k2 + 16 + 4 * kb + (l16 >> 2)) * S + 16 * db + 4 * (l16 & 3)));
        acc += (uint32_t)(lo[0] ^ lo[1] ^ lo[2] ^ lo[3] ^ hi[0] ^ hi[1] ^ hi[2] ^ hi[3]) + (uint32_t)it;
      }
    asm volatile("" ::: "memory");
  }
  out[blockIdx.x * 256 + tid] = acc;
}

template <int S, int M>
__global__ void store(uint32_t* out) {
  __shared__ __align__(16) uint16_t t[kKeys * S];
  const int tid = threadIdx.x;
  const int key = M == 0 ? tid / 4 : 4 * (tid / 16) + (tid / 8) % 2 + 2 * ((tid % 8) / 4);
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = M == 0 ? 4 * (tid % 4) + i : 4 * i + tid % 4;
      *reinterpret_cast<uint4*>(&t[key * S + 8 * chunk]) = make_uint4(it, i, tid, 0);
    }
    asm volatile("" ::: "memory");
  }
  __syncthreads();
  out[blockIdx.x * 256 + tid] = t[tid * 3];
}


__global__ void k_read_swz(uint32_t* out) {
  __shared__ __align__(16) uint16_t t[kKeys * kD];
  const int tid = threadIdx.x, l16 = tid & 15, kb = (tid & 63) >> 4;
  for (int i = tid; i < kKeys * kD / 8; i += 256) reinterpret_cast<uint4*>(t)[i] = make_uint4(i, i, i, i);
  __syncthreads();
  const int sw = 2 * (l16 & 7);
  uint32_t acc = 0;
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(&t[(16 * tb + l16) * kD + 8 * (((4 * ks + kb) ^ sw) ^ (it & 1))]);
        acc += a.x ^ a.y ^ a.z ^ a.w;
      }
    asm volatile("" ::: "memory");
  }
  out[blockIdx.x * 256 + tid] = acc;
}

__global__ void v_tr_swz(uint32_t* out) {
  __shared__ __align__(16) uint16_t t[kKeys * kD];
  const int tid = threadIdx.x, l16 = tid & 15, kb = (tid & 63) >> 4;
  for (int i = tid; i < kKeys * kD / 8; i += 256) reinterpret_cast<uint4*>(t)[i] = make_uint4(i, i, i, i);
  __syncthreads();
  const int sw = 2 * ((4 * kb + (l16 >> 2)) & 7);
  uint32_t acc = 0;
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int col = 8 * ((2 * db + ((l16 & 3) >> 1)) ^ sw) + 4 * (l16 & 1);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (32 * k2 + 4 * kb + (l16 >> 2)) * kD + col));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (32 * k2 + 16 + 4 * kb + (l16 >> 2)) * kD + col));
        acc += (uint32_t)(lo[0] ^ lo[1] ^ lo[2] ^ lo[3] ^ hi[0] ^ hi[1] ^ hi[2] ^ hi[3]) + (uint32_t)it;
      }
    asm volatile("" ::: "memory");
  }
  out[blockIdx.x * 256 + tid] = acc;
}

template <typename K>
void run(const char* name, K kern, uint32_t* out) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  hipLaunchKernelGGL(kern, dim3(256), dim3(256), 0, 0, out);
  CHECK(hipEventRecord(a));
  hipLaunchKernelGGL(kern, dim3(256), dim3(256), 0, 0, out);
  CHECK(hipEventRecord(b));
  CHECK(hipEventSynchronize(b));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, a, b));
  std::printf("| %s | %.1f |\n", name, ms * 1e3);
  CHECK(hipEventDestroy(a));
  CHECK(hipEventDestroy(b));
}

}  // namespace

int main() {
  uint32_t* out;
  CHECK(hipMalloc(&out, 256 * 256 * 4));
  // Each kernel runs twice (the first launch warms up); the counters read
  // the same per launch.
  std::printf("| pattern (row stride in elements) | kernel time (us) |\n|---|---|\n");
  run("k_read, stride D+8", k_read<kD + 8>, out);
  run("k_read, stride D+16", k_read<kD + 16>, out);
  run("v_tr, stride D+8", v_tr<kD + 8>, out);
  run("v_tr, stride D+16", v_tr<kD + 16>, out);
  run("store quarters (M=0), stride D+8", store<kD + 8, 0>, out);
  run("store quarters (M=0), stride D+16", store<kD + 16, 0>, out);
  run("store paired rows (M=1), stride D+16", store<kD + 16, 1>, out);
  run("k_read, stride D, chunks XOR-swizzled", k_read_swz, out);
  run("v_tr, stride D, chunks XOR-swizzled", v_tr_swz, out);
  CHECK(hipDeviceSynchronize());
  CHECK(hipFree(out));
  return 0;
}
