// Kernel launch helper for the HIP sources (device compilation units only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace astr {

// Launches `kernel` with one argument struct; with timing events the
// dispatch itself stamps them at kernel start and end (hipExtLaunchKernel).
template <typename Kernel, typename Args>
hipError_t launch_kernel(Kernel kernel, dim3 grid, dim3 block, hipStream_t s, const Timing& t, const Args& args) {
  if (t.start != nullptr || t.stop != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t.start, t.stop, 0, args);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args);
  return hipGetLastError();
}

}  // namespace astr
