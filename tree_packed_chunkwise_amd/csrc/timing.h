// timing.h -- optional per-kernel launch timing (off unless kda_timing_enable(1)).
//
// When enabled, every kernel launch of the library is bracketed by a pair of
// hipEvents recorded on the launch stream; kda_timing_read() sums their
// elapsed times per kernel name.  Used by benchmarks to measure kernel
// durations live, next to rocprofv3's trace of the same run.
#pragma once

#include <hip/hip_runtime.h>

namespace kda {

bool timing_on();
void timing_begin(const char* name, hipStream_t st);
void timing_end(hipStream_t st);

}  // namespace kda

#define KDA_LAUNCH(name, kernel, grid, block, st, ...)               \
  do {                                                              \
    const bool kda_t_ = kda::timing_on();                           \
    if (kda_t_) kda::timing_begin(name, st);                        \
    hipLaunchKernelGGL(kernel, grid, block, 0, st, __VA_ARGS__);    \
    if (kda_t_) kda::timing_end(st);                                \
  } while (0)
