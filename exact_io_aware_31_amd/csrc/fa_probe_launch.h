// fa_probe_launch.h -- launchers of the measurement kernels (fa_probe.hip).
// Arguments are checked by fa_probe_api.cpp before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa_probe {

hipError_t launch_mfma(float* out, unsigned long long* stamps, int blocks, int iters,
                       hipStream_t s);
hipError_t launch_stream_read(const void* buf, size_t bytes, unsigned* out, int blocks,
                              hipStream_t s);

}  // namespace fa_probe
