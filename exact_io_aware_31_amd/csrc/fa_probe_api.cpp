// fa_probe_api.cpp -- host side of libfa_probe (include/fa_probe.h): argument
// checks and launches of the two measurement kernels in fa_probe.hip.
#include "../../include/fa_probe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_probe_launch.h"

extern "C" {

int fa_probe_mfma_bf16(float* out, unsigned long long* stamps, int blocks, int iters,
                       void* stream) {
  if (!out || !stamps) return 1;
  if (blocks < 1 || iters < 1 || blocks > (1 << 20) || iters > (1 << 24)) return 2;
  if ((reinterpret_cast<uintptr_t>(out) & 3) || (reinterpret_cast<uintptr_t>(stamps) & 7)) return 4;
  return fa_probe::launch_mfma(out, stamps, blocks, iters, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? 0
             : 7;
}

int fa_probe_stream_read(const void* buf, size_t bytes, unsigned* out, int blocks, void* stream) {
  if (!buf || !out) return 1;
  if (blocks < 1 || blocks > (1 << 20) || bytes == 0 || bytes % FA_PROBE_READ_CHUNK != 0) return 2;
  if ((reinterpret_cast<uintptr_t>(buf) & 15) || (reinterpret_cast<uintptr_t>(out) & 3)) return 4;
  return fa_probe::launch_stream_read(buf, bytes, out, blocks, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? 0
             : 7;
}

}  // extern "C"
