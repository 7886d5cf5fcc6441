// bf16 MFMA kernels for gfx950 (placeholder until the MFMA kernels land).
#include "device.h"
#include "kata.h"

namespace kata {
bool quadratic_fast_supported(const kata_problem*) { return false; }
bool chunk_fast_available() { return false; }
hipError_t launch_quadratic_fast(const DevProblem&, bool, const void*, const void*, const void*,
                                 void*, float*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_chunk_state_fast(const DevProblem&, int, int, const void*, const void*, float*,
                                   hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_chunk_output_fast(const DevProblem&, bool, int, int, const void*, const void*,
                                    const void*, void*, float*, const float*, hipStream_t) {
  return hipErrorInvalidValue;
}
}  // namespace kata
