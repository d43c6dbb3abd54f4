#include "fast.hpp"
bool fast_supported(int32_t, const Dims&) { return false; }
size_t fast_sparse_workspace(const Dims&) { return 0; }
hipError_t launch_cmp_fast(int, const Dims&, const void*, const void*, const void*, const uint8_t*, void*, float*, float*,
                           hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_sparse_fast(const Dims&, const void*, const void*, const void*, const int32_t*, const uint8_t*,
                              const void*, const float*, void*, void*, void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
