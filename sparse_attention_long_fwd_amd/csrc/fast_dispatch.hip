// Dispatch of the MFMA path: coverage test, workspace sizes, launch order.
#include "fast_common.hpp"

hipError_t launch_flash_fast(const Dims& dm, const void* q, const void* k, const void* v, const uint8_t* vid,
                             float* swa32, void* swa_bf, void* text, void* ws, hipStream_t s);
size_t flash_workspace(const Dims& dm);
hipError_t launch_slc_fast(const Dims& dm, const void* q, const void* k, const void* v, const int32_t* idx,
                           const uint8_t* vid, const void* ocmp, bool ocmp_f32, const float* swa32,
                           const float* gates, void* out, void* o_slc, hipStream_t s, bool head_major,
                           bool group_seq);

// [B, T, H, D] -> [B, H, T, D] copy, 16 bytes per thread.
__global__ void __launch_bounds__(256) head_major_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         int64_t T, int H, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // destination chunk
  if (i >= total) return;
  const int64_t c = i % 16;  // 16-byte chunk of a 128-element row
  int64_t rest = i / 16;
  const int64_t tt = rest % T;
  rest /= T;
  const int64_t h = rest % H, b = rest / H;
  dst[i] = src[((b * T + tt) * H + h) * 16 + c];
}

#include <stdlib.h>
static int slc_mode() {
  static int m = -1;
  if (m < 0) {
    const char* e = getenv("NSA_SLC_MODE");
    m = e ? atoi(e) : 0;
  }
  return m;
}

bool fast_supported(int32_t dtype, const Dims& dm) {
  return dtype == 1 && dm.D == 128 && dm.l == 32 && dm.d == 16 && dm.ls == 64 && dm.G >= 4 && dm.G <= 8 &&
         dm.n <= 32;
}

static size_t rup(size_t x) { return (x + 255) & ~(size_t)255; }

// [window output, fp32][split partials of long text rows][head-major K, V]
size_t fast_sparse_workspace(const Dims& dm) {
  return rup((size_t)dm.B * dm.Tq * dm.Hq * dm.D * 4) + rup(flash_workspace(dm)) +
         2 * rup((size_t)dm.B * dm.T * dm.Hkv * dm.D * 2);
}

hipError_t launch_sparse_fast(const Dims& dm, const void* q, const void* k, const void* v, const int32_t* idx,
                              const uint8_t* vid, const void* o_cmp, bool ocmp_f32, const float* gates, void* out,
                              void* o_slc, void* o_swa, void* ws, hipStream_t s, void (*mark)(hipStream_t)) {
  float* swa32 = (float*)ws;
  void* part = (char*)ws + rup((size_t)dm.B * dm.Tq * dm.Hq * dm.D * 4);
  // window branch (fp32 for the combine, bf16 copy if asked) and dense text rows
  hipError_t e = launch_flash_fast(dm, q, k, v, vid, swa32, o_swa, out, part, s);
  if (e != hipSuccess) return e;
  if (mark) mark(s);
  // selection branch and the gated combine of video rows
  const int mode = slc_mode();
  const bool head_major = mode & 1, group_seq = (mode & 2) != 0;
  if (head_major) {
    char* p = (char*)part + rup(flash_workspace(dm));
    const size_t kvb = rup((size_t)dm.B * dm.T * dm.Hkv * dm.D * 2);
    const int64_t total = dm.B * dm.T * dm.Hkv * 16;
    head_major_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s>>>((const uint4*)k, (uint4*)p, dm.T,
                                                                                   dm.Hkv, total);
    head_major_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s>>>((const uint4*)v,
                                                                                   (uint4*)(p + kvb), dm.T, dm.Hkv,
                                                                                   total);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_slc_fast(dm, q, p, p + kvb, idx, vid, o_cmp, ocmp_f32, swa32, gates, out, o_slc, s, true,
                           group_seq);
  }
  return launch_slc_fast(dm, q, k, v, idx, vid, o_cmp, ocmp_f32, swa32, gates, out, o_slc, s, false, group_seq);
}
