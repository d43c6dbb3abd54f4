// Top-n block selection per (video row, KV group) from block importance
// (top168.com digest of VideoNSA, section 一: the selection branch keeps the
// most important segments).  Forced blocks (the first n_init and the n_local
// most recent ones up to the row's own block) are always taken and count
// inside n; the free places go to the remaining candidates by importance,
// ties to the lower block index.  Output ascending, -1 padded.
//
// One wave per (row, group); the selection itself is wave_select.
#include "topk_wave.hpp"

__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ imp, const uint8_t* __restrict__ vid,
                                                   int32_t* __restrict__ idx, Dims dm) {
  __shared__ TopkScratch s_sc[4];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * 4 + wv;
  const int64_t total = dm.B * dm.Tq * dm.Hkv;
  if (item >= total) return;
  const int g = (int)(item % dm.Hkv);
  const int64_t rr = item / dm.Hkv;
  const int64_t r = rr % dm.Tq;
  const int64_t b = rr / dm.Tq;
  if (vid && !vid[b * dm.Tq + r]) return;
  int lo, hi, nj;
  const int kk = tk_bounds(dm.q0 + r, dm.ls, dm.Ns, dm.n, dm.n_init, dm.n_local, &lo, &hi, &nj);
  wave_select(imp + (rr * dm.Hkv + g) * dm.Ns, lo, hi, nj, kk, dm.n, &s_sc[wv], idx + (rr * dm.Hkv + g) * dm.n,
              lane);
}

hipError_t launch_topk(const Dims& dm, const float* imp, const uint8_t* vid, int32_t* idx, hipStream_t s) {
  const int64_t total = dm.B * dm.Tq * dm.Hkv;
  if (total <= 0) return hipSuccess;
  const int64_t grid = (total + 3) / 4;
  topk_kernel<<<dim3((unsigned)grid), dim3(256), 0, s>>>(imp, vid, idx, dm);
  return hipGetLastError();
}
