// Top-n block selection per (video row, KV group) from block importance
// (top168.com digest of VideoNSA, section 一: the selection branch keeps the
// most important segments).  Forced blocks (the first n_init and the n_local
// most recent ones up to the row's own block) are always taken and count
// inside n; the free places go to the remaining candidates by importance,
// ties to the lower block index.  Output ascending, -1 padded.
//
// One wave per (row, group).  The free places are filled in k rounds; round r
// takes the wave-wide best candidate that ranks strictly after the pick of
// round r-1 in the total order (importance desc, index asc), so no pick can
// repeat and no per-lane list is needed.  Each lane caches its first 32
// strided candidates in registers; longer rows re-read the rest from L1/L2.
#include "common.hpp"

#define TOPK_MAXN 32
#define TOPK_REG 32

// (a, ja) ranks before (b, jb)
__device__ __forceinline__ bool before(float a, int ja, float b, int jb) { return a > b || (a == b && ja < jb); }

__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ imp, const uint8_t* __restrict__ vid,
                                                   int32_t* __restrict__ idx, Dims dm) {
  __shared__ int s_items[4][64];
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
  const int64_t t = dm.q0 + r;
  const int jt = (int)(t / dm.ls);
  const int nj = (int)((jt + 1 < dm.Ns) ? jt + 1 : dm.Ns);
  const int lo_cnt = dm.n_init < nj ? dm.n_init : nj;
  int hi0 = jt - dm.n_local + 1;
  if (hi0 < lo_cnt) hi0 = lo_cnt;
  const int nf = lo_cnt + (nj > hi0 ? nj - hi0 : 0);
  const int k = dm.n - nf;  // >= 0 (validated: n >= n_init + n_local)
  const float* row = imp + rr * dm.Hkv * dm.Ns + (int64_t)g * dm.Ns;

  // free candidates are j in [lo_cnt, hi0)
  float cache[TOPK_REG];
#pragma unroll
  for (int c = 0; c < TOPK_REG; ++c) {
    const int j = lo_cnt + lane + 64 * c;
    cache[c] = (j < hi0) ? row[j] : -INFINITY;
  }
  const int jspill = lo_cnt + 64 * TOPK_REG;  // first candidate not cached

  int ntot = 0;
  for (int j = 0; j < lo_cnt; ++j) s_items[wv][ntot++] = j;
  for (int j = hi0; j < nj; ++j) s_items[wv][ntot++] = j;
  float pv = INFINITY;
  int pj = -1;
  for (int round = 0; round < k; ++round) {
    float bv = -INFINITY;
    int bj = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < TOPK_REG; ++c) {
      const int j = lo_cnt + lane + 64 * c;
      const float x = cache[c];
      if (j < hi0 && before(pv, pj, x, j) && before(x, j, bv, bj)) {
        bv = x;
        bj = j;
      }
    }
    for (int j = jspill + lane; j < hi0; j += 64) {
      const float x = row[j];
      if (before(pv, pj, x, j) && before(x, j, bv, bj)) {
        bv = x;
        bj = j;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oj = __shfl_xor(bj, o, 64);
      if (before(ov, oj, bv, bj)) {
        bv = ov;
        bj = oj;
      }
    }
    if (bj == 0x7fffffff) break;  // every free candidate is taken
    if (lane == 0) s_items[wv][ntot] = bj;
    ++ntot;
    pv = bv;
    pj = bj;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  int32_t* out = idx + (rr * dm.Hkv + g) * dm.n;
  if (lane < ntot) {
    const int me = s_items[wv][lane];
    int rank = 0;
    for (int c = 0; c < ntot; ++c) rank += (s_items[wv][c] < me);
    out[rank] = me;
  } else if (lane < dm.n) {
    out[lane] = -1;
  }
}

hipError_t launch_topk(const Dims& dm, const float* imp, const uint8_t* vid, int32_t* idx, hipStream_t s) {
  const int64_t total = dm.B * dm.Tq * dm.Hkv;
  if (total <= 0) return hipSuccess;
  const int64_t grid = (total + 3) / 4;
  topk_kernel<<<dim3((unsigned)grid), dim3(256), 0, s>>>(imp, vid, idx, dm);
  return hipGetLastError();
}
