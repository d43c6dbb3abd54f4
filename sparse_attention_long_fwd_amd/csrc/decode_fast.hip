// Decode step (one query row per sequence) of the hybrid NSA layer, gfx950.
//
// Same definitions as the prefill path (top168.com digest of VideoNSA, section
// 一: compression, importance-scored selection, sliding window, per-head
// gates); the compressed cache comes in precomputed.  With one row per
// sequence the work is an HBM stream: the compressed cache (2 x Nc x D per KV
// head) dominates, then the chosen blocks and the window.  Parallelism comes
// from splitting the keys:
//
//  1. dcmp_split: one workgroup per (sequence, KV group, 128 compressed keys):
//     scores for the G heads (16x16x32 MFMA, heads on N), a local softmax, the
//     value sum, and the importance of the chunk's 32 selection blocks, all in
//     the chunk's own frame (max, sum), written as a partial.
//  2. dcmp_merge: one workgroup per (sequence, group): merges the partials per
//     head (log-sum-exp), rescales the importance partials to the final
//     normaliser, sums them over the heads, and picks the top-n blocks.
//  3. dsparse_blocks: one wave per (sequence, group, block of the union of the
//     chosen blocks and the window): scores once, then a selection partial and
//     a window partial with their own masks.
//  4. dsparse_merge: merges the block partials per head and applies the gated
//     combine.
#include "fast_common.hpp"

namespace {
constexpr int HD = 128;
constexpr int DCH = 128;           // compressed keys per split
constexpr int DBLK = DCH / 4;      // selection blocks per split (4 compressed keys per 64-token block)
constexpr int PSTRIDE = 2 + HD + DBLK + 1;  // per head: max, sum, O[128], E[32] + carry
constexpr int SB = 64;
}  // namespace

__device__ __forceinline__ void dwait() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// 1. compression-branch partials
template <bool SPLIT>
__global__ void __launch_bounds__(256) dcmp_split_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kh,
                                                         const bf16* __restrict__ kl, const bf16* __restrict__ vh,
                                                         const bf16* __restrict__ vl, const uint8_t* __restrict__ vid,
                                                         float* __restrict__ part, Dims dm, int nsplit) {
  constexpr int NA = SPLIT ? 2 : 1;  // staged V arrays (hi, lo)
  // per wave: V rows; after the value products the same bytes hold the waves' outputs [4][16][HD] fp32
  __shared__ __attribute__((aligned(16))) unsigned char d_smem[4 * NA * 32 * HD * 2];
  bf16* vt0 = (bf16*)d_smem;
  float(*s_o)[16][HD] = (float(*)[16][HD])d_smem;
  __shared__ float s_m[4][16], s_l[4][16];
  __shared__ float s_a[4][16][8], s_c[4][16][8];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, hn = l & 15, grp = l >> 4;
  const int s = blockIdx.x % nsplit;
  const int unit = blockIdx.x / nsplit;
  const int64_t b = unit / dm.Hkv;
  const int g = unit % dm.Hkv;
  if (vid && !vid[b]) return;
  const int G = dm.G;
  const int64_t t = dm.q0;
  const int64_t nv = cmp_visible(t, dm.l, dm.d, dm.Nc);
  const float c2 = dm.scale * LOG2E_F;
  const bool hvalid = hn < G;
  const int h = g * G + (hvalid ? hn : 0);
  bf16x8 qf[4];
  {
    const bf16* qrow = q + (b * dm.Hq + h) * (int64_t)HD + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = hvalid ? *(const bf16x8*)(qrow + 32 * ks) : zero8();
  }
  const int64_t stride = (int64_t)dm.Hkv * HD;
  const int64_t base = (b * dm.Nc * dm.Hkv + g) * (int64_t)HD;
  const int64_t k0 = (int64_t)s * DCH + 32 * w;  // this wave's 32 keys
  // stage V rows k0 .. k0+31 into this wave's LDS (16 B a lane, 8 instructions per array)
  auto stage = [&](bf16* dst, const bf16* src) {
#pragma unroll
    for (int ins = 0; ins < 8; ++ins) {
      const int p = ins * 64 + l, row = p >> 4, cpos = p & 15, c = cpos ^ (row & 15);
      int64_t key = k0 + row;
      if (key >= dm.Nc) key = dm.Nc - 1;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + key * stride + c * 8),
                                       (__attribute__((address_space(3))) void*)(dst + ins * 512), 16, 0, 0);
    }
  };
  bf16* vth = vt0 + (w * NA) * 32 * HD;
  bf16* vtl = vth + 32 * HD;
  stage(vth, vh + base);
  if constexpr (SPLIT) stage(vtl, vl + base);
  bf16x8 kf[2][4], kfl[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    int64_t key = k0 + 16 * kb + hn;
    if (key >= dm.Nc) key = dm.Nc - 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kf[kb][ks] = *(const bf16x8*)(kh + base + key * stride + 32 * ks + 8 * grp);
      if constexpr (SPLIT) kfl[kb][ks] = *(const bf16x8*)(kl + base + key * stride + 32 * ks + 8 * grp);
    }
  }
  f32x4 sc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    sc[kb] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      sc[kb] = mfma16(kf[kb][ks], qf[ks], sc[kb]);
      if constexpr (SPLIT) sc[kb] = mfma16(kfl[kb][ks], qf[ks], sc[kb]);
    }
  }
  float x[8];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int64_t key = k0 + 16 * kb + 4 * grp + jj;
      x[4 * kb + jj] = key < nv ? sc[kb][jj] * c2 : -INFINITY;
    }
  float mx = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  float p[8], ls = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = mx > -INFINITY ? fexp2(x[e] - mx) : 0.f;
    ls += p[e];
  }
  ls += __shfl_xor(ls, 16, 64);
  ls += __shfl_xor(ls, 32, 64);
  // importance pieces: this lane's 4 keys of sub-block kb are one selection block
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s_a[w][hn][4 * kb + grp] = p[4 * kb] + p[4 * kb + 1] + p[4 * kb + 2] + 0.5f * p[4 * kb + 3];
    s_c[w][hn][4 * kb + grp] = 0.5f * p[4 * kb + 3];
  }
  // O^T += V^T P^T over the 32 keys
  dwait();
  __builtin_amdgcn_wave_barrier();
  bf16x8 pb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pb[e] = (bf16)p[e];
    pb[4 + e] = (bf16)p[4 + e];
  }
  f32x4 oacc[8];
  const int vr = 4 * grp + (hn >> 2);
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const int col = 16 * db + 4 * (hn & 3);
    oacc[db] = mfma16(cat(lds_read_tr(vth + swz128(vr, col >> 3) + (col & 7)),
                          lds_read_tr(vth + swz128(vr + 16, col >> 3) + (col & 7))),
                      pb, f32x4{});
    if constexpr (SPLIT)
      oacc[db] = mfma16(cat(lds_read_tr(vtl + swz128(vr, col >> 3) + (col & 7)),
                            lds_read_tr(vtl + swz128(vr + 16, col >> 3) + (col & 7))),
                        pb, oacc[db]);
  }
  if (grp == 0) {
    s_m[w][hn] = mx;
    s_l[w][hn] = ls;
  }
  __syncthreads();  // every wave is done with its V rows
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_o[w][hn][16 * db + 4 * grp + e] = oacc[db][e];
  __syncthreads();
  // merge the 4 waves of the chunk into one partial per head
  float* pp = part + ((int64_t)unit * nsplit + s) * G * PSTRIDE;
  for (int i = threadIdx.x; i < G * (HD + DBLK + 1); i += 256) {
    const int hh = i / (HD + DBLK + 1), e = i % (HD + DBLK + 1);
    float M = -INFINITY;
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_m[ww][hh]);
    float sc_[4];
    for (int ww = 0; ww < 4; ++ww) sc_[ww] = (M > -INFINITY && s_m[ww][hh] > -INFINITY) ? fexp2(s_m[ww][hh] - M) : 0.f;
    float* ph = pp + hh * PSTRIDE;
    if (e < HD) {
      float o = 0.f;
      for (int ww = 0; ww < 4; ++ww) o += sc_[ww] * s_o[ww][hh][e];
      ph[2 + e] = o;
      if (e == 0) {
        float L = 0.f;
        for (int ww = 0; ww < 4; ++ww) L += sc_[ww] * s_l[ww][hh];
        ph[0] = M;
        ph[1] = L;
      }
    } else {
      const int jb = e - HD;  // 0..32: block of the chunk, 32 = carry into the next chunk's first block
      float v = 0.f;
      if (jb < DBLK) v += sc_[jb / 8] * s_a[jb / 8][hh][jb % 8];
      if (jb > 0) v += sc_[(jb - 1) / 8] * s_c[(jb - 1) / 8][hh][(jb - 1) % 8];
      ph[2 + HD + jb] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// 2. importance and top-n (one workgroup of 16 waves per (sequence, group))
__device__ __forceinline__ bool dbefore(float a, int ja, float b, int jb) { return a > b || (a == b && ja < jb); }

// Per-head softmax statistics of the split partials, one wave per head:
// s_fac[h][s] = exp2(m_s - M_h) / L_h (0 for empty splits), s_M[h], s_L[h].
__device__ __forceinline__ void dsplit_stats(const float* pu, int G, int nsplit, float* s_fac, float* s_M,
                                             float* s_L) {
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wv >= G) return;
  const int hh = wv;
  float m = -INFINITY;
  for (int s = lane; s < nsplit; s += 64) m = fmaxf(m, pu[(s * G + hh) * PSTRIDE]);
  const float M = wave_max(m);
  float l = 0.f;
  for (int s = lane; s < nsplit; s += 64) {
    const float ms = pu[(s * G + hh) * PSTRIDE];
    if (ms > -INFINITY) l += pu[(s * G + hh) * PSTRIDE + 1] * fexp2(ms - M);
  }
  const float L = wave_sum(l);
  for (int s = lane; s < nsplit; s += 64) {
    const float ms = pu[(s * G + hh) * PSTRIDE];
    s_fac[hh * nsplit + s] = (ms > -INFINITY && L > 0.f) ? fexp2(ms - M) / L : 0.f;
  }
  if (lane == 0) {
    s_M[hh] = M;
    s_L[hh] = L;
  }
}

__global__ void __launch_bounds__(1024) dcmp_merge_kernel(const float* __restrict__ part, const uint8_t* __restrict__ vid,
                                                          float* __restrict__ imp_out, int32_t* __restrict__ idx,
                                                          Dims dm, int nsplit) {
  extern __shared__ float dsm[];
  float* s_imp = dsm;             // [Ns]
  float* s_fac = dsm + dm.Ns;     // [G][nsplit]
  __shared__ float s_M[16], s_L[16];
  __shared__ float s_cv[4][32];   // per-wave candidates (value, index) for the final merge
  __shared__ int s_cj[4][32];
  __shared__ int s_items[64];
  const int unit = blockIdx.x;
  const int64_t b = unit / dm.Hkv;
  const int g = unit % dm.Hkv;
  if (vid && !vid[b]) return;
  const int G = dm.G, tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const float* pu = part + (int64_t)unit * nsplit * G * PSTRIDE;
  dsplit_stats(pu, G, nsplit, s_fac, s_M, s_L);
  __syncthreads();
  // importance of blocks 0 .. jt, heads summed in a fixed order
  const int64_t t = dm.q0;
  const int jt = (int)(t / dm.ls);
  for (int j = tid; j <= jt; j += blockDim.x) {
    const int s = j / DBLK, jb = j % DBLK;
    float a[8], c[8];
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
      a[hh] = (hh < G && s < nsplit) ? pu[(s * G + hh) * PSTRIDE + 2 + HD + jb] : 0.f;
      c[hh] = (hh < G && jb == 0 && s > 0) ? pu[((s - 1) * G + hh) * PSTRIDE + 2 + HD + DBLK] : 0.f;
    }
    float v = 0.f;
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
      if (hh < G && s < nsplit) v += s_fac[hh * nsplit + s] * a[hh];
      if (hh < G && jb == 0 && s > 0) v += s_fac[hh * nsplit + s - 1] * c[hh];
    }
    s_imp[j] = v;
    if (imp_out) imp_out[(b * dm.Hkv + g) * dm.Ns + j] = v;
  }
  __syncthreads();
  // top-n: the free candidates [lo_cnt, hi0) are split over 4 waves; each wave keeps its best k
  // (rounds of a wave-wide arg-max strictly below the previous pick), wave 0 merges the 4 lists.
  const int nj = jt + 1 < dm.Ns ? jt + 1 : (int)dm.Ns;
  const int lo_cnt = dm.n_init < nj ? dm.n_init : nj;
  int hi0 = jt - dm.n_local + 1;
  if (hi0 < lo_cnt) hi0 = lo_cnt;
  const int nf = lo_cnt + (nj > hi0 ? nj - hi0 : 0);
  const int k = dm.n - nf;
  if (wv < 4) {
    const int per = (hi0 - lo_cnt + 3) / 4;
    const int c0 = lo_cnt + wv * per, c1 = c0 + per < hi0 ? c0 + per : hi0;
    constexpr int NREG = 8;
    float cache[NREG];
#pragma unroll
    for (int c = 0; c < NREG; ++c) {
      const int j = c0 + lane + 64 * c;
      cache[c] = j < c1 ? s_imp[j] : -INFINITY;
    }
    float pv = INFINITY;
    int pj = -1;
    for (int round = 0; round < k; ++round) {
      float bv = -INFINITY;
      int bj = 0x7fffffff;
#pragma unroll
      for (int c = 0; c < NREG; ++c) {
        const int j = c0 + lane + 64 * c;
        if (j < c1 && dbefore(pv, pj, cache[c], j) && dbefore(cache[c], j, bv, bj)) {
          bv = cache[c];
          bj = j;
        }
      }
      for (int j = c0 + lane + 64 * NREG; j < c1; j += 64) {
        const float x = s_imp[j];
        if (dbefore(pv, pj, x, j) && dbefore(x, j, bv, bj)) {
          bv = x;
          bj = j;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oj = __shfl_xor(bj, o, 64);
        if (dbefore(ov, oj, bv, bj)) {
          bv = ov;
          bj = oj;
        }
      }
      if (lane == 0) {
        s_cv[wv][round] = bv;
        s_cj[wv][round] = bj;
      }
      pv = bv;
      pj = bj;
    }
  }
  __syncthreads();
  if (wv != 0) return;
  // merge: lane holds candidate (wave lane / 32... ) -- at most 4 x 32 entries, two per lane
  float v0 = -INFINITY, v1 = -INFINITY;
  int j0 = 0x7fffffff, j1 = 0x7fffffff;
  {
    const int w0 = lane >> 5, r0 = lane & 31;  // entries (w0, r0) and (w0 + 2, r0)
    if (r0 < k) {
      v0 = s_cv[w0][r0];
      j0 = s_cj[w0][r0];
      v1 = s_cv[w0 + 2][r0];
      j1 = s_cj[w0 + 2][r0];
    }
  }
  int ntot = 0;
  for (int j = 0; j < lo_cnt; ++j) s_items[ntot++] = j;
  for (int j = hi0; j < nj; ++j) s_items[ntot++] = j;
  float pv = INFINITY;
  int pj = -1;
  for (int round = 0; round < k; ++round) {
    float bv = -INFINITY;
    int bj = 0x7fffffff;
    if (j0 != 0x7fffffff && dbefore(pv, pj, v0, j0)) {
      bv = v0;
      bj = j0;
    }
    if (j1 != 0x7fffffff && dbefore(pv, pj, v1, j1) && dbefore(v1, j1, bv, bj)) {
      bv = v1;
      bj = j1;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oj = __shfl_xor(bj, o, 64);
      if (dbefore(ov, oj, bv, bj)) {
        bv = ov;
        bj = oj;
      }
    }
    if (bj == 0x7fffffff) break;
    if (lane == 0) s_items[ntot] = bj;
    ++ntot;
    pv = bv;
    pj = bj;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  int32_t* out = idx + (b * dm.Hkv + g) * dm.n;
  if (lane < ntot) {
    const int me = s_items[lane];
    int rank = 0;
    for (int c = 0; c < ntot; ++c) rank += (s_items[c] < me);
    out[rank] = me;
  } else if (lane < dm.n) {
    out[lane] = -1;
  }
}
// ---------------------------------------------------------------------------
// 3. selection / window partials per block of the union
// Slot k of a unit: the k-th block of (chosen blocks below the window) ++ (window blocks).
__device__ __forceinline__ int64_t union_block(const int32_t* sel, int n, int64_t jt, int64_t wb0, int k, bool* in_sel,
                                               bool* in_win) {
  int cnt_lt = 0;
  for (int c = 0; c < n; ++c)
    if (sel[c] >= 0 && sel[c] < wb0) {
      if (cnt_lt == k) {
        *in_sel = true;
        *in_win = false;
        return sel[c];
      }
      ++cnt_lt;
    }
  const int64_t j = wb0 + (k - cnt_lt);
  if (j > jt) return -1;
  bool s_ = false;
  for (int c = 0; c < n; ++c) s_ |= (sel[c] == j);
  *in_sel = s_;
  *in_win = true;
  return j;
}

__global__ void __launch_bounds__(256) dsparse_blocks_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                             const bf16* __restrict__ v,
                                                             const int32_t* __restrict__ idx,
                                                             const uint8_t* __restrict__ vid,
                                                             float* __restrict__ part3, Dims dm, int nslot) {
  __shared__ __attribute__((aligned(16))) bf16 vt[4][SB * HD];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, hn = l & 15, grp = l >> 4;
  const int slots_per_wg = 4;
  const int wgs = (nslot + slots_per_wg - 1) / slots_per_wg;
  const int unit = blockIdx.x / wgs;
  const int slot = (blockIdx.x % wgs) * slots_per_wg + w;
  const int64_t b = unit / dm.Hkv;
  const int g = unit % dm.Hkv;
  if (vid && !vid[b]) return;
  if (slot >= nslot) return;
  const int G = dm.G;
  const int64_t t = dm.q0, jt = t / SB;
  int64_t wlo = t - dm.w + 1;
  if (wlo < 0) wlo = 0;
  const int64_t wb0 = wlo / SB;
  const int32_t* sel = idx + (b * dm.Hkv + g) * dm.n;
  bool in_sel = false, in_win = false;
  const int64_t j = union_block(sel, dm.n, jt, wb0, slot, &in_sel, &in_win);
  float* ps = part3 + (((int64_t)unit * nslot + slot) * 2) * G * (HD + 2);
  if (j < 0) {  // unused slot: empty partials
    for (int i = l; i < 2 * G; i += 64) ps[(i / G) * G * (HD + 2) + (i % G) * (HD + 2) + 1] = 0.f;
    return;
  }
  const float c2 = dm.scale * LOG2E_F;
  const bool hvalid = hn < G;
  const int h = g * G + (hvalid ? hn : 0);
  bf16x8 qf[4];
  {
    const bf16* qrow = q + (b * dm.Hq + h) * (int64_t)HD + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = hvalid ? *(const bf16x8*)(qrow + 32 * ks) : zero8();
  }
  const int64_t stride = (int64_t)dm.Hkv * HD;
  const bf16* kbase = k + (b * dm.T * dm.Hkv + g) * (int64_t)HD;
  const bf16* vbase = v + (b * dm.T * dm.Hkv + g) * (int64_t)HD;
  stage_tile64(vt[w], vbase, stride, j * SB, dm.T, 0, 1, l);
  f32x4 sc[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    int64_t key = j * SB + 16 * kb + hn;
    if (key >= dm.T) key = dm.T - 1;
    const bf16* kr = kbase + key * stride + 8 * grp;
    sc[kb] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) sc[kb] = mfma16(*(const bf16x8*)(kr + 32 * ks), qf[ks], sc[kb]);
  }
  dwait();
  __builtin_amdgcn_wave_barrier();
  for (int br = 0; br < 2; ++br) {
    const bool act = br == 0 ? in_sel : in_win;
    float* pb_ = ps + br * G * (HD + 2);
    if (!act) {
      if (hvalid && grp == 0) pb_[hn * (HD + 2) + 1] = 0.f;
      continue;
    }
    float x[16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int64_t u = j * SB + 16 * kb + 4 * grp + jj;
        const bool ok = br == 0 ? (u <= t) : (u <= t && u >= wlo);
        x[4 * kb + jj] = ok ? sc[kb][jj] * c2 : -INFINITY;
      }
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float p[16], ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = mx > -INFINITY ? fexp2(x[e] - mx) : 0.f;
      ls += p[e];
    }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    f32x4 oacc[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] = f32x4{};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pb[e] = (bf16)p[4 * (2 * st) + e];
        pb[4 + e] = (bf16)p[4 * (2 * st + 1) + e];
      }
      const int vr = 32 * st + 4 * grp + (hn >> 2);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int col = 16 * db + 4 * (hn & 3);
        oacc[db] = mfma16(cat(lds_read_tr(vt[w] + swz128(vr, col >> 3) + (col & 7)),
                              lds_read_tr(vt[w] + swz128(vr + 16, col >> 3) + (col & 7))),
                          pb, oacc[db]);
      }
    }
    if (hvalid) {
      float* ph = pb_ + hn * (HD + 2);
      if (grp == 0) {
        ph[0] = mx;
        ph[1] = ls;
      }
#pragma unroll
      for (int db = 0; db < 8; ++db)
        *(float4*)(ph + 2 + 16 * db + 4 * grp) = make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
    }
  }
}

// ---------------------------------------------------------------------------
// 4. merge the compression partials and the block partials, gated combine
__global__ void __launch_bounds__(1024) dsparse_merge_kernel(const float* __restrict__ part,
                                                            const float* __restrict__ part3,
                                                            const uint8_t* __restrict__ vid,
                                                            const float* __restrict__ gates, bf16* __restrict__ out,
                                                            bf16* __restrict__ o_cmp, bf16* __restrict__ o_slc,
                                                            bf16* __restrict__ o_swa, float* __restrict__ lse, Dims dm,
                                                            int nsplit, int nslot) {
  const int unit = blockIdx.x;
  const int64_t b = unit / dm.Hkv;
  const int g = unit % dm.Hkv;
  if (vid && !vid[b]) return;
  const int G = dm.G;
  extern __shared__ float s_w[];  // [nslot][2][G] weights exp2(m - M) / L of the block partials
  float* s_mx = s_w + nslot * 2 * G;
  float* s_fac = s_mx + nslot * 2 * G;  // [G][nsplit] weights of the compression partials
  __shared__ float s_M[16], s_L[16];
  const float* pc = part + (int64_t)unit * nsplit * G * PSTRIDE;
  const float* pu = part3 + (int64_t)unit * nslot * 2 * G * (HD + 2);
  dsplit_stats(pc, G, nsplit, s_fac, s_M, s_L);
  for (int i = threadIdx.x; i < nslot * 2 * G; i += blockDim.x) {
    const float* ph = pu + i * (HD + 2);
    s_w[i] = ph[1] > 0.f ? ph[1] : 0.f;  // sum for now
    s_mx[i] = ph[1] > 0.f ? ph[0] : -INFINITY;
  }
  __syncthreads();
  {  // one wave per (branch, head) pair
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (wv < 2 * G) {
      const int br = wv / G, hh = wv % G;
      float m = -INFINITY;
      for (int s = lane; s < nslot; s += 64) m = fmaxf(m, s_mx[(s * 2 + br) * G + hh]);
      const float M = wave_max(m);
      float l = 0.f;
      for (int s = lane; s < nslot; s += 64) {
        const int i = (s * 2 + br) * G + hh;
        if (s_mx[i] > -INFINITY) l += s_w[i] * fexp2(s_mx[i] - M);
      }
      const float L = wave_sum(l);
      for (int s = lane; s < nslot; s += 64) {
        const int i = (s * 2 + br) * G + hh;
        s_mx[i] = (s_mx[i] > -INFINITY && L > 0.f) ? fexp2(s_mx[i] - M) / L : 0.f;
      }
    }
  }
  __syncthreads();
  if (lse && threadIdx.x < G)
    lse[b * dm.Hq + g * G + threadIdx.x] =
        s_L[threadIdx.x] > 0.f ? (s_M[threadIdx.x] + flog2(s_L[threadIdx.x])) * LN2_F : -INFINITY;
  for (int i = threadIdx.x; i < G * HD; i += blockDim.x) {
    const int hh = i / HD, e = i % HD;
    float oc = 0.f;
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) oc += s_fac[hh * nsplit + s] * pc[(s * G + hh) * PSTRIDE + 2 + e];
    float ob[2];
    for (int br = 0; br < 2; ++br) {
      float o = 0.f;
#pragma unroll 5
      for (int s = 0; s < nslot; ++s) {
        const float f = s_mx[(s * 2 + br) * G + hh];
        const float val = pu[((s * 2 + br) * G + hh) * (HD + 2) + 2 + e];  // unwritten for empty partials
        o += (f != 0.f) ? f * val : 0.f;
      }
      ob[br] = o;
    }
    const int hq = g * G + hh;
    const int64_t off = (b * dm.Hq + hq) * (int64_t)HD + e;
    if (o_cmp) o_cmp[off] = (bf16)oc;
    if (o_slc) o_slc[off] = (bf16)ob[0];
    if (o_swa) o_swa[off] = (bf16)ob[1];
    if (out) {
      const float* gg = gates + (b * dm.Hq + hq) * 3;
      out[off] = (bf16)(gg[0] * oc + gg[1] * ob[0] + gg[2] * ob[1]);
    }
  }
}

// ---------------------------------------------------------------------------
static size_t drup(size_t x) { return (x + 255) & ~(size_t)255; }
static int dsplits(const Dims& dm) { return (int)((dm.Nc + DCH - 1) / DCH); }
static int dslots(const Dims& dm) { return dm.n + (dm.w + SB - 1) / SB + 1; }

bool decode_supported(const Dims& dm) { return dm.Tq == 1 && dm.Nc > 0; }

size_t decode_workspace(const Dims& dm) {
  const size_t units = (size_t)dm.B * dm.Hkv;
  return drup(units * dsplits(dm) * dm.G * PSTRIDE * 4) + drup(units * dslots(dm) * 2 * dm.G * (HD + 2) * 4);
}

// kh/vh: compressed cache (bf16), kl/vl: low parts or NULL.  Text rows are not handled here.
hipError_t launch_decode_fast(const Dims& dm, const void* q, const void* kh, const void* kl, const void* vh,
                              const void* vl, const void* k, const void* v, const uint8_t* vid, const float* gates,
                              void* out, void* o_cmp, void* o_slc, void* o_swa, int32_t* idx, float* lse,
                              float* imp, void* ws, hipStream_t s, void (*mark)(hipStream_t)) {
  const int units = (int)(dm.B * dm.Hkv);
  const int ns = dsplits(dm), nslot = dslots(dm);
  char* p = (char*)ws;
  float* part = (float*)p;
  p += drup((size_t)units * ns * dm.G * PSTRIDE * 4);
  float* part3 = (float*)p;
  if (kl)
    dcmp_split_kernel<true><<<dim3(units * ns), dim3(256), 0, s>>>((const bf16*)q, (const bf16*)kh, (const bf16*)kl,
                                                                   (const bf16*)vh, (const bf16*)vl, vid, part, dm, ns);
  else
    dcmp_split_kernel<false><<<dim3(units * ns), dim3(256), 0, s>>>((const bf16*)q, (const bf16*)kh, nullptr,
                                                                    (const bf16*)vh, nullptr, vid, part, dm, ns);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dcmp_merge_kernel<<<dim3(units), dim3(1024), (size_t)(dm.Ns + dm.G * ns) * 4, s>>>(part, vid, imp, idx, dm, ns);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (mark) mark(s);
  const int wgs = (nslot + 3) / 4;
  dsparse_blocks_kernel<<<dim3(units * wgs), dim3(256), 0, s>>>((const bf16*)q, (const bf16*)k, (const bf16*)v, idx,
                                                                vid, part3, dm, nslot);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t shm4 = (size_t)(nslot * 4 * dm.G + dm.G * ns) * 4;
  dsparse_merge_kernel<<<dim3(units), dim3(1024), shm4, s>>>(part, part3, vid, gates, (bf16*)out, (bf16*)o_cmp,
                                                             (bf16*)o_slc, (bf16*)o_swa, lse, dm, ns, nslot);
  return hipGetLastError();
}
