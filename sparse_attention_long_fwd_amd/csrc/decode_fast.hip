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
//  2. dsel: a few workgroups per (sequence, group).  Each merges the importance
//     partials (rescaled to the final normaliser, summed over the heads) and
//     picks the top-n blocks itself (wave 0) while its other waves already work
//     on the window blocks, which need no selection; then every wave takes one
//     chosen block below the window.  A block is scored once for both the
//     selection and the window branch; each workgroup leaves one partial per
//     (branch, head), and the first one the split weights of the compression
//     output.
//  3. dmerge: one thread per (head, channel) merges those partials and the
//     compression split partials and applies the gated combine.  Text rows
//     (dense causal attention, ungated): their split workgroups exit at once;
//     in dsel each wave runs an online softmax over a strided share of the
//     blocks.
#include "fast_common.hpp"
#include "topk_wave.hpp"

namespace {
constexpr int HD = 128;
constexpr int DCH = 128;           // compressed keys per split
constexpr int DBLK = DCH / 4;      // selection blocks per split (4 compressed keys per 64-token block)
constexpr int PSTRIDE = 2 + HD + DBLK + 1;  // per head: max, sum, O[128], E[32] + carry
constexpr int SB = 64;
static_assert(kPageRows == SB, "a page holds one selection block");
}  // namespace

__device__ __forceinline__ void dwait() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

// Tokens in sequence b (clamped to [1, capacity]).
__device__ __forceinline__ int64_t dv_len(const DecVar& dv, const Dims& dm, int64_t b) {
  if (!dv.lens) return dm.T;
  const int64_t n = dv.lens[b];
  return n < 1 ? 1 : (n > dm.T ? dm.T : n);
}
// Row u (of KV head g) of sequence b in a K or V cache, contiguous [B, T, Hkv, D] or paged
// [num_pages, 64, Hkv, D] (page ids clamped into the pool).
__device__ __forceinline__ const bf16* dv_row(const DecVar& dv, const Dims& dm, const bf16* base, int64_t b, int g,
                                              int64_t u) {
  if (dv.pages) {
    int64_t pg = dv.pages[b * dv.max_pages + u / kPageRows];
    pg = pg < 0 ? 0 : (pg >= dv.num_pages ? dv.num_pages - 1 : pg);
    return base + ((pg * kPageRows + u % kPageRows) * dm.Hkv + g) * (int64_t)HD;
  }
  return base + ((b * dm.T + u) * dm.Hkv + g) * (int64_t)HD;
}

// ---------------------------------------------------------------------------
// 1. compression-branch partials
template <bool SPLIT>
__global__ void __launch_bounds__(256) dcmp_split_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kh,
                                                         const bf16* __restrict__ kl, const bf16* __restrict__ vh,
                                                         const bf16* __restrict__ vl, const uint8_t* __restrict__ vid,
                                                         float* __restrict__ part, Dims dm,
                                                         int nsplit) {
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

// Compression-branch partials from a bf16 cache, streamed: each wave owns one split of DCH keys
// (the partial record above) and walks it in 4 steps of 32 keys; the K and V loads of step
// i + 1 are in flight (into registers) while step i computes, with an online softmax over the
// steps.  V goes through the wave's own LDS tile for the transposed reads; the waves of a
// workgroup never synchronise.  When Hkv divides 4, the 4 waves of a workgroup take the same
// split of all KV heads of a sequence (4 / Hkv splits), so together they read whole token rows
// of the cache ([Nc, Hkv, D]: Hkv x 256 contiguous bytes a key) at the same time; otherwise
// the 4 waves take 4 splits of one (sequence, KV head).  Workgroup 0 zeroes the completion
// counters of dsel_kernel.
__global__ void __launch_bounds__(256) dcmp_pipe_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kh,
                                                        const bf16* __restrict__ vh, const uint8_t* __restrict__ vid,
                                                        float* __restrict__ part, Dims dm,
                                                        DecVar dv, int nsplit) {
  constexpr int NSTEP = DCH / 32;
  __shared__ __attribute__((aligned(16))) bf16 s_v[4][32 * HD];
  __shared__ float s_ea[4][16][DBLK + 1], s_ec[4][16][DBLK + 1];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, hn = l & 15, grp = l >> 4;
  int64_t b;
  int g, s;
  if (4 % dm.Hkv == 0) {
    const int spw = 4 / dm.Hkv;                   // splits per workgroup
    const int wps = (nsplit + spw - 1) / spw;      // workgroups per sequence
    b = blockIdx.x / wps;
    g = w % dm.Hkv;
    s = (blockIdx.x % wps) * spw + w / dm.Hkv;
  } else {
    const int wpu = (nsplit + 3) / 4;  // workgroups per unit
    b = (blockIdx.x / wpu) / dm.Hkv;
    g = (blockIdx.x / wpu) % dm.Hkv;
    s = (blockIdx.x % wpu) * 4 + w;
  }
  const int unit = (int)(b * dm.Hkv + g);
  if ((vid && !vid[b]) || s >= nsplit) return;
  const int G = dm.G;
  // compressed blocks of this sequence seen by its query (every block of a full cache)
  const int64_t nv = cmp_visible(dv.lens ? dv_len(dv, dm, b) - 1 : dm.q0, dm.l, dm.d, dm.Nc);
  if ((int64_t)s * DCH >= nv) {  // a split past the sequence's blocks: an empty partial
    float* ph = part + ((int64_t)unit * nsplit + s) * G * PSTRIDE;
    for (int i = l; i < G * PSTRIDE; i += 64) ph[i] = (i % PSTRIDE) == 0 ? -INFINITY : 0.f;
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
  const int64_t base = (b * dm.Nc * dm.Hkv + g) * (int64_t)HD;
  const int64_t kbeg = (int64_t)s * DCH;
  // step j: K fragments (rows kbeg + 32j + 16kb + hn, dims 32ks + 8grp) and V rows in the order
  // of the wave's swizzled LDS tile (16-byte chunk ins*64 + l holds row p >> 4, chunk
  // (p & 15) ^ (row & 15), p = ins*64 + l); rows past the cache repeat its last row (masked)
  auto load_step = [&](int j, bf16x8* kf, bf16x8* vf) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      int64_t key = kbeg + 32 * j + 16 * kb + hn;
      if (key >= nv) key = nv - 1;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[4 * kb + ks] = *(const bf16x8*)(kh + base + key * stride + 32 * ks + 8 * grp);
    }
#pragma unroll
    for (int ins = 0; ins < 8; ++ins) {
      const int p = ins * 64 + l, row = p >> 4, c = (p & 15) ^ (row & 15);
      int64_t key = kbeg + 32 * j + row;
      if (key >= nv) key = nv - 1;
      vf[ins] = *(const bf16x8*)(vh + base + key * stride + c * 8);
    }
  };
  bf16x8 kfa[8], vfa[8], kfb[8], vfb[8];
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{};
  float ea[NSTEP][2], ec[NSTEP][2], mus[NSTEP];
  bool live[NSTEP];
  bf16* vt = s_v[w];
  const int vr = 4 * grp + (hn >> 2);
  load_step(0, kfa, vfa);
#pragma unroll
  for (int j = 0; j < NSTEP; ++j) {
    bf16x8* kf = (j & 1) ? kfb : kfa;
    bf16x8* vf = (j & 1) ? vfb : vfa;
    if (j + 1 < NSTEP) load_step(j + 1, (j & 1) ? kfa : kfb, (j & 1) ? vfa : vfb);
    f32x4 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc[kb] = mfma16(kf[4 * kb + ks], qf[ks], sc[kb]);
    }
    float x[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int64_t key = kbeg + 32 * j + 16 * kb + 4 * grp + jj;
        x[4 * kb + jj] = key < nv ? sc[kb][jj] * c2 : -INFINITY;
      }
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m_run, mx);
    live[j] = mnew > -INFINITY;
    const float mu = live[j] ? mnew : 0.f;  // nothing visible yet: every term below is 0
    mus[j] = mu;
    float p[8], ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fexp2(x[e] - mu);
      ls += p[e];
    }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    const float fac = fexp2(m_run - mu);  // 0 while m_run is -inf
    l_run = l_run * fac + ls;
    m_run = mnew;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[db][e] *= fac;
    // importance pieces: this lane's 4 keys of sub-block kb are one selection block
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      ea[j][kb] = p[4 * kb] + p[4 * kb + 1] + p[4 * kb + 2] + 0.5f * p[4 * kb + 3];
      ec[j][kb] = 0.5f * p[4 * kb + 3];
    }
    // V rows of this step into the wave's tile, then O^T += V^T P^T (LDS is in order per wave)
#pragma unroll
    for (int ins = 0; ins < 8; ++ins) *(bf16x8*)(vt + (ins * 64 + l) * 8) = vf[ins];
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pb[e] = (bf16)p[e];
      pb[4 + e] = (bf16)p[4 + e];
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int col = 16 * db + 4 * (hn & 3);
      oacc[db] = mfma16(cat(lds_read_tr(vt + swz128(vr, col >> 3) + (col & 7)),
                            lds_read_tr(vt + swz128(vr + 16, col >> 3) + (col & 7))),
                        pb, oacc[db]);
    }
  }
  // the split's partial: per head max, sum, O and the importance of its DBLK blocks + carry,
  // every piece rescaled to the final maximum
  const float M = m_run;
#pragma unroll
  for (int j = 0; j < NSTEP; ++j) {
    const float f = live[j] ? fexp2(mus[j] - M) : 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int jb = 8 * j + 4 * kb + grp;
      s_ea[w][hn][jb] = ea[j][kb] * f;
      s_ec[w][hn][jb + 1] = ec[j][kb] * f;
    }
  }
  if (grp == 0) s_ec[w][hn][0] = 0.f;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float* pp = part + ((int64_t)unit * nsplit + s) * G * PSTRIDE;
  if (hvalid) {
    float* ph = pp + hn * PSTRIDE;
    if (grp == 0) {
      ph[0] = M;
      ph[1] = l_run;
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) ph[2 + 16 * db + 4 * grp + e] = oacc[db][e];
    for (int jb = grp; jb <= DBLK; jb += 4)
      ph[2 + HD + jb] = (jb < DBLK ? s_ea[w][hn][jb] : 0.f) + s_ec[w][hn][jb];
  }
}

// ---------------------------------------------------------------------------
// 2. selection, window and the final merge

// Per-head softmax statistics of the split partials, 32 lanes per head (heads threadIdx.x / 32,
// so one load round for up to blockDim.x / 32 heads and 32 splits; more loop):
// s_fac[h][s] = exp2(m_s - M_h) / L_h (0 for empty splits), s_M[h], s_L[h].
__device__ __forceinline__ void dsplit_stats(const float* pu, int G, int nsplit, float* s_fac, float* s_M,
                                             float* s_L) {
  const int sl = threadIdx.x & 31, nh = blockDim.x >> 5;
  for (int hh = threadIdx.x >> 5; hh < G; hh += nh) {
    float m0 = -INFINITY, l0 = 0.f;
    if (sl < nsplit) {
      m0 = pu[(sl * G + hh) * PSTRIDE];
      l0 = pu[(sl * G + hh) * PSTRIDE + 1];
    }
    float m = m0;
    for (int s = sl + 32; s < nsplit; s += 32) m = fmaxf(m, pu[(s * G + hh) * PSTRIDE]);
    float M = m;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float l = m0 > -INFINITY ? l0 * fexp2(m0 - M) : 0.f;
    for (int s = sl + 32; s < nsplit; s += 32) {
      const float ms = pu[(s * G + hh) * PSTRIDE];
      if (ms > -INFINITY) l += pu[(s * G + hh) * PSTRIDE + 1] * fexp2(ms - M);
    }
    float L = l;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
    if (sl < nsplit) s_fac[hh * nsplit + sl] = (m0 > -INFINITY && L > 0.f) ? fexp2(m0 - M) / L : 0.f;
    for (int s = sl + 32; s < nsplit; s += 32) {
      const float ms = pu[(s * G + hh) * PSTRIDE];
      s_fac[hh * nsplit + s] = (ms > -INFINITY && L > 0.f) ? fexp2(ms - M) / L : 0.f;
    }
    if (sl == 0) {
      s_M[hh] = M;
      s_L[hh] = L;
    }
  }
}

// One workgroup per (unit, share): wgs workgroups per (sequence, KV group) with 4 waves each.
// Every workgroup of a unit first merges the importance partials of the compression split and
// picks the unit's blocks (the same deterministic result in each; wave 0 selects).  Meanwhile
// waves 1-3 take the window blocks, which need no selection: window block wb0 + sg*3 + w-1
// (scores once, a window partial, and after the selection a selection partial if the block
// was chosen).  Then wave w takes chosen block sg*4 + w of those below the window.  A wave's
// blocks accumulate online into one selection and one window partial (max, sum, O), which the
// workgroup merges in LDS and writes as one partial per (branch, head); workgroup 0 of the unit
// also writes the split weights of the compression partials (facw).  dmerge_kernel combines them.
// Text rows: dense causal attention, every wave an online softmax over blocks sg*4+w, +4*wgs, ...
__global__ void __launch_bounds__(256) dsel_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                   const bf16* __restrict__ v, const float* __restrict__ part,
                                                   const uint8_t* __restrict__ vid, float* __restrict__ lse,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ imp_out, float* __restrict__ part3,
                                                   float* __restrict__ facw, Dims dm,
                                                   DecVar dv, int nsplit, int wgs) {
  extern __shared__ float dsm[];
  const int G = dm.G;
  float* s_imp = dsm;                   // [Ns] importance of the unit's blocks
  float* s_fac = s_imp + dm.Ns;         // [G][nsplit] weights of the compression partials
  __shared__ __attribute__((aligned(16))) bf16 vt[4][SB * HD];
  __shared__ float s_M[16], s_L[16];
  __shared__ int32_t s_idx[32];
  __shared__ TopkScratch s_tk;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hn = l & 15, grp = l >> 4;
  const int unit = blockIdx.x / wgs, sg = blockIdx.x % wgs;
  const int64_t b = unit / dm.Hkv;
  const int g = unit % dm.Hkv;
  const bool text = vid && !vid[b];  // the same for the whole workgroup
  const int64_t len = dv_len(dv, dm, b);  // tokens of this sequence; the query sits at len - 1
  const int64_t t = dv.lens ? len - 1 : dm.q0, jt = t / SB;
  int64_t wlo = t - dm.w + 1;
  if (wlo < 0) wlo = 0;
  const int64_t wb0 = wlo / SB;
  const float* pc = part + (int64_t)unit * nsplit * G * PSTRIDE;
  constexpr int PO = 4;        // O offset within a partial (16-byte aligned rows)
  constexpr int PW = HD + PO;  // partial of one (branch, head): max, sum, -, -, O[128]
  const bool hvalid = hn < G;
  const float c2 = dm.scale * LOG2E_F;

  // ---- per-wave state: one selection (0) and one window (1) partial, online over its blocks
  float pm[2] = {-INFINITY, -INFINITY}, pl[2] = {0.f, 0.f};
  f32x4 po[2][8];
#pragma unroll
  for (int br = 0; br < 2; ++br)
#pragma unroll
    for (int db = 0; db < 8; ++db) po[br][db] = f32x4{};
  bf16x8 qf[4];
  {
    const int h = g * G + (hvalid ? hn : 0);
    const bf16* qrow = q + (b * dm.Hq + h) * (int64_t)HD + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = hvalid ? *(const bf16x8*)(qrow + 32 * ks) : zero8();
  }
  const int64_t stride = (int64_t)dm.Hkv * HD;
  // block j's rows: 64 consecutive rows of stride Hkv*D from its first row (contiguous cache) or
  // from its page (paged cache); rows past the sequence repeat its last row (masked)
  auto krow0 = [&](int64_t j) { return dv_row(dv, dm, k, b, g, j * SB); };
  auto vrow0 = [&](int64_t j) { return dv_row(dv, dm, v, b, g, j * SB); };
  auto rows_in = [&](int64_t j) { return len - j * SB < SB ? len - j * SB : (int64_t)SB; };
  // block j: stage V into the wave's tile, scores S^T (keys on M, heads on N), per lane
  auto block_scores = [&](int64_t j, f32x4* sc) {
    const int64_t nr = rows_in(j);
    stage_tile64(vt[w], vrow0(j), stride, 0, nr, 0, 1, l);
    const bf16* kb0 = krow0(j);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      int64_t r = 16 * kb + hn;
      if (r >= nr) r = nr - 1;
      const bf16* kr = kb0 + r * stride + 8 * grp;
      sc[kb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc[kb] = mfma16(*(const bf16x8*)(kr + 32 * ks), qf[ks], sc[kb]);
    }
    dwait();
    __builtin_amdgcn_wave_barrier();
  };
  // masked scores of block j for branch br (0: u <= t; 1: also u >= wlo), log2 units
  auto masked = [&](int64_t j, const f32x4* sc, int br, float* x) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int64_t u = j * SB + 16 * kb + 4 * grp + jj;
        const bool ok = br == 0 ? (u <= t) : (u <= t && u >= wlo);
        x[4 * kb + jj] = ok ? sc[kb][jj] * c2 : -INFINITY;
      }
  };
  // online update of partial br with masked scores x of the block whose V tile is staged
  auto accumulate = [&](int br, const float* x) {
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(pm[br], mx);
    if (mnew == -INFINITY) return;
    const float sc_old = pm[br] > -INFINITY ? fexp2(pm[br] - mnew) : 0.f;
    float p[16], ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = fexp2(x[e] - mnew);
      ls += p[e];
    }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
#pragma unroll
    for (int db = 0; db < 8; ++db) po[br][db] *= sc_old;
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
        po[br][db] = mfma16(cat(lds_read_tr(vt[w] + swz128(vr, col >> 3) + (col & 7)),
                                lds_read_tr(vt[w] + swz128(vr + 16, col >> 3) + (col & 7))),
                            pb, po[br][db]);
      }
    }
    pl[br] = pl[br] * sc_old + ls;
    pm[br] = mnew;
  };

  if (!text) {
    // ---- importance of blocks 0 .. jt (heads summed in a fixed order)
    dsplit_stats(pc, G, nsplit, s_fac, s_M, s_L);
    __syncthreads();
    if (sg == 0 && lse && tid < G)
      lse[b * dm.Hq + g * G + tid] = s_L[tid] > 0.f ? (s_M[tid] + flog2(s_L[tid])) * LN2_F : -INFINITY;
    // the split weights, for the merge kernel's compression output
    if (sg == 0)
      for (int i = tid; i < G * nsplit; i += blockDim.x) facw[(int64_t)unit * G * nsplit + i] = s_fac[i];
    // 4 blocks a thread per pass; loads clamped to valid addresses and unconditional, so a
    // pass has all of them in flight at once (invalid terms get weight 0)
    for (int j0 = 0; j0 <= jt; j0 += 4 * blockDim.x) {
      float a[4][8], c[4][8], fa[4][8], fc[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * blockDim.x + tid;
        const int s = j / DBLK, jb = j % DBLK;
        const int sa = s < nsplit ? s : nsplit - 1, scar = s > 0 ? s - 1 : 0;
        const bool va = j <= jt && s < nsplit, vc = j <= jt && jb == 0 && s > 0;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
          const int hc = hh < G ? hh : G - 1;
          a[u][hh] = pc[(sa * G + hc) * PSTRIDE + 2 + HD + jb];
          c[u][hh] = pc[(scar * G + hc) * PSTRIDE + 2 + HD + DBLK];
          fa[u][hh] = (va && hh < G) ? s_fac[hc * nsplit + sa] : 0.f;
          fc[u][hh] = (vc && hh < G) ? s_fac[hc * nsplit + scar] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * blockDim.x + tid;
        float val = 0.f;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
          val += fa[u][hh] * a[u][hh];
          val += fc[u][hh] * c[u][hh];
        }
        if (j > jt) continue;
        s_imp[j] = val;
        if (imp_out && sg == 0) imp_out[(b * dm.Hkv + g) * dm.Ns + j] = val;
      }
    }
    __syncthreads();
    // ---- wave 0 selects; waves 1-3 meanwhile score their window block
    const int wslot = sg * 3 + w - 1;
    const int64_t jw = wb0 + wslot;
    const bool has_win = w > 0 && jw <= jt;
    f32x4 scw[4];
    if (w == 0) {
      int lo, hi, nj;
      const int kk = tk_bounds(t, dm.ls, dm.Ns, dm.n, dm.n_init, dm.n_local, &lo, &hi, &nj);
      wave_select(s_imp, lo, hi, nj, kk, dm.n, &s_tk, s_idx, l);
      if (sg == 0 && l < dm.n) idx[(b * dm.Hkv + g) * dm.n + l] = s_idx[l];
    } else {
      if (has_win) {
        float x[16];
        block_scores(jw, scw);
        masked(jw, scw, 1, x);
        accumulate(1, x);
      }
    }
    __syncthreads();
    if (has_win) {  // the window block also counts for the selection branch if it was chosen
      bool chosen = false;
      for (int c = 0; c < dm.n; ++c) chosen |= s_idx[c] == jw;
      if (chosen) {
        float x[16];
        masked(jw, scw, 0, x);
        accumulate(0, x);
      }
    }
    // ---- chosen block sg*4 + w among those below the window
    {
      const int want = sg * 4 + w;
      int64_t js = -1;
      int cnt_lt = 0;
      for (int c = 0; c < dm.n; ++c)
        if (s_idx[c] >= 0 && s_idx[c] < wb0) {
          if (cnt_lt == want) js = s_idx[c];
          ++cnt_lt;
        }
      if (js >= 0) {
        tk_wave_sync();  // done reading the window block's tile
        f32x4 sc[4];
        float x[16];
        block_scores(js, sc);
        masked(js, sc, 0, x);
        accumulate(0, x);
      }
    }
  } else {
    for (int64_t j = sg * 4 + w; j <= jt; j += 4 * wgs) {
      f32x4 sc[4];
      float x[16];
      block_scores(j, sc);
      masked(j, sc, 0, x);
      accumulate(0, x);
      tk_wave_sync();  // the tile is read before the next block overwrites it
    }
  }

  // ---- the wave's partials into LDS over its V tile, merged per workgroup
  float* wp = (float*)vt[w];  // [2][G][PW]
  tk_wave_sync();
  if (hvalid) {
#pragma unroll
    for (int br = 0; br < 2; ++br) {
      float* ph = wp + (br * G + hn) * PW;
      if (grp == 0) {
        ph[0] = pm[br];
        ph[1] = pl[br];
      }
      if (pl[br] > 0.f) {
#pragma unroll
        for (int db = 0; db < 8; ++db)
          *(float4*)(ph + PO + 16 * db + 4 * grp) = make_float4(po[br][db][0], po[br][db][1], po[br][db][2],
                                                                po[br][db][3]);
      }
    }
  }
  __syncthreads();
  float* pw = part3 + ((int64_t)unit * wgs + sg) * 2 * G * PW;
  for (int i = tid; i < 2 * G * HD / 4; i += blockDim.x) {
    const int bh = (4 * i) / HD, e = (4 * i) % HD;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float* ph = (const float*)vt[ww] + bh * PW;
      if (ph[1] > 0.f) M = fmaxf(M, ph[0]);
    }
    float L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float* ph = (const float*)vt[ww] + bh * PW;
      if (ph[1] > 0.f) {
        const float f = fexp2(ph[0] - M);
        const float4 x = *(const float4*)(ph + PO + e);
        L += f * ph[1];
        O.x += f * x.x;
        O.y += f * x.y;
        O.z += f * x.z;
        O.w += f * x.w;
      }
    }
    *(float4*)(pw + bh * PW + PO + e) = O;
    if (e == 0) {
      pw[bh * PW] = M;
      pw[bh * PW + 1] = L;
    }
  }

  // the workgroup partials are merged by dmerge_kernel (the kernel boundary orders the stores)
}


// ---------------------------------------------------------------------------
// One thread per (head, channel) of a (sequence, KV group), mq workgroups per (sequence, group):
// merges per head the selection kernel's workgroup partials of the selection and window branches
// (text rows: the dense partials) and, for video rows, the compression split partials with the
// weights the selection kernel derived (2^(m_s - M) / L per split, summed over the splits in
// order), then writes the outputs, gated for video rows.  Every load of a thread is independent of
// the others (partials of empty entries are read and then given weight 0), so they go out
// together.
__global__ void __launch_bounds__(256) dmerge_kernel(const float* __restrict__ part3, const float* __restrict__ part,
                                                     const float* __restrict__ facw,
                                                     const uint8_t* __restrict__ vid, const float* __restrict__ gates,
                                                     bf16* __restrict__ out, bf16* __restrict__ o_cmp,
                                                     bf16* __restrict__ o_slc, bf16* __restrict__ o_swa, Dims dm,
                                                     int wgs, int nsplit, int mq) {
  constexpr int PO = 4;        // O offset within a partial (16-byte aligned rows)
  constexpr int PW = HD + PO;  // partial of one (branch, head): max, sum, -, -, O[128]
  const int G = dm.G;
  const int unit = blockIdx.x / mq;
  const int i = (blockIdx.x % mq) * blockDim.x + threadIdx.x;
  if (i >= G * HD) return;
  const int hh = i / HD, e = i % HD;
  const int64_t b = unit / dm.Hkv;
  const int g = unit % dm.Hkv;
  const bool text = vid && !vid[b];
  const float* pu = part3 + (int64_t)unit * wgs * 2 * G * PW;
  float ob[2];
#pragma unroll
  for (int br = 0; br < 2; ++br) {
    // online over the workgroup partials: (max, sum, O) rescaled as the maximum grows
    float M = -INFINITY, L = 0.f, o = 0.f;
#pragma unroll 4
    for (int s = 0; s < wgs; ++s) {
      const float* ph = pu + (s * 2 * G + br * G + hh) * PW;
      const float m1 = ph[0], l1 = ph[1], x = ph[PO + e];
      const bool live = l1 > 0.f;  // the O of empty partials is never written: selected away
      const float Mn = live ? fmaxf(M, m1) : M;
      const float a = M > -INFINITY ? fexp2(M - Mn) : 0.f;
      const float c = live ? fexp2(m1 - Mn) : 0.f;
      L = L * a + l1 * c;
      o = o * a + (live ? x * c : 0.f);
      M = Mn;
    }
    ob[br] = L > 0.f ? o / L : 0.f;
  }
  const int hq = g * G + hh;
  const int64_t off = (b * dm.Hq + hq) * (int64_t)HD + e;
  if (text) {  // dense attention, ungated
    if (out) out[off] = (bf16)ob[0];
    return;
  }
  const float* pc = part + (int64_t)unit * nsplit * G * PSTRIDE + hh * PSTRIDE + 2 + e;
  const float* fu = facw + ((int64_t)unit * G + hh) * nsplit;
  float oc = 0.f;
#pragma unroll 16
  for (int s = 0; s < nsplit; ++s) oc += fu[s] * pc[(int64_t)s * G * PSTRIDE];
  const float* gg = gates + (b * dm.Hq + hq) * 3;
  if (o_cmp) o_cmp[off] = (bf16)oc;
  if (o_slc) o_slc[off] = (bf16)ob[0];
  if (o_swa) o_swa[off] = (bf16)ob[1];
  if (out) out[off] = (bf16)(gg[0] * oc + gg[1] * ob[0] + gg[2] * ob[1]);
}

// ---------------------------------------------------------------------------
static unsigned dcmp_pipe_grid(const Dims& dm, int ns) {
  if (4 % dm.Hkv == 0) {
    const int spw = 4 / (int)dm.Hkv;
    return (unsigned)(dm.B * ((ns + spw - 1) / spw));
  }
  return (unsigned)(dm.B * dm.Hkv * ((ns + 3) / 4));
}
static size_t drup(size_t x) { return (x + 255) & ~(size_t)255; }
static int dsplits(const Dims& dm) { return (int)((dm.Nc + DCH - 1) / DCH); }
// workgroups per (sequence, group): window blocks 3 a workgroup, chosen blocks below the window 4
static int dwgs(const Dims& dm) {
  const int nwin = (dm.w + SB - 1) / SB + 1, a = (nwin + 2) / 3, c = (dm.n + 3) / 4;
  return a > c ? a : c;
}

// The selection kernel keeps the importance of all Ns blocks in LDS.
bool decode_supported(const Dims& dm) { return dm.Tq == 1 && dm.Nc > 0 && dm.Ns <= 16384 && dm.ls == 64; }

size_t decode_workspace(const Dims& dm) {
  const size_t units = (size_t)dm.B * dm.Hkv;
  const size_t wgs = dwgs(dm);
  return drup(units * dsplits(dm) * dm.G * PSTRIDE * 4) + drup(units * wgs * 2 * dm.G * (HD + 4) * 4) +
         drup(units * dm.G * dsplits(dm) * 4);
}

// kh/vh: compressed cache (bf16), kl/vl: low parts or NULL.  Text rows take dense causal
// attention in the selection kernel (their compression split is skipped).
hipError_t launch_decode_fast(const Dims& dm, const DecVar& dv, const void* q, const void* kh, const void* kl,
                              const void* vh, const void* vl, const void* k, const void* v, const uint8_t* vid,
                              const float* gates, void* out, void* o_cmp, void* o_slc, void* o_swa, int32_t* idx,
                              float* lse, float* imp, void* ws, hipStream_t s, void (*mark)(hipStream_t)) {
  if (kl && (dv.lens || dv.pages)) return hipErrorInvalidValue;  // split parts: full contiguous caches only
  const int units = (int)(dm.B * dm.Hkv);
  const int ns = dsplits(dm);
  char* p = (char*)ws;
  float* part = (float*)p;
  p += drup((size_t)units * ns * dm.G * PSTRIDE * 4);
  const int wgs = dwgs(dm);
  float* part3 = (float*)p;
  p += drup((size_t)units * wgs * 2 * dm.G * (HD + 4) * 4);
  float* facw = (float*)p;
  if (kl)
    dcmp_split_kernel<true><<<dim3(units * ns), dim3(256), 0, s>>>((const bf16*)q, (const bf16*)kh, (const bf16*)kl,
                                                                   (const bf16*)vh, (const bf16*)vl, vid, part,
                                                                   dm, ns);
  else
    dcmp_pipe_kernel<<<dim3(dcmp_pipe_grid(dm, ns)), dim3(256), 0, s>>>((const bf16*)q, (const bf16*)kh,
                                                                        (const bf16*)vh, vid, part, dm, dv, ns);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (mark) mark(s);
  const size_t shm = (size_t)(dm.Ns + dm.G * ns) * 4;
  e = hipFuncSetAttribute((const void*)dsel_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  dsel_kernel<<<dim3(units * wgs), dim3(256), shm, s>>>(
      (const bf16*)q, (const bf16*)k, (const bf16*)v, part, vid, lse, idx, imp, part3, facw, dm, dv, ns, wgs);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int mq = (int)((dm.G * HD + 255) / 256);
  dmerge_kernel<<<dim3(units * mq), dim3(256), 0, s>>>(part3, part, facw, vid, gates, (bf16*)out, (bf16*)o_cmp,
                                                        (bf16*)o_slc, (bf16*)o_swa, dm, wgs, ns, mq);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 3. compressed-cache update for a decode stream
// Compressed block i covers tokens [i d, i d + l) and is complete once token i d + l - 1 is in
// the cache.  After n_new tokens were appended to every sequence, the blocks whose last token
// is among them are computed from the sequence's K / V rows (contiguous or paged), with the same
// weights, order of summation and rounding as the full compression.  One thread per 8 channels
// of one (sequence, new-block slot, KV head).
__global__ void __launch_bounds__(256) compress_append_kernel(const bf16* __restrict__ k, const bf16* __restrict__ v,
                                                              const float* __restrict__ w_k,
                                                              const float* __restrict__ w_v, bf16* __restrict__ kc,
                                                              bf16* __restrict__ vc, Dims dm, DecVar dv, int n_new,
                                                              int slots) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int c8 = (int)(gid % (HD / 8));
  int64_t rest = gid / (HD / 8);
  const int h = (int)(rest % dm.Hkv);
  rest /= dm.Hkv;
  const int slot = (int)(rest % slots);
  const int64_t b = rest / slots;
  if (b >= dm.B) return;
  const int64_t len = dv_len(dv, dm, b);
  if (len < dm.l) return;
  const int64_t hi = (len - dm.l) / dm.d;  // last complete block
  const int64_t lo_num = len - n_new - dm.l + 1;
  const int64_t i = (lo_num <= 0 ? 0 : (lo_num + dm.d - 1) / dm.d) + slot;
  if (i > hi || i >= dm.Nc) return;
  float ak[8] = {0, 0, 0, 0, 0, 0, 0, 0}, av[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int m = 0; m < dm.l; ++m) {
    const int64_t u = i * dm.d + m;
    const bf16x8 xk = *(const bf16x8*)(dv_row(dv, dm, k, b, h, u) + c8 * 8);
    const bf16x8 xv = *(const bf16x8*)(dv_row(dv, dm, v, b, h, u) + c8 * 8);
    const float wk = w_k[m], wv = w_v[m];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ak[e] = fmaf(wk, (float)xk[e], ak[e]);
      av[e] = fmaf(wv, (float)xv[e], av[e]);
    }
  }
  bf16x8 ok, ov;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ok[e] = (bf16)ak[e];
    ov[e] = (bf16)av[e];
  }
  const int64_t o = ((b * dm.Nc + i) * dm.Hkv + h) * (int64_t)HD + c8 * 8;
  *(bf16x8*)(kc + o) = ok;
  *(bf16x8*)(vc + o) = ov;
}

hipError_t launch_compress_append(const Dims& dm, const DecVar& dv, const void* k, const void* v, const float* w_k,
                                  const float* w_v, void* kc, void* vc, int n_new, hipStream_t s) {
  if (dm.B <= 0 || dm.Nc <= 0 || n_new <= 0) return hipSuccess;
  if (dm.D != HD) return hipErrorInvalidValue;
  const int slots = (n_new + dm.d - 1) / dm.d + 1;
  const int64_t total = dm.B * slots * dm.Hkv * (HD / 8);
  compress_append_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s>>>(
      (const bf16*)k, (const bf16*)v, w_k, w_v, (bf16*)kc, (bf16*)vc, dm, dv, n_new, slots);
  return hipGetLastError();
}
