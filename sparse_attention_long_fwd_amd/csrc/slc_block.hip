// Selection branch of the video rows, block-major, and the gated combine (gfx950).
//
// What it computes (top168.com digest of VideoNSA, section 一; csdn page
// "VideoNSA：重新定义视频理解的稀疏注意力机制", section 2.2): for a video row t and
// KV group g, the heads of g attend over the tokens u <= t of the blocks chosen
// for (t, g); the output of the layer is g_cmp o_cmp + g_slc o_slc + g_swa o_swa
// per head (section 3.1 of the csdn page: three gate values per head).
//
// The chosen blocks of different rows barely overlap (beyond the forced ones),
// so a row-major kernel gathers 16 whole blocks (32 KB of K and V) per (row,
// group).  Here the work is turned around: each chosen block is loaded once
// per chunk of 32 rows that chose it, and each (row, slot, head) leaves a
// partial softmax (max and sum in one array, the unnormalised value sum in fp16
// in another, 256-byte aligned) that a merge kernel combines.  Per (row, slot) pair that moves the row's query (1.8 KB for
// 7 heads) and the partial (1.8 KB) instead of 32 KB of keys and values.
//
//  1. slc_count: per (batch, group, 2048-row range) an LDS histogram of the
//     chosen blocks, added to the global per-block counts.
//  2. slc_scan: per (batch, group) the first chunk of each block's pair list
//     (lists are padded to whole chunks of 32 pairs, -1 filled, so a chunk's
//     pairs sit at chunk * 32); the chunk -> block map the attention grid uses.
//  3. slc_scatter: the same histogram again, one global reservation per
//     (workgroup, block), then each pair (row, slot) lands in its block's list.
//  4. slc_chunk: per chunk, the block's K / V staged in LDS (swizzled rows), a
//     wave per head: S^T = K Q^T (32x32x16 MFMA, the 32 rows on N), the causal
//     mask on the row's own block, a local softmax, O^T = V^T P^T with
//     transposing LDS reads; the partial goes to (row, group, slot, head).
//  5. slc_merge: a wave per (row, group) merges the slots' partials per head
//     and writes o_slc and the gated output.
// The order of a block's pair list depends on atomics, but every partial has a
// fixed home and the merge runs over the slots in order: results are
// deterministic.
#include "fast_common.hpp"

namespace {
constexpr int HD = 128;
constexpr int RC = 32;       // rows per chunk
constexpr int RROWS = 512;   // rows per bucketing workgroup
}  // namespace

// Bucketing layout in the workspace (per bg = b * Hkv + g):
//  count[bg][Ns], off[bg][Ns] (pair list of block j starts at pairs + bg*cap_c*RC + off,
//  off = 32 * its first chunk), cfirst[bg][Ns] (first chunk of block j), cursor[bg][Ns],
//  chunk_blk[bg][cap_c], pairs[bg][cap_c * RC] = (row << 5) | slot, or -1 past a list's end.
// Partials: ml[(b*Tq + row)*Hkv + g][slot][head] = (max in log2 units, sum) and
// po[same index][128] fp16 (one 256-byte record).
struct SlcBuckets {
  int* count;
  int* off;
  int* cfirst;
  int* cursor;
  int* chunk_blk;
  int* pairs;
  int cap_c;
};

static inline int slc_cap_chunks(const Dims& dm) { return (int)((dm.Tq * dm.n + RC - 1) / RC + dm.Ns); }

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) slc_zero_kernel(int* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// A pair (row, slot) takes part when its block holds a key at or before the row (blocks after
// the row's own block jt, which a caller's set may list, contribute no key, and every such id
// would index past the block tables), and it is left to the window pass when that pass forms the
// row's forced local blocks (local_fused): blocks jt - n_local + 1 .. jt.
__device__ __forceinline__ bool slc_pair_kept(int j, int64_t r, const Dims& dm, int local_fused) {
  const int64_t jt = (dm.q0 + r) / dm.ls;  // < Ns for every row of the sequence
  return j >= 0 && (int64_t)j <= jt && !(local_fused && (int64_t)j > jt - dm.n_local);
}

// Calls f(r, s, j) for each kept pair (row r, slot s, block j) of group g among rows [r0, r1): one
// entry (r, s) per thread and step, consecutive threads on consecutive entries (coalesced), eight
// steps' loads issued before their uses so that the loop is not one load latency per entry.
template <typename F>
__device__ __forceinline__ void slc_for_pairs(const int32_t* __restrict__ idx, const uint8_t* __restrict__ vid,
                                              const Dims& dm, int64_t b, int g, int64_t r0, int64_t r1,
                                              int local_fused, F f) {
  constexpr int U = 8;
  const int64_t e1 = r1 * dm.n;
  for (int64_t e0 = r0 * dm.n + threadIdx.x; e0 < e1; e0 += (int64_t)U * blockDim.x) {
    int js[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = e0 + (int64_t)u * blockDim.x;
      js[u] = -1;
      if (e < e1) {
        const int64_t r = e / dm.n;
        if (!vid || vid[b * dm.Tq + r]) js[u] = idx[((b * dm.Tq + r) * dm.Hkv + g) * dm.n + e % dm.n];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = e0 + (int64_t)u * blockDim.x;
      if (e < e1 && slc_pair_kept(js[u], e / dm.n, dm, local_fused)) f(e / dm.n, (int)(e % dm.n), js[u]);
    }
  }
}

__global__ void __launch_bounds__(256) slc_count_kernel(const int32_t* __restrict__ idx,
                                                        const uint8_t* __restrict__ vid, SlcBuckets bk, Dims dm,
                                                        int wgs_per_bg, int local_fused) {
  extern __shared__ int hist[];  // [Ns]
  const int bg = blockIdx.x / wgs_per_bg, part = blockIdx.x % wgs_per_bg;
  const int64_t b = bg / dm.Hkv;
  const int g = bg % dm.Hkv;
  for (int j = threadIdx.x; j < dm.Ns; j += blockDim.x) hist[j] = 0;
  __syncthreads();
  const int64_t r0 = (int64_t)part * RROWS;
  const int64_t r1 = r0 + RROWS < dm.Tq ? r0 + RROWS : dm.Tq;
  slc_for_pairs(idx, vid, dm, b, g, r0, r1, local_fused, [&](int64_t, int, int j) { atomicAdd(&hist[j], 1); });
  __syncthreads();
  for (int j = threadIdx.x; j < dm.Ns; j += blockDim.x)
    if (hist[j]) atomicAdd(&bk.count[(int64_t)bg * dm.Ns + j], hist[j]);
}

// Exclusive scan of x[0..n) in place with 1024 threads; returns the total.
__device__ int block_excl_scan(int* x, int n, int* s_w) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wv = tid >> 6;
  const int per = (n + nt - 1) / nt;
  const int a = tid * per, e = a + per < n ? a + per : n;
  int sum = 0;
  for (int i = a; i < e; ++i) sum += x[i];
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_w[wv] = incl;
  __syncthreads();
  int wbase = 0, total = 0;
  for (int i = 0; i < (nt >> 6); ++i) {
    if (i < wv) wbase += s_w[i];
    total += s_w[i];
  }
  int run = wbase + incl - sum;
  for (int i = a; i < e; ++i) {
    const int v = x[i];
    x[i] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

__global__ void __launch_bounds__(1024) slc_scan_kernel(SlcBuckets bk, Dims dm) {
  extern __shared__ int sm[];  // [2][Ns]
  __shared__ int s_w[16];
  int* s_off = sm;
  int* s_cf = sm + dm.Ns;
  const int bg = blockIdx.x;
  const int64_t base = (int64_t)bg * dm.Ns;
  for (int j = threadIdx.x; j < dm.Ns; j += blockDim.x) {
    const int c = bk.count[base + j];
    s_off[j] = c;
    s_cf[j] = (c + RC - 1) / RC;
  }
  __syncthreads();
  const int nch = block_excl_scan(s_cf, (int)dm.Ns, s_w);
  int* cb = bk.chunk_blk + (int64_t)bg * bk.cap_c;
  int* pl = bk.pairs + (int64_t)bg * bk.cap_c * RC;
  for (int j = threadIdx.x; j < dm.Ns; j += blockDim.x) {
    const int c0 = s_cf[j], c1 = j + 1 < dm.Ns ? s_cf[j + 1] : nch;
    bk.off[base + j] = c0 * RC;
    bk.cfirst[base + j] = c0;
    bk.cursor[base + j] = 0;
    for (int c = c0; c < c1; ++c) cb[c] = j;
    for (int e = c0 * RC + s_off[j]; e < c1 * RC; ++e) pl[e] = -1;  // the last chunk's unused places
  }
  for (int c = nch + threadIdx.x; c < bk.cap_c; c += blockDim.x) cb[c] = -1;
}

__global__ void __launch_bounds__(256) slc_scatter_kernel(const int32_t* __restrict__ idx,
                                                          const uint8_t* __restrict__ vid, SlcBuckets bk, Dims dm,
                                                          int wgs_per_bg, int local_fused) {
  extern __shared__ int sm[];  // hist[Ns], base[Ns]
  int* hist = sm;
  int* pbase = sm + dm.Ns;
  const int bg = blockIdx.x / wgs_per_bg, part = blockIdx.x % wgs_per_bg;
  const int64_t b = bg / dm.Hkv;
  const int g = bg % dm.Hkv;
  for (int j = threadIdx.x; j < dm.Ns; j += blockDim.x) hist[j] = 0;
  __syncthreads();
  const int64_t r0 = (int64_t)part * RROWS;
  const int64_t r1 = r0 + RROWS < dm.Tq ? r0 + RROWS : dm.Tq;
  slc_for_pairs(idx, vid, dm, b, g, r0, r1, local_fused, [&](int64_t, int, int j) { atomicAdd(&hist[j], 1); });
  __syncthreads();
  const int64_t base = (int64_t)bg * dm.Ns;
  for (int j = threadIdx.x; j < dm.Ns; j += blockDim.x) {
    const int c = hist[j];
    pbase[j] = c ? bk.off[base + j] + atomicAdd(&bk.cursor[base + j], c) : 0;
    hist[j] = 0;
  }
  __syncthreads();
  int* pl = bk.pairs + (int64_t)bg * bk.cap_c * RC;
  slc_for_pairs(idx, vid, dm, b, g, r0, r1, local_fused,
                [&](int64_t r, int s, int j) { pl[pbase[j] + atomicAdd(&hist[j], 1)] = (int)(r << 5) | s; });
}

// ---------------------------------------------------------------------------
// Stage rows [key0, key0 + ROWS) of a [*, 128] bf16 array into a swizzled ROWS x 128 LDS tile (the
// swz128 layout) with direct global -> LDS loads, ROWS / 4 instructions of 64 lanes x 16 bytes
// spread over nw waves; rows at or past nrows repeat row nrows - 1 (masked by the caller).
template <int ROWS>
__device__ __forceinline__ void stage_rows(bf16* lds_tile, const bf16* src, int64_t stride, int64_t key0,
                                           int64_t nrows, int w, int nw, int lane) {
  for (int ins = w; ins < ROWS / 4; ins += nw) {
    const int p = ins * 64 + lane;
    const int row = p >> 4, c = (p & 15) ^ (row & 15);
    int64_t key = key0 + row;
    if (key >= nrows) key = nrows - 1;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + key * stride + c * 8),
                                     (__attribute__((address_space(3))) void*)(lds_tile + ins * 512), 16, 0, 0);
  }
}

// One workgroup per chunk of up to 32 (row, slot) pairs of one block of SB tokens (32, 64 or 128);
// wave w = head g*G + w.
template <int SB>
__global__ void __launch_bounds__(512) slc_chunk_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                        const bf16* __restrict__ v, SlcBuckets bk,
                                                        float2* __restrict__ pml, unsigned char* __restrict__ po, Dims dm) {
  constexpr int NKB = SB / 32;  // 32-key blocks of the score tile
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* kt = (bf16*)smem;
  bf16* vt = kt + SB * HD;
  const int G = dm.G;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, n = l & 31;
  const int bg = blockIdx.x / bk.cap_c, cc = blockIdx.x % bk.cap_c;
  // the chunk's block and this lane's pair (row n of the chunk): two independent loads
  const int64_t ci = (int64_t)bg * bk.cap_c + cc;
  const int j = bk.chunk_blk[ci];
  const int pr = bk.pairs[ci * RC + n];
  if (j < 0) return;
  const int64_t b = bg / dm.Hkv;
  const int g = bg % dm.Hkv;
  const int64_t stride = (int64_t)dm.Hkv * HD;
  const int64_t kvb = (b * dm.T * dm.Hkv + g) * (int64_t)HD;
  stage_rows<SB>(kt, k + kvb, stride, (int64_t)j * SB, dm.T, w, G, l);
  stage_rows<SB>(vt, v + kvb, stride, (int64_t)j * SB, dm.T, w, G, l);
  // the lane's query, loaded while the tile streams in
  const bool valid = pr >= 0;
  const int64_t row = valid ? (pr >> 5) : 0;
  const int slot = pr & 31;
  const int h = g * G + w;
  const int64_t t = dm.q0 + row;
  bf16x8 qf[8];
  {
    const bf16* qrow = q + ((b * dm.Tq + row) * dm.Hq + h) * (int64_t)HD + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)(qrow + 16 * ks);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    if (!valid) qf[ks] = zero8();
  // S^T: keys on M (NKB 32-key blocks), the chunk's rows on N
  f32x16 s[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    s[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) s[kb] = mfma32(lds_read8(kt + swz128(kb * 32 + n, 2 * ks + hl)), qf[ks], s[kb]);
  }
  const float c2 = dm.scale * LOG2E_F;
  const int64_t u0 = (int64_t)j * SB;
  const bool need_mask = u0 + SB - 1 > t || u0 + SB > dm.T;  // the row's own block, or past the end
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      if (need_mask) {
        const int64_t u = u0 + kb * 32 + 8 * (jj >> 2) + 4 * hl + (jj & 3);
        if (u > t || u >= dm.T) s[kb][jj] = -INFINITY;
      }
      mx = fmaxf(mx, s[kb][jj]);
    }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(mx, __uint_as_float(hl ? r[0] : r[1]));
  }
  const float off = -mx * c2;
  float ls = 0.f;
  f32x16 oacc[4] = {};
  const int g16 = l >> 4, i16 = l & 15;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    float p[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      p[jj] = fexp2(fmaf(s[kb][jj], c2, off));
      ls += p[jj];
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (bf16)p[8 * st + e];
      const int vr = kb * 32 + 16 * st + 4 * (g16 >> 1) + (i16 >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int col = 32 * db + (g16 & 1) * 16 + 4 * (i16 & 3);
        oacc[db] = mfma32(cat(lds_read_tr(vt + swz128(vr, col >> 3) + (col & 7)),
                              lds_read_tr(vt + swz128(vr + 8, col >> 3) + (col & 7))),
                          pb, oacc[db]);
      }
    }
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ls), __float_as_uint(ls), false, false);
    ls += __uint_as_float(hl ? r[0] : r[1]);
  }
  // O^T register j of dims block db holds dim 32 db + 8 (j >> 2) + 4 hl + (j & 3) of row n: the
  // layout of a 12-bit record half; the record's exponent comes from both halves' largest value.
  float amax = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) amax = fmaxf(amax, fabsf(oacc[db][jj]));
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax), false, false);
    amax = fmaxf(amax, __uint_as_float(hl ? r[0] : r[1]));
  }
  const int ex = rec12_exp(amax);
  if (!valid) return;
  const int64_t ri = (((b * dm.Tq + row) * dm.Hkv + g) * dm.n + slot) * G + w;
  if (hl == 0) pml[ri] = rec12_ml(mx * c2, ls, ex);
  rec12_store_half(po + ri * SLC_REC_BYTES, hl, oacc, 1.f, ex);
}

// ---------------------------------------------------------------------------
// One wave per (video row, group): merge the slots per head, gated combine.  Lane l takes pack
// l & 15 (8 dims) of the records of head w0 + (l >> 4), four heads a pass.
template <bool OCMP_F32>
__global__ void __launch_bounds__(256) slc_merge_kernel(const float2* __restrict__ pml,
                                                        const unsigned char* __restrict__ po,
                                                        const int32_t* __restrict__ idx,
                                                        const uint8_t* __restrict__ vid, const void* __restrict__ ocmp,
                                                        const bf16* __restrict__ swa,
                                                        const float* __restrict__ gates, bf16* __restrict__ out,
                                                        bf16* __restrict__ o_slc, Dims dm) {
  __shared__ float s_wt[4][8][32];  // per wave: slot weights 2^(m - M) / L of each head
  const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * 4 + wv;
  if (item >= dm.B * dm.Tq * dm.Hkv) return;
  const int g = (int)(item % dm.Hkv);
  const int64_t br = item / dm.Hkv;  // b * Tq + r
  if (vid && !vid[br]) return;
  const int G = dm.G;
  const int32_t* sel = idx + item * dm.n;
  const float2* mls = pml + item * dm.n * G;
  const unsigned char* ors = po + item * dm.n * G * (int64_t)SLC_REC_BYTES;
  // weights: lane s (< n) holds slot s; one load round for the (max, sum) of every head.  Slots
  // whose block lies after the row (no key, no partial: see slc_pair_kept) weigh nothing.
  {
    const int64_t jt = (dm.q0 + br % dm.Tq) / dm.ls;
    const int js = sel[l < dm.n ? l : 0];
    const bool lv = l < dm.n && js >= 0 && (int64_t)js <= jt;
    float2 ml[8];
#pragma unroll
    for (int w = 0; w < 8; ++w)
      ml[w] = (lv && w < G) ? mls[l * G + w] : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      if (w >= G) break;
      float M = ml[w].x;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
      const float f = lv ? fexp2(ml[w].x - M) : 0.f;
      float L = f * ml[w].y;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
      if (l < 32) s_wt[wv][w][l] = (L > 0.f && l < dm.n) ? f / L : 0.f;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // values: 16 slots a pass, all loads of a pass in flight.  Integer records hold no NaN or
  // infinity, so unused slots (stale data) need only their zero weight.
  const int P = l & 15, hsub = l >> 4;
  const int d0 = 32 * ((P & 7) >> 1) + 16 * (P & 1) + 4 * (P >> 3);  // dims d0 .. d0+3, d0+8 .. d0+11
  for (int w0 = 0; w0 < G; w0 += 4) {
    const int w = w0 + hsub;
    const int wc = w < G ? w : G - 1;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < dm.n; s0 += 16) {
      uint32_t x[16][3];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int s = s0 + u < dm.n ? s0 + u : dm.n - 1;
        const uint32_t* src = (const uint32_t*)(ors + ((int64_t)s * G + wc) * SLC_REC_BYTES + 12 * P);
        x[u][0] = src[0];
        x[u][1] = src[1];
        x[u][2] = src[2];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float ws = (s0 + u < dm.n) ? s_wt[wv][wc][s0 + u] : 0.f;
        float y[8];
        rec12_unpack8(x[u][0], x[u][1], x[u][2], y);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = fmaf(ws, y[i], o[i]);
      }
    }
    if (w >= G) continue;
    const int hq = g * G + w;
    const int64_t rowoff = (br * dm.Hq + hq) * (int64_t)HD;
    const float* gg = gates + (br * dm.Hq + hq) * 3;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int64_t off = rowoff + d0 + 8 * half;
      const float* oh = o + 4 * half;
      if (o_slc) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)oh[e];
        *(bf16x4*)(o_slc + off) = v4;
      }
      if (out) {
        float c[4];
        if constexpr (OCMP_F32) {
          const float4 c4 = *(const float4*)((const float*)ocmp + off);
          c[0] = c4.x; c[1] = c4.y; c[2] = c4.z; c[3] = c4.w;
        } else {
          const bf16x4 c4 = *(const bf16x4*)((const bf16*)ocmp + off);
#pragma unroll
          for (int e = 0; e < 4; ++e) c[e] = (float)c4[e];
        }
        const bf16x4 sw = *(const bf16x4*)(swa + off);
        const float swv[4] = {(float)sw[0], (float)sw[1], (float)sw[2], (float)sw[3]};
        const float g0 = gg[0], g1 = gg[1], g2 = gg[2];
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)(g0 * c[e] + g1 * oh[e] + g2 * swv[e]);
        *(bf16x4*)(out + off) = v4;
      }
    }
  }
}

// ---------------------------------------------------------------------------
static size_t srup(size_t x) { return (x + 255) & ~(size_t)255; }

// Bytes of the bucketing arrays (counts, offsets, first chunks, cursors, the chunk -> block map and
// the pair lists); the selection partials follow them in the forward's workspace.
size_t slc_bucket_bytes(const Dims& dm) {
  const size_t bgs = (size_t)dm.B * dm.Hkv;
  return 4 * srup(bgs * dm.Ns * 4) + srup(bgs * slc_cap_chunks(dm) * 4) + srup(bgs * slc_cap_chunks(dm) * RC * 4);
}

size_t slc_block_workspace(const Dims& dm) {
  const size_t recs = (size_t)dm.B * dm.Tq * dm.Hkv * dm.n * dm.G;
  return slc_bucket_bytes(dm) + srup(recs * 8) + srup(recs * SLC_REC_BYTES);
}

// The (max, sum) and value-record arrays of the selection partials inside the workspace.
void slc_partial_arrays(const Dims& dm, void* ws, void** ml, void** o) {
  const size_t recs = (size_t)dm.B * dm.Tq * dm.Hkv * dm.n * dm.G;
  char* p = (char*)ws + slc_bucket_bytes(dm);
  *ml = p;
  *o = p + srup(recs * 8);
}

// Buckets the kept (row, slot) pairs by chosen block (slc_count, slc_scan, slc_scatter) into the
// arrays at the start of ws (slc_bucket_bytes(dm) bytes).
static hipError_t slc_buckets(const Dims& dm, const int32_t* idx, const uint8_t* vid, void* ws, bool local_fused,
                              SlcBuckets* out, hipStream_t s) {
  const int bgs = (int)(dm.B * dm.Hkv);
  char* p = (char*)ws;
  SlcBuckets bk;
  const size_t nb = srup((size_t)bgs * dm.Ns * 4);
  bk.count = (int*)p;
  bk.off = (int*)(p + nb);
  bk.cfirst = (int*)(p + 2 * nb);
  bk.cursor = (int*)(p + 3 * nb);
  p += 4 * nb;
  bk.cap_c = slc_cap_chunks(dm);
  bk.chunk_blk = (int*)p;
  p += srup((size_t)bgs * bk.cap_c * 4);
  bk.pairs = (int*)p;
  const int wpb = (int)((dm.Tq + RROWS - 1) / RROWS);
  const size_t hist = (size_t)dm.Ns * 4;
  // counts start at zero (a kernel, not a memset: callers may capture the launch in a graph)
  const int64_t ncount = (int64_t)bgs * dm.Ns;
  slc_zero_kernel<<<dim3((unsigned)((ncount + 255) / 256)), dim3(256), 0, s>>>(bk.count, ncount);
  for (const void* fn : {(const void*)slc_count_kernel, (const void*)slc_scatter_kernel, (const void*)slc_scan_kernel}) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(2 * hist));
    if (e != hipSuccess) return e;
  }
  slc_count_kernel<<<dim3(bgs * wpb), dim3(256), hist, s>>>(idx, vid, bk, dm, wpb, local_fused ? 1 : 0);
  slc_scan_kernel<<<dim3(bgs), dim3(1024), 2 * hist, s>>>(bk, dm);
  slc_scatter_kernel<<<dim3(bgs * wpb), dim3(256), 2 * hist, s>>>(idx, vid, bk, dm, wpb, local_fused ? 1 : 0);
  *out = bk;
  return hipGetLastError();
}

hipError_t launch_slc_pair_lists(const Dims& dm, const int32_t* idx, const uint8_t* vid, void* ws, SlcPairLists* pl,
                                 hipStream_t s) {
  SlcBuckets bk;
  const hipError_t e = slc_buckets(dm, idx, vid, ws, false, &bk, s);
  pl->chunk_blk = bk.chunk_blk;
  pl->pairs = bk.pairs;
  pl->cfirst = bk.cfirst;
  pl->cap_c = bk.cap_c;
  return e;
}

hipError_t launch_slc_block(const Dims& dm, const void* q, const void* k, const void* v, const int32_t* idx,
                            const uint8_t* vid, const void* ocmp, bool ocmp_f32, const void* swa,
                            const float* gates, void* out, void* o_slc, void* ws, hipStream_t s, bool local_fused,
                            hipEvent_t before_merge) {
  if (dm.B <= 0 || dm.Tq <= 0) return hipSuccess;
  const int bgs = (int)(dm.B * dm.Hkv);
  SlcBuckets bk;
  hipError_t e = slc_buckets(dm, idx, vid, ws, local_fused, &bk, s);
  if (e != hipSuccess) return e;
  const size_t recs = (size_t)dm.B * dm.Tq * dm.Hkv * dm.n * dm.G;
  float2* pml = (float2*)((char*)ws + slc_bucket_bytes(dm));
  unsigned char* po = (unsigned char*)pml + srup(recs * 8);
  auto chunk = [&](auto kernel, int sb) -> hipError_t {
    const int shm = 2 * sb * HD * 2;
    hipError_t e2 = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, shm);
    if (e2 != hipSuccess) return e2;
    kernel<<<dim3((unsigned)bgs * bk.cap_c), dim3(dm.G * 64), shm, s>>>((const bf16*)q, (const bf16*)k,
                                                                        (const bf16*)v, bk, pml, po, dm);
    return hipGetLastError();
  };
  e = dm.ls == 32 ? chunk(slc_chunk_kernel<32>, 32)
                  : dm.ls == 128 ? chunk(slc_chunk_kernel<128>, 128) : chunk(slc_chunk_kernel<64>, 64);
  if (e != hipSuccess) return e;
  // the merge reads the window pass's outputs (run on another stream when before_merge is given)
  if (before_merge) {
    e = hipStreamWaitEvent(s, before_merge, 0);
    if (e != hipSuccess) return e;
  }
  const int64_t items = dm.B * dm.Tq * dm.Hkv;
  const dim3 mg((unsigned)((items + 3) / 4));
  if (ocmp_f32)
    slc_merge_kernel<true><<<mg, dim3(256), 0, s>>>(pml, po, idx, vid, ocmp, (const bf16*)swa, gates, (bf16*)out,
                                                    (bf16*)o_slc, dm);
  else
    slc_merge_kernel<false><<<mg, dim3(256), 0, s>>>(pml, po, idx, vid, ocmp, (const bf16*)swa, gates, (bf16*)out,
                                                     (bf16*)o_slc, dm);
  return hipGetLastError();
}
