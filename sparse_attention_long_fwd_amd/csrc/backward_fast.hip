// Backward pass of the hybrid layer on the matrix cores (bf16 inputs, head_dim 128, gfx950).
//
// The forward is the layer of the other kernels (top168.com digest of VideoNSA, section 一; csdn
// page "VideoNSA：重新定义视频理解的稀疏注意力机制", sections 2.2 and 3.1): for video rows
// out = g_c o_c + g_s o_s + g_w o_w over the compression, selection and window branches, for text
// rows dense causal attention.  Per branch b of one (row, head), with P the probabilities over its
// keys and E_b = sum_u P_u <d_out, v_u>:
//   d g_b = E_b,   ds_u = g_b P_u (<d_out, v_u> - E_b),
//   dq += scale sum_u ds_u k_u,   dk_u += scale ds_u q,   dv_u += g_b P_u d_out
// (text rows: one branch over the keys [0, t], g = 1).  The chosen blocks are an input and pass no
// gradient.  Compressed keys and values are weighted block sums of k and v; their gradients go
// back through the weights afterwards (launch_bwd_compress_grads).
//
// Every score is formed again from bf16 q, k, v and d_out (exact products, fp32 sums): once for the
// branch statistics (log-sum-exp and E) and once for each gradient product.  P and ds enter the
// matrix products as a bf16 high part plus a bf16 remainder (two products, within 2^-17 of the
// fp32 value), and so do the compressed keys and values (their fp32 sums split at compression),
// so the gradients keep the accuracy of fp32 accumulation.
//
// Kernels, per (batch, KV group):
//  bwdf_row_kernel<CMP>: 16 query rows x the group's heads (a wave per head); two sweeps over the
//    rows' keys, staged 64 at a time in LDS: the statistics (online max, sum and sum P dP), then
//    dq^T += K^T ds^T.  CMP: the compressed keys visible to the video rows (the first writer of dq
//    and of statistics slot 0); else the window keys of video rows and the keys [0, t] of text rows
//    (adds to dq; slot 2).
//  bwdf_key_kernel<CMP>: 64 keys (16 a wave) x the rows that can see them, 32 rows of one head at a
//    time with their q and d_out staged in LDS: S = Q K^T, dv^T += d_out^T (g P),
//    dk^T += Q^T ds.  Row tiles are split into chunks whose sums go out with atomic adds.
//    Row and key tiles of one (sequence, KV group) run on as few XCDs as possible, neighbours
//    (which share keys or rows) together.
//  Selection, per (sequence, run of rows) sub-problem, block-major over the pair lists of
//    launch_slc_pair_lists (chunks of 32 (row, slot) pairs of one chosen block):
//    bwdf_sel_stats_kernel leaves per (row, slot, head) the block's max, sum and sum P dP;
//    bwdf_sel_merge_kernel combines a row's slots (statistics slot 1, d gates);
//    bwdf_sel_grad_kernel (a workgroup per run of up to 32 chunks of a block) adds dk, dv (atomic
//    adds) and writes per-pair dq records that bwdf_sel_dq_merge_kernel adds to dq in slot order.
// The order of the atomic adds depends on scheduling: the last bits of dk and dv can differ from
// one call to the next (dq and the d gates are summed in a fixed order).
#include "backward.hpp"
#include "fast_common.hpp"

namespace {
constexpr int HD = 128;
constexpr int RT = 16;                 // query rows per row-kernel tile
constexpr int KT = 64;                 // keys per key tile
constexpr int KR = 32;                 // query rows per key-kernel row tile
constexpr int PRC = 32;                // pairs per selection chunk
constexpr int NOKEY = 0x7fffffff;      // first key of a row that sees none
constexpr int RTC_WIN = 128, RTC_CMP = 32;  // row tiles per chunk of the key kernels
}  // namespace

// Element i of hv / lv: the bf16 high part and remainder of x (x - hi is exact in fp32; hi + lo is
// within 2^-17 |x| of x)
__device__ __forceinline__ void split2(float x, bf16x8& hv, bf16x8& lv, int i) {
  const bf16 hi = (bf16)x;
  hv[i] = hi;
  lv[i] = (bf16)(x - (float)hi);
}

// Rows [row0, row0 + ROWS) of a [*, 128] bf16 array (row stride `stride` elements) into a swizzled
// ROWS x 128 LDS tile (swz128) with direct global -> LDS loads, ROWS / 4 instructions of 64 lanes x
// 16 bytes over nw waves; rows at or past nrows repeat row nrows - 1 (masked by the callers).
template <int ROWS>
__device__ __forceinline__ void stage_rows_bw(bf16* lds_tile, const bf16* src, int64_t stride, int64_t row0,
                                              int64_t nrows, int w, int nw, int lane) {
  for (int ins = w; ins < ROWS / 4; ins += nw) {
    const int p = ins * 64 + lane;
    const int row = p >> 4, c = (p & 15) ^ (row & 15);
    int64_t r = row0 + row;
    if (r >= nrows) r = nrows - 1;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + r * stride + c * 8),
                                     (__attribute__((address_space(3))) void*)(lds_tile + ins * 512), 16, 0, 0);
  }
}

// A operand of a 16x16x32 product, read transposed from a swizzled [rows][128] LDS tile: lane
// (c = l % 16, gi = l / 16) gets column 16 db + c of rows r0 + 4 gi .. +3, then of rows
// r0 + 16 + 4 gi .. +3 — the K order of a B operand built from two 16-row accumulator blocks
// (elements j = 0..3 of the first block, then of the second).
__device__ __forceinline__ bf16x8 tr_a16(const bf16* tile, int r0, int db, int c, int gi) {
  const int col = 16 * db + 4 * (c & 3);
  const int ra = r0 + 4 * gi + (c >> 2);
  return cat(lds_read_tr(tile + swz128(ra, col >> 3) + (col & 7)),
             lds_read_tr(tile + swz128(ra + 16, col >> 3) + (col & 7)));
}

__device__ __forceinline__ float swap_halves(float x, int hl) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(hl ? r[0] : r[1]);
}

// Keys [klo, khi] of a row in the branch's key index space (klo = NOKEY, khi = -1: none).  CMP: the
// compressed keys a video row sees; else the window keys of a video row and [0, t] for a text row.
template <bool CMP>
__device__ __forceinline__ void row_keys(int64_t t, bool isv, const Dims& dm, int& klo, int& khi) {
  klo = NOKEY;
  khi = -1;
  if (CMP) {
    if (isv) {
      const int64_t nv = cmp_visible(t, dm.l, dm.d, dm.Nc);
      if (nv > 0) {
        klo = 0;
        khi = (int)nv - 1;
      }
    }
  } else {
    klo = isv ? (int)(t - dm.w + 1 > 0 ? t - dm.w + 1 : 0) : 0;
    khi = (int)t;
  }
}

// ---------------------------------------------------------------------------
// Row kernel: one workgroup per (batch, 16-row tile, KV group), wave w = head g G + w.  S^T = K Q^T
// (keys on M, the tile's rows on N: lane (c, gi) holds rows c, keys 16 mb + 4 gi + j), the row
// statistics per lane, dq^T = K^T ds^T with K^T read transposed from the key tile.
template <bool CMP>
__global__ void __launch_bounds__(512)
    bwdf_row_kernel(const bf16* __restrict__ q, const bf16* __restrict__ dout, const bf16* __restrict__ kh,
                    const bf16* __restrict__ kl, const bf16* __restrict__ vh, const bf16* __restrict__ vl,
                    const uint8_t* __restrict__ vid, const float* __restrict__ gates, float* __restrict__ dq,
                    float* __restrict__ dgates, float* __restrict__ st_l, float* __restrict__ st_e, Dims dm) {
  constexpr int NT = CMP ? 4 : 2;  // LDS tiles per key tile: K, V (and their remainders)
  const int ntile = (int)((dm.Tq + RT - 1) / RT);
  // the row tiles of one (sequence, KV group) stay on as few XCDs as possible (their keys overlap)
  int unit, rank;
  if (!xcd_remap(blockIdx.x, (int)(dm.B * dm.Hkv), ntile, &unit, &rank)) return;
  constexpr int SLOT = CMP ? 0 : 2;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* lds = (bf16*)smem;
  const int G = dm.G;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, gi = l >> 4;
  const int64_t r0 = (int64_t)(ntile - 1 - rank) * RT;  // later (longer) tiles first
  const int g = unit % dm.Hkv;
  const int64_t b = unit / dm.Hkv;
  const int64_t r = r0 + c;
  const bool rvalid = r < dm.Tq;
  const int64_t rr = rvalid ? r : dm.Tq - 1;
  const int64_t t = dm.q0 + rr;
  const bool isv = vid ? vid[b * dm.Tq + rr] != 0 : true;
  const int h = g * G + w;
  const int64_t row = (b * dm.Tq + rr) * dm.Hq + h;
  const int64_t N = CMP ? dm.Nc : dm.T;
  int klo, khi;
  row_keys<CMP>(t, isv, dm, klo, khi);
  if (!rvalid) {
    klo = NOKEY;
    khi = -1;
  }
  // the tile's key range and the range every row sees in full (the same in every wave)
  int kmin = klo, kmax = khi, maxlo = klo, minhi = khi;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    kmin = min(kmin, __shfl_xor(kmin, o, 64));
    kmax = max(kmax, __shfl_xor(kmax, o, 64));
    maxlo = max(maxlo, __shfl_xor(maxlo, o, 64));
    minhi = min(minhi, __shfl_xor(minhi, o, 64));
  }
  kmin = __builtin_amdgcn_readfirstlane(kmin);
  kmax = __builtin_amdgcn_readfirstlane(kmax);
  maxlo = __builtin_amdgcn_readfirstlane(maxlo);
  minhi = __builtin_amdgcn_readfirstlane(minhi);
  const int kt0 = kmax >= kmin ? kmin / KT : 0;
  const int nk = kmax >= kmin ? kmax / KT - kmin / KT + 1 : 0;

  bf16x8 qf[4], df[4];  // Q^T and d_out^T operands: row c, dims 32 ks + 8 gi .. +8
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qf[ks] = *(const bf16x8*)(q + row * HD + 32 * ks + 8 * gi);
    df[ks] = *(const bf16x8*)(dout + row * HD + 32 * ks + 8 * gi);
  }
  const float gate = CMP ? (isv ? gates[row * 3] : 0.f) : (isv ? gates[row * 3 + 2] : 1.f);
  const float cs = dm.scale * LOG2E_F;

  const int64_t kstride = (int64_t)dm.Hkv * HD;
  const int64_t koff = (b * N * dm.Hkv + g) * (int64_t)HD;
  auto stage = [&](int buf, int kt) {
    bf16* base = lds + (size_t)buf * NT * KT * HD;
    stage_rows_bw<KT>(base, kh + koff, kstride, (int64_t)kt * KT, N, w, G, l);
    stage_rows_bw<KT>(base + KT * HD, vh + koff, kstride, (int64_t)kt * KT, N, w, G, l);
    if constexpr (CMP) {
      stage_rows_bw<KT>(base + 2 * KT * HD, kl + koff, kstride, (int64_t)kt * KT, N, w, G, l);
      stage_rows_bw<KT>(base + 3 * KT * HD, vl + koff, kstride, (int64_t)kt * KT, N, w, G, l);
    }
  };
  // one pass over the key tiles, each staged one ahead into the other buffer
  auto sweep = [&](auto body) {
    if (nk <= 0) return;
    stage(0, kt0);
    for (int i = 0; i < nk; ++i) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (i + 1 < nk) stage((i + 1) & 1, kt0 + i + 1);
      body((const bf16*)(lds + (size_t)(i & 1) * NT * KT * HD), kt0 + i);
    }
    __syncthreads();  // every wave is done with the buffers before they are staged again
  };
  // S^T and dP^T = V d_out^T of one key tile
  auto scores = [&](const bf16* base, f32x4(&S)[4], f32x4(&P)[4]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) S[mb] = P[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int o = swz128(16 * mb + c, 4 * ks + gi);
        S[mb] = mfma16(lds_read8(base + o), qf[ks], S[mb]);
        P[mb] = mfma16(lds_read8(base + KT * HD + o), df[ks], P[mb]);
        if constexpr (CMP) {
          S[mb] = mfma16(lds_read8(base + 2 * KT * HD + o), qf[ks], S[mb]);
          P[mb] = mfma16(lds_read8(base + 3 * KT * HD + o), df[ks], P[mb]);
        }
      }
  };
  auto full_tile = [&](int kt) { return kt * KT >= maxlo && kt * KT + KT - 1 <= minhi; };

  // sweep 1: this lane's share of the row's max, sum and sum P dP (log2 units)
  float m_run = -INFINITY, l_run = 0.f, e_run = 0.f;
  sweep([&](const bf16* base, int kt) {
    f32x4 S[4], P[4];
    scores(base, S, P);
    const bool full = full_tile(kt);
    float x[16], mt = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v = S[mb][j] * cs;
        if (!full) {
          const int u = kt * KT + 16 * mb + 4 * gi + j;
          if (u < klo || u > khi) v = -INFINITY;
        }
        x[4 * mb + j] = v;
        mt = fmaxf(mt, v);
      }
    const float mn = fmaxf(m_run, mt), mref = mn == -INFINITY ? 0.f : mn;
    const float a = fexp2(m_run - mref);
    float ls = 0.f, es = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fexp2(x[i] - mref);
      ls += p;
      es = fmaf(p, P[i >> 2][i & 3], es);
    }
    l_run = fmaf(l_run, a, ls);
    e_run = fmaf(e_run, a, es);
    m_run = mn;
  });
#pragma unroll
  for (int o = 16; o < 64; o <<= 1) {
    const float mo = __shfl_xor(m_run, o, 64), lo = __shfl_xor(l_run, o, 64), eo = __shfl_xor(e_run, o, 64);
    const float mn = fmaxf(m_run, mo), mref = mn == -INFINITY ? 0.f : mn;
    const float a = fexp2(m_run - mref), a2 = fexp2(mo - mref);
    l_run = l_run * a + lo * a2;
    e_run = e_run * a + eo * a2;
    m_run = mn;
  }
  const bool has = l_run > 0.f;
  const float L2 = has ? m_run + log2f(l_run) : INFINITY;  // P = 2^(S cs - L2); none when empty
  const float E = has ? e_run / l_run : 0.f;

  // sweep 2: dq^T += K^T ds^T, ds = g P (dP - E) as bf16 high part + remainder
  f32x4 dqa[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) dqa[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  sweep([&](const bf16* base, int kt) {
    f32x4 S[4], P[4];
    scores(base, S, P);
    const bool full = full_tile(kt);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      bf16x8 bh, bl;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int mb = 2 * hh + sub;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float p = fexp2(fmaf(S[mb][j], cs, -L2));
          if (!full) {
            const int u = kt * KT + 16 * mb + 4 * gi + j;
            if (u < klo || u > khi) p = 0.f;
          }
          split2(gate * p * (P[mb][j] - E), bh, bl, 4 * sub + j);
        }
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const bf16x8 a = tr_a16(base, 32 * hh, db, c, gi);
        dqa[db] = mfma16(a, bh, dqa[db]);
        dqa[db] = mfma16(a, bl, dqa[db]);
        if constexpr (CMP) dqa[db] = mfma16(tr_a16(base + 2 * KT * HD, 32 * hh, db, c, gi), bh, dqa[db]);
      }
    }
  });
  if (!rvalid) return;
  // dq^T register j of dims block db holds dim 16 db + 4 gi + j of row c
  float* dst = dq + row * HD + 4 * gi;
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    float4 v = make_float4(dqa[db][0] * dm.scale, dqa[db][1] * dm.scale, dqa[db][2] * dm.scale,
                           dqa[db][3] * dm.scale);
    if constexpr (!CMP) {
      const float4 o = *(const float4*)(dst + 16 * db);
      v.x += o.x;
      v.y += o.y;
      v.z += o.z;
      v.w += o.w;
    }
    *(float4*)(dst + 16 * db) = v;
  }
  if (gi == 0) {
    st_l[row * 3 + SLOT] = L2;
    st_e[row * 3 + SLOT] = E;
    dgates[row * 3 + SLOT] = isv ? E : 0.f;
  }
}

// ---------------------------------------------------------------------------
// Key kernel: one workgroup per (batch, 64 keys, row chunk, KV group); wave w owns keys
// kbase + 16 w .. +15 (N of the products; K and V operands in registers) and sums over the heads and
// the rows that see them.  S = Q K^T (the rows on M: lane (c, gi) holds rows 16 mb + 4 gi + j,
// key c), dv^T += d_out^T (g P), dk^T += Q^T ds with Q and d_out read transposed from LDS.
template <bool CMP>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
    bwdf_key_kernel(const bf16* __restrict__ q, const bf16* __restrict__ dout, const bf16* __restrict__ kh,
                    const bf16* __restrict__ kl, const bf16* __restrict__ vh, const bf16* __restrict__ vl,
                    const uint8_t* __restrict__ vid, const float* __restrict__ gates, const float* __restrict__ st_l,
                    const float* __restrict__ st_e, const uint32_t* __restrict__ tbits, float* __restrict__ dk,
                    float* __restrict__ dv, Dims dm, int nch) {
  constexpr int SLOT = CMP ? 0 : 2;
  constexpr int RTC = CMP ? RTC_CMP : RTC_WIN;
  __shared__ __attribute__((aligned(16))) bf16 tq[2][KR * HD];
  __shared__ __attribute__((aligned(16))) bf16 tdo[2][KR * HD];
  __shared__ __attribute__((aligned(16))) float sL[2][KR], sE[2][KR], sG[2][KR];
  __shared__ __attribute__((aligned(16))) int sLo[2][KR], sHi[2][KR];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, gi = l >> 4;
  const int G = dm.G;
  const int64_t N = CMP ? dm.Nc : dm.T;
  // the work of one (sequence, KV group) is kept on as few XCDs as possible, in an order whose
  // neighbours read the same q / d_out tiles from the XCD's L2: window keys key-tile-major (the
  // bands of neighbouring key tiles overlap), compressed keys chunk-major (every key tile of a
  // row chunk reads all its rows)
  const int nkt = (int)((N + KT - 1) / KT);
  int unit, rank;
  if (!xcd_remap(blockIdx.x, (int)(dm.B * dm.Hkv), nkt * nch, &unit, &rank)) return;
  const int64_t ktile = CMP ? rank % nkt : rank / nch;
  const int ch = CMP ? rank / nkt : rank % nch;
  const int g = unit % dm.Hkv;
  const int64_t b = unit / dm.Hkv;
  const int64_t kbase = ktile * KT;
  const int64_t ntr = (dm.Tq + KR - 1) / KR;
  // the first position that sees a key of the tile, the chunk's row tiles from there
  const int64_t tfirst = CMP ? kbase * dm.d + dm.l - 1 : kbase;
  const int64_t rfirst = tfirst - dm.q0 > 0 ? tfirst - dm.q0 : 0;
  int64_t ra = rfirst / KR;
  if (ra < (int64_t)ch * RTC) ra = (int64_t)ch * RTC;
  const int64_t rb = (int64_t)(ch + 1) * RTC < ntr ? (int64_t)(ch + 1) * RTC : ntr;
  // window rows past row tile `band` see none of the tile's keys; text rows see every key before them
  const int64_t lastw = kbase + KT + dm.w - 2 - dm.q0;
  const int64_t band = CMP ? ntr : (lastw < 0 ? 0 : lastw / KR + 1);
  auto visit = [&](int64_t rt) -> bool { return rt < band || tbits[b * ntr + rt] != 0u; };
  auto next_rt = [&](int64_t rt) -> int64_t {
    for (++rt; rt < rb; ++rt)
      if (visit(rt)) break;
    return rt;
  };
  int64_t rt_first = ra;
  if (rt_first < rb && !visit(rt_first)) rt_first = next_rt(rt_first);
  if (rt_first >= rb) return;  // no row of the chunk sees the tile

  const int64_t u = kbase + 16 * w + c;
  const bool uvalid = u < N;
  const int64_t ur = uvalid ? u : N - 1;
  bf16x8 kf[4], vf[4], kfl[4], vfl[4];  // K^T, V^T operands: key c, dims 32 ks + 8 gi .. +8
  {
    const int64_t o = ((b * N + ur) * dm.Hkv + g) * (int64_t)HD + 8 * gi;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kf[ks] = *(const bf16x8*)(kh + o + 32 * ks);
      vf[ks] = *(const bf16x8*)(vh + o + 32 * ks);
      if constexpr (CMP) {
        kfl[ks] = *(const bf16x8*)(kl + o + 32 * ks);
        vfl[ks] = *(const bf16x8*)(vl + o + 32 * ks);
      }
    }
  }
  const int64_t qstride = (int64_t)dm.Hq * HD;
  auto stage = [&](int buf, int h, int64_t rt) {
    const int64_t qo = (b * dm.Tq * dm.Hq + g * G + h) * (int64_t)HD;
    stage_rows_bw<KR>(tq[buf], q + qo, qstride, rt * KR, dm.Tq, w, 4, l);
    stage_rows_bw<KR>(tdo[buf], dout + qo, qstride, rt * KR, dm.Tq, w, 4, l);
  };
  // statistics of row rt KR + tid (tid < KR) of head g G + h
  struct RowSt {
    float L, E, G;
    int lo, hi;
  };
  auto load_st = [&](int h, int64_t rt) -> RowSt {
    RowSt s{INFINITY, 0.f, 0.f, NOKEY, -1};
    const int64_t r = rt * KR + tid;
    if (r < dm.Tq) {
      const int64_t ri = (b * dm.Tq + r) * dm.Hq + g * G + h;
      const bool isv = vid ? vid[b * dm.Tq + r] != 0 : true;
      s.L = st_l[ri * 3 + SLOT];
      s.E = st_e[ri * 3 + SLOT];
      s.G = CMP ? (isv ? gates[ri * 3] : 0.f) : (isv ? gates[ri * 3 + 2] : 1.f);
      row_keys<CMP>(dm.q0 + r, isv, dm, s.lo, s.hi);
    }
    return s;
  };
  auto put_st = [&](int buf, const RowSt& s) {
    sL[buf][tid] = s.L;
    sE[buf][tid] = s.E;
    sG[buf][tid] = s.G;
    sLo[buf][tid] = s.lo;
    sHi[buf][tid] = s.hi;
  };
  const float cs = dm.scale * LOG2E_F;
  f32x4 dka[8], dva[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) dka[db] = dva[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  stage(0, 0, rt_first);
  if (tid < KR) put_st(0, load_st(0, rt_first));
  int hcur = 0, buf = 0;
  int64_t rtcur = rt_first;
  for (;;) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    int hn = hcur;
    int64_t rtn = next_rt(rtcur);
    if (rtn >= rb) {
      hn = hcur + 1;
      rtn = rt_first;
    }
    const bool more = hn < G;
    RowSt nst{};
    if (more) {
      stage(buf ^ 1, hn, rtn);
      if (tid < KR) nst = load_st(hn, rtn);
    }
    // this item: head hcur, rows rtcur KR .. +31
    {
      const bf16* Qt = tq[buf];
      const bf16* Dt = tdo[buf];
      f32x4 S[2], P[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) S[mb] = P[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int o = swz128(16 * mb + c, 4 * ks + gi);
          const bf16x8 qa = lds_read8(Qt + o), da = lds_read8(Dt + o);
          S[mb] = mfma16(qa, kf[ks], S[mb]);
          P[mb] = mfma16(da, vf[ks], P[mb]);
          if constexpr (CMP) {
            S[mb] = mfma16(qa, kfl[ks], S[mb]);
            P[mb] = mfma16(da, vfl[ks], P[mb]);
          }
        }
      bf16x8 ph, pl, sh, sl;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int rq = 16 * mb + 4 * gi;
        const float4 L4 = *(const float4*)&sL[buf][rq];
        const float4 E4 = *(const float4*)&sE[buf][rq];
        const float4 G4 = *(const float4*)&sG[buf][rq];
        const int4 lo4 = *(const int4*)&sLo[buf][rq];
        const int4 hi4 = *(const int4*)&sHi[buf][rq];
        const float Lv[4] = {L4.x, L4.y, L4.z, L4.w}, Ev[4] = {E4.x, E4.y, E4.z, E4.w};
        const float Gv[4] = {G4.x, G4.y, G4.z, G4.w};
        const int lov[4] = {lo4.x, lo4.y, lo4.z, lo4.w}, hiv[4] = {hi4.x, hi4.y, hi4.z, hi4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float p = fexp2(fmaf(S[mb][j], cs, -Lv[j]));
          if (!(uvalid && u >= lov[j] && u <= hiv[j])) p = 0.f;
          const float gp = Gv[j] * p;
          split2(gp, ph, pl, 4 * mb + j);
          split2(gp * (P[mb][j] - Ev[j]), sh, sl, 4 * mb + j);
        }
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const bf16x8 ad = tr_a16(Dt, 0, db, c, gi);
        dva[db] = mfma16(ad, ph, dva[db]);
        dva[db] = mfma16(ad, pl, dva[db]);
        const bf16x8 aq = tr_a16(Qt, 0, db, c, gi);
        dka[db] = mfma16(aq, sh, dka[db]);
        dka[db] = mfma16(aq, sl, dka[db]);
      }
    }
    if (!more) break;
    if (tid < KR) put_st(buf ^ 1, nst);
    hcur = hn;
    rtcur = rtn;
    buf ^= 1;
  }
  if (!uvalid) return;
  // dk^T / dv^T register j of dims block db holds dim 16 db + 4 gi + j of key c
  float* dkp = dk + ((b * N + u) * dm.Hkv + g) * (int64_t)HD + 4 * gi;
  float* dvp = dv + ((b * N + u) * dm.Hkv + g) * (int64_t)HD + 4 * gi;
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      unsafeAtomicAdd(dkp + 16 * db + j, dka[db][j] * dm.scale);
      unsafeAtomicAdd(dvp + 16 * db + j, dva[db][j]);
    }
}

// tbits[b][wi] bit i: row 32 wi + i of batch b is a text row.
__global__ void __launch_bounds__(256) bwdf_tbits_kernel(const uint8_t* __restrict__ vid, uint32_t* __restrict__ tbits,
                                                         Dims dm) {
  const int64_t ntr = (dm.Tq + 31) / 32;
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= dm.B * ntr) return;
  const int64_t b = x / ntr, wi = x % ntr;
  uint32_t m = 0;
  if (vid)
    for (int i = 0; i < 32; ++i) {
      const int64_t r = wi * 32 + i;
      if (r < dm.Tq && !vid[b * dm.Tq + r]) m |= 1u << i;
    }
  tbits[x] = m;
}

__global__ void __launch_bounds__(256) bwdf_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    *(float4*)(p + i) = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    for (int64_t j = i; j < n; ++j) p[j] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Selection, block-major.  One workgroup per chunk of up to 32 (row, slot) pairs of one block of SB
// tokens.  The stats and dq kernels take a wave per head (wave w = head g G + w) with the block's K
// and V staged in LDS and the pair's row on N (lane n = l % 32): S^T = K Q^T, dP^T = V d_out^T.
struct SelChunk {
  int64_t b, row, t, rowi;
  int g, slot, j;
  bool valid;
};

__device__ __forceinline__ bool sel_chunk_setup(const SlcPairLists& pl, const Dims& dm, int w, int n,
                                                SelChunk& sc) {
  const int bg = blockIdx.x / pl.cap_c, cc = blockIdx.x % pl.cap_c;
  const int64_t ci = (int64_t)bg * pl.cap_c + cc;
  sc.j = pl.chunk_blk[ci];
  const int pr = pl.pairs[ci * PRC + n];
  if (sc.j < 0) return false;
  sc.b = bg / dm.Hkv;
  sc.g = bg % dm.Hkv;
  sc.valid = pr >= 0;
  sc.row = sc.valid ? (pr >> 5) : 0;
  sc.slot = pr & 31;
  sc.t = dm.q0 + sc.row;
  sc.rowi = (sc.b * dm.Tq + sc.row) * dm.Hq + sc.g * dm.G + w;
  return true;
}

// S^T and dP^T of the chunk's block (keys kb 32 + 8 (jj / 4) + 4 hl + jj % 4 of register jj),
// scaled to log2 units, keys after the row or past the sequence at -inf.
template <int SB>
__device__ __forceinline__ void sel_scores(const bf16* kt, const bf16* vt, const bf16x8 (&qf)[8],
                                           const bf16x8 (&df)[8], const SelChunk& sc, const Dims& dm, int n,
                                           int hl, float cs, f32x16 (&s)[SB / 32], f32x16 (&dp)[SB / 32]) {
  constexpr int NKB = SB / 32;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    s[kb] = f32x16{};
    dp[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int o = swz128(kb * 32 + n, 2 * ks + hl);
      s[kb] = mfma32(lds_read8(kt + o), qf[ks], s[kb]);
      dp[kb] = mfma32(lds_read8(vt + o), df[ks], dp[kb]);
    }
  }
  const int64_t u0 = (int64_t)sc.j * SB;
  const bool need_mask = u0 + SB - 1 > sc.t || u0 + SB > dm.T;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      float x = s[kb][jj] * cs;
      if (need_mask) {
        const int64_t u = u0 + kb * 32 + 8 * (jj >> 2) + 4 * hl + (jj & 3);
        if (u > sc.t || u >= dm.T) x = -INFINITY;
      }
      s[kb][jj] = x;
    }
}

template <int SB>
__device__ __forceinline__ void sel_load_rows(const bf16* q, const bf16* dout, const SelChunk& sc, int hl,
                                              bf16x8 (&qf)[8], bf16x8 (&df)[8]) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qf[ks] = sc.valid ? *(const bf16x8*)(q + sc.rowi * HD + 16 * ks + 8 * hl) : zero8();
    df[ks] = sc.valid ? *(const bf16x8*)(dout + sc.rowi * HD + 16 * ks + 8 * hl) : zero8();
  }
}

// Per (pair, head): the block's max (log2 units), sum of 2^(x - max) and sum of 2^(x - max) dP.
template <int SB>
__global__ void __launch_bounds__(512)
    bwdf_sel_stats_kernel(const bf16* __restrict__ q, const bf16* __restrict__ dout, const bf16* __restrict__ k,
                          const bf16* __restrict__ v, SlcPairLists pl, float4* __restrict__ rec, Dims dm) {
  constexpr int NKB = SB / 32;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* kt = (bf16*)smem;
  bf16* vt = kt + SB * HD;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, n = l & 31;
  SelChunk sc;
  if (!sel_chunk_setup(pl, dm, w, n, sc)) return;
  const int64_t stride = (int64_t)dm.Hkv * HD;
  const int64_t kvb = (sc.b * dm.T * dm.Hkv + sc.g) * (int64_t)HD;
  stage_rows_bw<SB>(kt, k + kvb, stride, (int64_t)sc.j * SB, dm.T, w, dm.G, l);
  stage_rows_bw<SB>(vt, v + kvb, stride, (int64_t)sc.j * SB, dm.T, w, dm.G, l);
  bf16x8 qf[8], df[8];
  sel_load_rows<SB>(q, dout, sc, hl, qf, df);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x16 s[NKB], dp[NKB];
  sel_scores<SB>(kt, vt, qf, df, sc, dm, n, hl, dm.scale * LOG2E_F, s, dp);
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, s[kb][jj]);
  mx = fmaxf(mx, swap_halves(mx, hl));
  const float mref = mx == -INFINITY ? 0.f : mx;
  float ls = 0.f, es = 0.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const float p = fexp2(s[kb][jj] - mref);
      ls += p;
      es = fmaf(p, dp[kb][jj], es);
    }
  ls += swap_halves(ls, hl);
  es += swap_halves(es, hl);
  if (sc.valid && hl == 0)
    rec[(((sc.b * dm.Tq + sc.row) * dm.Hkv + sc.g) * dm.n + sc.slot) * dm.G + w] = make_float4(mx, ls, es, 0.f);
}

// One thread per (batch, row, head): the selection branch's log-sum-exp (log2 units) and E over the
// row's kept slots; d gates slot 1.  Text rows and rows with no kept slot: no keys.
__global__ void __launch_bounds__(256)
    bwdf_sel_merge_kernel(const float4* __restrict__ rec, const int32_t* __restrict__ idx,
                          const uint8_t* __restrict__ vid, float* __restrict__ st_l, float* __restrict__ st_e,
                          float* __restrict__ dgates, Dims dm) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= dm.B * dm.Tq * dm.Hq) return;
  const int64_t br = x / dm.Hq;
  const int h = (int)(x % dm.Hq), g = h / dm.G, w = h % dm.G;
  const int64_t jt = (dm.q0 + br % dm.Tq) / dm.ls;
  const bool isv = vid ? vid[br] != 0 : true;
  const int32_t* sel = idx + (br * dm.Hkv + g) * dm.n;
  const float4* rr = rec + (br * dm.Hkv + g) * dm.n * dm.G + w;
  float M = -INFINITY;
  if (isv)
    for (int s = 0; s < dm.n; ++s) {
      const int j = sel[s];
      if (j >= 0 && j <= jt) M = fmaxf(M, rr[s * dm.G].x);
    }
  float ls = 0.f, es = 0.f;
  if (M > -INFINITY)
    for (int s = 0; s < dm.n; ++s) {
      const int j = sel[s];
      if (j >= 0 && j <= jt) {
        const float4 r4 = rr[s * dm.G];
        const float a = fexp2(r4.x - M);
        ls = fmaf(a, r4.y, ls);
        es = fmaf(a, r4.z, es);
      }
    }
  const bool has = ls > 0.f;
  const float E = has ? es / ls : 0.f;
  st_l[x * 3 + 1] = has ? M + log2f(ls) : INFINITY;
  st_e[x * 3 + 1] = E;
  dgates[x * 3 + 1] = isv ? E : 0.f;
}

// dq[row, head] += the records of the row's kept slots, in slot order: a thread per 4 channels.
__global__ void __launch_bounds__(256)
    bwdf_sel_dq_merge_kernel(const float* __restrict__ dqrec, const int32_t* __restrict__ idx,
                             const uint8_t* __restrict__ vid, float* __restrict__ dq, Dims dm) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= dm.B * dm.Tq * dm.Hq * (HD / 4)) return;
  const int64_t rh = x / (HD / 4);  // (b Tq + row) Hq + head
  const int c4 = (int)(x % (HD / 4));
  const int64_t br = rh / dm.Hq;
  const int h = (int)(rh % dm.Hq), g = h / dm.G, w = h % dm.G;
  if (vid && !vid[br]) return;
  const int64_t jt = (dm.q0 + br % dm.Tq) / dm.ls;
  const int32_t* sel = idx + (br * dm.Hkv + g) * dm.n;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < dm.n; ++s) {
    const int j = sel[s];
    if (j < 0 || j > jt) continue;
    const float4 r = *(const float4*)(dqrec + (((br * dm.Hkv + g) * dm.n + s) * dm.G + w) * HD + 4 * c4);
    acc.x += r.x;
    acc.y += r.y;
    acc.z += r.z;
    acc.w += r.w;
  }
  float4* d = (float4*)(dq + rh * HD + 4 * c4);
  float4 o = *d;
  o.x += acc.x;
  o.y += acc.y;
  o.z += acc.z;
  o.w += acc.w;
  *d = o;
}

// dk, dv of a block's keys and the pairs' dq records: one workgroup per run of up to CPW
// consecutive chunks of the block (the workgroup of the run's first chunk; the others exit), SB / 16
// waves of 16 keys each, the (chunk, head) items one after the other with the pairs' q and d_out
// rows gathered into LDS.  Per item: S = Q K^T with the rows on M (as in the key kernel),
// dv^T += d_out^T (g P), dk^T += Q^T ds; ds goes through LDS ([row][key], high part and remainder)
// so that wave w forms dq^T = K^T ds^T for dims 32 db (db = w, w + NW, .. < 4) over all the block's
// keys, K^T read transposed from the block's key tile; those go to the pairs' fp32 dq records.
// One atomic add per key and channel for dk, dv at the end of the run.
constexpr int CPW = 32;
template <int SB>
constexpr int sel_grad_lds() {
  return (2 * 2 * PRC * HD + SB * HD + 2 * 2 * PRC * (SB + 8)) * 2;
}
template <int SB>
__global__ void __launch_bounds__(512)
    bwdf_sel_grad_kernel(const bf16* __restrict__ q, const bf16* __restrict__ dout, const bf16* __restrict__ k,
                         const bf16* __restrict__ v, const float* __restrict__ gates, const float* __restrict__ st_l,
                         const float* __restrict__ st_e, SlcPairLists pl, float* __restrict__ dk,
                         float* __restrict__ dv, float* __restrict__ dqrec, Dims dm) {
  constexpr int NW = SB / 16;
  constexpr int DSW = SB + 8;  // row stride of the ds tiles (elements; 16 bytes of padding)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* tq = (bf16*)smem;             // [2][PRC][HD] swizzled
  bf16* tdo = tq + 2 * PRC * HD;      // [2][PRC][HD] swizzled
  bf16* tk = tdo + 2 * PRC * HD;      // [SB][HD] swizzled: the block's keys
  bf16* tds = tk + SB * HD;           // [2 items][2 parts][PRC][DSW]
  __shared__ __attribute__((aligned(16))) float sL[2][PRC], sE[2][PRC], sG[2][PRC];
  __shared__ __attribute__((aligned(16))) int sT[2][PRC];
  __shared__ int sPr[CPW * PRC];  // the run's pairs
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, gi = l >> 4;
  const int hl = l >> 5, n32 = l & 31, g16 = l >> 4, i16 = l & 15;
  const int bg = blockIdx.x / pl.cap_c, cc = blockIdx.x % pl.cap_c;
  const int64_t ci = (int64_t)bg * pl.cap_c + cc;
  const int j = pl.chunk_blk[ci];
  if (j < 0) return;
  const int64_t b = bg / dm.Hkv;
  const int g = bg % dm.Hkv;
  const int G = dm.G;
  if ((cc - pl.cfirst[(int64_t)bg * dm.Ns + j]) % CPW != 0) return;
  int nchk = 1;
  while (nchk < CPW && cc + nchk < pl.cap_c && pl.chunk_blk[ci + nchk] == j) ++nchk;
  const int nitems = nchk * G;
  for (int x = tid; x < nchk * PRC; x += NW * 64) sPr[x] = pl.pairs[ci * PRC + x];
  const int64_t u = (int64_t)j * SB + 16 * w + c;
  const bool uvalid = u < dm.T;
  const int64_t kvb = (b * dm.T * dm.Hkv + g) * (int64_t)HD;
  stage_rows_bw<SB>(tk, k + kvb, (int64_t)dm.Hkv * HD, (int64_t)j * SB, dm.T, w, NW, l);
  __syncthreads();  // sPr
  bf16x8 kf[4], vf[4];
  {
    const int64_t o = kvb + (uvalid ? u : dm.T - 1) * dm.Hkv * (int64_t)HD + 8 * gi;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kf[ks] = *(const bf16x8*)(k + o + 32 * ks);
      vf[ks] = *(const bf16x8*)(v + o + 32 * ks);
    }
  }
  // item i: chunk ci + i / G, head g G + i % G.  Gathered rows: instruction ins fills LDS chunks
  // [64 ins, +64) = pair rows 4 ins .. 4 ins + 3 (an empty pair reads row 0, masked).
  auto stage = [&](int buf, int i) {
    const int* prs = sPr + (i / G) * PRC;
    const int hq = g * G + i % G;
    for (int ins = w; ins < PRC / 4; ins += NW) {
      const int p = ins * 64 + l;
      const int pr = p >> 4, cpos = p & 15, cl = cpos ^ (pr & 15);
      const int pw = prs[pr];
      const int64_t rw = pw >= 0 ? (pw >> 5) : 0;
      const int64_t o = ((b * dm.Tq + rw) * dm.Hq + hq) * (int64_t)HD + cl * 8;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(q + o),
                                       (__attribute__((address_space(3))) void*)(tq + buf * PRC * HD + ins * 512),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(dout + o),
                                       (__attribute__((address_space(3))) void*)(tdo + buf * PRC * HD + ins * 512),
                                       16, 0, 0);
    }
  };
  struct PairSt {
    float L, E, G;
    int t;
  };
  // statistics of pair tid (tid < PRC) of item i
  auto load_st = [&](int i) -> PairSt {
    PairSt st{INFINITY, 0.f, 0.f, -1};
    const int pw = sPr[(i / G) * PRC + tid];
    if (pw >= 0) {
      const int64_t row = pw >> 5;
      const int64_t ri = (b * dm.Tq + row) * dm.Hq + g * G + i % G;
      st.L = st_l[ri * 3 + 1];
      st.E = st_e[ri * 3 + 1];
      st.G = gates[ri * 3 + 1];
      st.t = (int)(dm.q0 + row);
    }
    return st;
  };
  auto put_st = [&](int buf, const PairSt& st) {
    sL[buf][tid] = st.L;
    sE[buf][tid] = st.E;
    sG[buf][tid] = st.G;
    sT[buf][tid] = st.t;
  };
  const float cs = dm.scale * LOG2E_F;
  f32x4 dka[8], dva[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) dka[db] = dva[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  stage(0, 0);
  if (tid < PRC) put_st(0, load_st(0));
  for (int i = 0; i < nitems; ++i) {
    const int buf = i & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    PairSt nst{};
    if (i + 1 < nitems) {
      stage(buf ^ 1, i + 1);
      if (tid < PRC) nst = load_st(i + 1);
    }
    const int pw = sPr[(i / G) * PRC + n32];  // the pair of row n32 of the item (dq records)
    const bf16* Qt = tq + buf * PRC * HD;
    const bf16* Dt = tdo + buf * PRC * HD;
    f32x4 S[2], P[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) S[mb] = P[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int o = swz128(16 * mb + c, 4 * ks + gi);
        S[mb] = mfma16(lds_read8(Qt + o), kf[ks], S[mb]);
        P[mb] = mfma16(lds_read8(Dt + o), vf[ks], P[mb]);
      }
    bf16x8 ph, pl2, sh, sl;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int rq = 16 * mb + 4 * gi;
      const float4 L4 = *(const float4*)&sL[buf][rq];
      const float4 E4 = *(const float4*)&sE[buf][rq];
      const float4 G4 = *(const float4*)&sG[buf][rq];
      const int4 T4 = *(const int4*)&sT[buf][rq];
      const float Lv[4] = {L4.x, L4.y, L4.z, L4.w}, Ev[4] = {E4.x, E4.y, E4.z, E4.w};
      const float Gv[4] = {G4.x, G4.y, G4.z, G4.w};
      const int Tv[4] = {T4.x, T4.y, T4.z, T4.w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float p = fexp2(fmaf(S[mb][jj], cs, -Lv[jj]));
        if (!(uvalid && u <= (int64_t)Tv[jj])) p = 0.f;
        const float gp = Gv[jj] * p;
        split2(gp, ph, pl2, 4 * mb + jj);
        split2(gp * (P[mb][jj] - Ev[jj]), sh, sl, 4 * mb + jj);
      }
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const bf16x8 ad = tr_a16(Dt, 0, db, c, gi);
      dva[db] = mfma16(ad, ph, dva[db]);
      dva[db] = mfma16(ad, pl2, dva[db]);
      const bf16x8 aq = tr_a16(Qt, 0, db, c, gi);
      dka[db] = mfma16(aq, sh, dka[db]);
      dka[db] = mfma16(aq, sl, dka[db]);
    }
    // ds of this wave's 16 keys into the item's [row][key] tiles (rows 16 mb + 4 gi + jj, key 16 w + c)
    bf16* dsh = tds + (size_t)buf * 2 * PRC * DSW;
    bf16* dsl = dsh + PRC * DSW;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int o = (16 * mb + 4 * gi + jj) * DSW + 16 * w + c;
        dsh[o] = sh[4 * mb + jj];
        dsl[o] = sl[4 * mb + jj];
      }
    __syncthreads();
    // dq^T (dims 32 db + l % 32, the item's 32 rows) = K^T ds^T over the block's keys
    for (int db = w; db < 4; db += NW) {
      f32x16 dqa = {};
#pragma unroll
      for (int ks = 0; ks < SB / 16; ++ks) {
        const int r0 = 16 * ks + 8 * hl + (i16 >> 2);
        const int col = 32 * db + 16 * (g16 & 1) + 4 * (i16 & 3);
        const bf16x8 a = cat(lds_read_tr(tk + swz128(r0, col >> 3) + (col & 7)),
                             lds_read_tr(tk + swz128(r0 + 4, col >> 3) + (col & 7)));
        const int ob = n32 * DSW + 16 * ks + 8 * hl;
        dqa = mfma32(a, *(const bf16x8*)(dsh + ob), dqa);
        dqa = mfma32(a, *(const bf16x8*)(dsl + ob), dqa);
      }
      // register jj holds dim 32 db + 8 (jj / 4) + 4 hl + jj % 4 of row n32
      if (pw >= 0) {
        float* dst = dqrec + (((((b * dm.Tq + (pw >> 5)) * dm.Hkv + g) * dm.n + (pw & 31)) * G + i % G) * HD) +
                     32 * db + 4 * hl;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *(float4*)(dst + 8 * qd) = make_float4(dqa[4 * qd] * dm.scale, dqa[4 * qd + 1] * dm.scale,
                                                 dqa[4 * qd + 2] * dm.scale, dqa[4 * qd + 3] * dm.scale);
      }
    }
    if (i + 1 < nitems && tid < PRC) put_st(buf ^ 1, nst);
  }
  if (!uvalid) return;
  float* dkp = dk + ((b * dm.T + u) * dm.Hkv + g) * (int64_t)HD + 4 * gi;
  float* dvp = dv + ((b * dm.T + u) * dm.Hkv + g) * (int64_t)HD + 4 * gi;
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      unsafeAtomicAdd(dkp + 16 * db + jj, dka[db][jj] * dm.scale);
      unsafeAtomicAdd(dvp + 16 * db + jj, dva[db][jj]);
    }
}

// ---------------------------------------------------------------------------
bool bwd_fast_supported(int32_t dtype, const Dims& dm) {
  if (dtype != 1 || dm.D != HD || dm.G < 1 || dm.G > 8 || dm.n < 0 || dm.n > 32) return false;
  if (dm.ls != 32 && dm.ls != 64 && dm.ls != 128) return false;
  return dm.T < (1ll << 31) - 2 * KT && dm.Tq < (1ll << 26) && dm.w >= 1;
}

static size_t frup(size_t x) { return (x + 255) & ~(size_t)255; }

namespace {
struct BwdWs {
  bf16 *kch, *kcl, *vch, *vcl;
  float *dkc, *dvc, *st_l, *st_e;
  uint32_t* tbits;
  float4* rec;
  float* dqrec;
  void* buckets;
  size_t total;
};
}  // namespace

// The selection branch runs per sub-problem: one sequence and a run of at most sel_rows(dm) rows,
// so that its per-(row, slot, head) dq records (512 bytes each) stay within kSelRecCap bytes.
constexpr size_t kSelRecCap = (size_t)2 << 30;
static int64_t sel_rows(const Dims& dm) {
  const size_t per_row = (size_t)dm.Hkv * (dm.n > 0 ? dm.n : 1) * dm.G * HD * 4;
  int64_t rc = (int64_t)(kSelRecCap / per_row);
  if (rc < 32) rc = 32;
  return rc < dm.Tq ? rc : dm.Tq;
}
static Dims sel_dims(const Dims& dm, int64_t rows, int64_t r0) {
  Dims d = dm;
  d.B = 1;
  d.Tq = rows;
  d.q0 = dm.q0 + r0;
  return d;
}

static BwdWs bwd_fast_carve(const Dims& dm, void* ws) {
  BwdWs w{};
  char* p = (char*)ws;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    char* r = p ? p + o : nullptr;
    o += frup(bytes);
    return r;
  };
  const size_t nc = (size_t)dm.B * dm.Nc * dm.Hkv * HD;
  w.kch = (bf16*)take(nc * 2);
  w.kcl = (bf16*)take(nc * 2);
  w.vch = (bf16*)take(nc * 2);
  w.vcl = (bf16*)take(nc * 2);
  w.dkc = (float*)take(nc * 4);
  w.dvc = (float*)take(nc * 4);
  const size_t rows = (size_t)dm.B * dm.Tq * dm.Hq * 3;
  w.st_l = (float*)take(rows * 4);
  w.st_e = (float*)take(rows * 4);
  w.tbits = (uint32_t*)take((size_t)dm.B * ((dm.Tq + 31) / 32) * 4);
  const Dims ds = sel_dims(dm, sel_rows(dm), 0);
  w.rec = (float4*)take((size_t)ds.Tq * ds.Hkv * ds.n * ds.G * 16);
  w.dqrec = (float*)take((size_t)ds.Tq * ds.Hkv * ds.n * ds.G * HD * 4);
  w.buckets = take(slc_bucket_bytes(ds));
  w.total = o;
  return w;
}

size_t bwd_fast_workspace(const Dims& dm) { return bwd_fast_carve(dm, nullptr).total; }

static void zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  bwdf_zero_kernel<<<dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0, s>>>(p, n);
}

// Selection arrays of one sub-problem (its rows' offsets applied).
struct SelArgs {
  const bf16 *q, *dout, *k, *v;
  const float* gates;
  const int32_t* idx;
  const uint8_t* vid;
  float *st_l, *st_e, *dgates, *dq, *dk, *dv;
  float4* rec;
  float* dqrec;
};

template <int SB>
static hipError_t launch_sel_bwd(const Dims& ds, const SlcPairLists& pl, const SelArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)(ds.B * ds.Hkv) * (unsigned)pl.cap_c;
  const int shm = 2 * SB * HD * 2;
  constexpr int shg = sel_grad_lds<SB>();
  hipError_t e = hipFuncSetAttribute((const void*)bwdf_sel_stats_kernel<SB>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, shm);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)bwdf_sel_grad_kernel<SB>, hipFuncAttributeMaxDynamicSharedMemorySize, shg);
  if (e != hipSuccess) return e;
  bwdf_sel_stats_kernel<SB><<<dim3(grid), dim3(ds.G * 64), shm, s>>>(a.q, a.dout, a.k, a.v, pl, a.rec, ds);
  const int64_t nrh = ds.B * ds.Tq * ds.Hq;
  bwdf_sel_merge_kernel<<<dim3((unsigned)((nrh + 255) / 256)), dim3(256), 0, s>>>(a.rec, a.idx, a.vid, a.st_l,
                                                                                  a.st_e, a.dgates, ds);
  bwdf_sel_grad_kernel<SB><<<dim3(grid), dim3(SB / 16 * 64), shg, s>>>(a.q, a.dout, a.k, a.v, a.gates, a.st_l,
                                                                         a.st_e, pl, a.dk, a.dv, a.dqrec, ds);
  const int64_t nth = ds.B * ds.Tq * ds.Hq * (HD / 4);
  bwdf_sel_dq_merge_kernel<<<dim3((unsigned)((nth + 255) / 256)), dim3(256), 0, s>>>(a.dqrec, a.idx, a.vid, a.dq,
                                                                                    ds);
  return hipGetLastError();
}

// The selection branch of every (sequence, run of rows) sub-problem: pair lists, statistics (slot 1
// and d gates), dq, dk, dv.
static hipError_t launch_sel_all(const Dims& dm, const bf16* q, const bf16* dout, const bf16* k, const bf16* v,
                                 const float* gates, const int32_t* idx, const uint8_t* vid, const BwdWs& w,
                                 float* dq, float* dk, float* dv, float* dgates, hipStream_t s) {
  const int64_t rc = sel_rows(dm);
  for (int64_t b = 0; b < dm.B; ++b)
    for (int64_t ra = 0; ra < dm.Tq; ra += rc) {
      const Dims ds = sel_dims(dm, rc < dm.Tq - ra ? rc : dm.Tq - ra, ra);
      const int64_t row0 = b * dm.Tq + ra;  // the sub-problem's first (sequence, row)
      SelArgs a;
      a.q = q + row0 * dm.Hq * HD;
      a.dout = dout + row0 * dm.Hq * HD;
      a.k = k + b * dm.T * dm.Hkv * HD;
      a.v = v + b * dm.T * dm.Hkv * HD;
      a.gates = gates + row0 * dm.Hq * 3;
      a.idx = idx + row0 * dm.Hkv * dm.n;
      a.vid = vid ? vid + row0 : nullptr;
      a.st_l = w.st_l + row0 * dm.Hq * 3;
      a.st_e = w.st_e + row0 * dm.Hq * 3;
      a.dgates = dgates + row0 * dm.Hq * 3;
      a.dq = dq + row0 * dm.Hq * HD;
      a.dk = dk + b * dm.T * dm.Hkv * HD;
      a.dv = dv + b * dm.T * dm.Hkv * HD;
      a.rec = w.rec;
      a.dqrec = w.dqrec;
      hipError_t e;
      if (ds.n <= 0) {
        const int64_t nrh = ds.Tq * ds.Hq;
        bwdf_sel_merge_kernel<<<dim3((unsigned)((nrh + 255) / 256)), dim3(256), 0, s>>>(a.rec, a.idx, a.vid, a.st_l,
                                                                                        a.st_e, a.dgates, ds);
        e = hipGetLastError();
      } else {
        SlcPairLists pl{};
        e = launch_slc_pair_lists(ds, a.idx, a.vid, w.buckets, &pl, s);
        if (e == hipSuccess)
          e = ds.ls == 32 ? launch_sel_bwd<32>(ds, pl, a, s)
                          : ds.ls == 128 ? launch_sel_bwd<128>(ds, pl, a, s) : launch_sel_bwd<64>(ds, pl, a, s);
      }
      if (e != hipSuccess) return e;
    }
  return hipSuccess;
}

hipError_t launch_layer_bwd_fast(const Dims& dm, const void* q_, const void* k_, const void* v_, const float* w_k,
                                 const float* w_v, const float* gates, const uint8_t* vid, const int32_t* idx,
                                 const void* dout_, float* dq, float* dk, float* dv, float* dgates, float* dw_k,
                                 float* dw_v, void* ws, hipStream_t s) {
  if (dm.B <= 0 || dm.Tq <= 0) return hipSuccess;
  const bf16* q = (const bf16*)q_;
  const bf16* k = (const bf16*)k_;
  const bf16* v = (const bf16*)v_;
  const bf16* dout = (const bf16*)dout_;
  const BwdWs w = bwd_fast_carve(dm, ws);
  hipError_t e = hipSuccess;
  const int64_t nkv = dm.B * dm.T * dm.Hkv * HD, nc = dm.B * dm.Nc * dm.Hkv * HD;
  zero_f32(dk, nkv, s);
  zero_f32(dv, nkv, s);
  zero_f32(w.dkc, nc, s);
  zero_f32(w.dvc, nc, s);
  if (dm.Nc > 0) {
    e = launch_compress(1, 2, k, w_k, w.kch, w.kcl, dm.B, dm.T, dm.Hkv, HD, dm.l, dm.d, dm.Nc, s);
    if (e == hipSuccess) e = launch_compress(1, 2, v, w_v, w.vch, w.vcl, dm.B, dm.T, dm.Hkv, HD, dm.l, dm.d, dm.Nc, s);
    if (e != hipSuccess) return e;
  }
  const int64_t ntr = (dm.Tq + 31) / 32;
  bwdf_tbits_kernel<<<dim3((unsigned)((dm.B * ntr + 255) / 256)), dim3(256), 0, s>>>(vid, w.tbits, dm);
  // row kernels: the compression branch first (it writes dq), then the window / text rows
  {
    const dim3 grid(xcd_grid((int)(dm.B * dm.Hkv), (int)((dm.Tq + RT - 1) / RT)));
    const int shc = 4 * 2 * KT * HD * 2, shw = 2 * 2 * KT * HD * 2;
    e = hipFuncSetAttribute((const void*)bwdf_row_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, shc);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)bwdf_row_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize, shw);
    if (e != hipSuccess) return e;
    bwdf_row_kernel<true><<<grid, dim3(dm.G * 64), shc, s>>>(q, dout, w.kch, w.kcl, w.vch, w.vcl, vid, gates, dq,
                                                             dgates, w.st_l, w.st_e, dm);
    bwdf_row_kernel<false><<<grid, dim3(dm.G * 64), shw, s>>>(q, dout, k, nullptr, v, nullptr, vid, gates, dq,
                                                              dgates, w.st_l, w.st_e, dm);
  }
  // selection branch (after the row kernels: its dq merge adds to their dq)
  e = launch_sel_all(dm, q, dout, k, v, gates, idx, vid, w, dq, dk, dv, dgates, s);
  if (e != hipSuccess) return e;
  // key kernels: window / text rows over the full-resolution keys, compression over the compressed ones
  {
    const int nchw = (int)((ntr + RTC_WIN - 1) / RTC_WIN);
    const dim3 gw(xcd_grid((int)(dm.B * dm.Hkv), (int)(((dm.T + KT - 1) / KT) * nchw)));
    bwdf_key_kernel<false><<<gw, dim3(256), 0, s>>>(q, dout, k, nullptr, v, nullptr, vid, gates, w.st_l, w.st_e,
                                                    w.tbits, dk, dv, dm, nchw);
    if (dm.Nc > 0) {
      const int nchc = (int)((ntr + RTC_CMP - 1) / RTC_CMP);
      const dim3 gc(xcd_grid((int)(dm.B * dm.Hkv), (int)(((dm.Nc + KT - 1) / KT) * nchc)));
      bwdf_key_kernel<true><<<gc, dim3(256), 0, s>>>(q, dout, w.kch, w.kcl, w.vch, w.vcl, vid, gates, w.st_l,
                                                     w.st_e, w.tbits, w.dkc, w.dvc, dm, nchc);
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_bwd_compress_grads(1, dm, w.dkc, w.dvc, w_k, w_v, k, v, dk, dv, dw_k, dw_v, s);
}
