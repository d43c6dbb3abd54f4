// Compression-branch attention fused with block importance, bf16 MFMA on gfx950.
//
// What it computes (top168.com digest of VideoNSA, section 一: the selection
// branch scores segments by importance, read here from the compression
// branch's probabilities): for each video row t and head h,
//   p_i = softmax_i(scale * <q_t,h, kc_i>) over the compressed blocks i whose
//         tokens all lie at or before t,  o_cmp = sum_i p_i vc_i,
//   imp[t, g, j] = sum_{h in group g} sum_i frac(i, j) p_{h,i},
// with compressed block 32 / stride 16 and selection block 64, so that block j
// takes compressed blocks 4j .. 4j+2 whole and half of 4j-1 and 4j+3.
//
// Layout on the chip: one workgroup = 32 consecutive query rows x the G heads
// of one KV group, one wave per head.  Scores are formed transposed,
// S^T = Kc Q^T (v_mfma_f32_32x32x16_bf16, keys on M, the wave's 32 rows on N),
// so each lane owns one (row, head) column: its softmax statistics need one
// cross-half exchange, and the score registers are already the B operand of
// O^T += Vc^T P^T after a bf16 conversion.  Vc^T comes from LDS with the
// gfx950 transposing read (ds_read_b64_tr_b16); Kc is read in A layout.
// Compressed K/V tiles of 64 keys go global -> LDS directly (global_load_lds,
// 16 bytes a lane), double-buffered: the next tile streams in while the
// current one is consumed, without staging registers.  LDS rows are 256 bytes
// with their 16-byte chunks XOR-swizzled by the row index, so the A-layout and
// transposing reads of 16 consecutive rows hit distinct banks.
//
// The importance needs the final softmax normaliser, so the kernel makes two
// sweeps over the keys: the first forms the log-sum-exp (Q Kc^T only), the
// second exact probabilities, the value sum and the importance.  Each lane's
// probabilities come in aligned runs of 4 compressed blocks (one selection
// block); the half-block shares cross lanes with one xor-32 shuffle and a
// carry, the G heads are summed in a fixed order through LDS, so the result is
// deterministic.
//
// Compressed K and V may come as bf16 high + low parts (compressed inside the
// layer from an fp32 sum); both parts enter every product, so the compression
// adds no bf16 rounding step to the scores or the value sum.
#include "fast_common.hpp"

namespace {
constexpr int CQ = 32;         // query rows per workgroup
constexpr int CK = 64;         // compressed keys per tile
constexpr int HD = 128;        // head dim
constexpr int TILE = CK * HD;  // bf16 elements of one staged array
}  // namespace

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <bool SPLIT>
__global__ void __launch_bounds__(512) cmp_fast_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kh,
                                                       const bf16* __restrict__ kl, const bf16* __restrict__ vh,
                                                       const bf16* __restrict__ vl, const uint8_t* __restrict__ vid,
                                                       bf16* __restrict__ o_bf, float* __restrict__ o_f32,
                                                       float* __restrict__ lse, float* __restrict__ imp, Dims dm,
                                                       int ntq) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int NARR = SPLIT ? 4 : 2;                   // staged arrays per buffer: K (hi, lo), V (hi, lo)
  bf16* buf0 = (bf16*)smem;                              // buffer b, array a at buf0 + (b * NARR + a) * TILE
  float* ipart = (float*)(smem + 2 * NARR * TILE * 2);  // [2][G][CQ][16]
  __shared__ int s_any;

  const int G = dm.G;
  const int nthr = G * 64;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, hl = l >> 5, n = l & 31;
  int unit, rank;
  if (!xcd_remap(blockIdx.x, (int)(dm.B * dm.Hkv), ntq, &unit, &rank)) return;
  const int64_t b = unit / dm.Hkv;
  const int g = unit % dm.Hkv;
  const int64_t rt0 = (int64_t)(ntq - 1 - rank) * CQ;  // heaviest tiles first

  if (tid == 0) s_any = 0;
  __syncthreads();
  if (tid < CQ) {
    const int64_t r = rt0 + tid;
    if (r < dm.Tq && (!vid || vid[b * dm.Tq + r])) s_any = 1;
  }
  __syncthreads();
  if (!s_any) return;

  const int64_t rlast = (rt0 + CQ < dm.Tq ? rt0 + CQ : dm.Tq) - 1;
  const int64_t nvmax = cmp_visible(dm.q0 + rlast, dm.l, dm.d, dm.Nc);
  const int64_t r = rt0 + n;
  const bool rvalid = r < dm.Tq;
  const bool isv = rvalid && (!vid || vid[b * dm.Tq + r]);
  const int64_t t = dm.q0 + r;
  const int64_t nv = rvalid ? cmp_visible(t, dm.l, dm.d, dm.Nc) : 0;
  const int h = g * G + w;
  const float c2 = dm.scale * LOG2E_F;

  // Q^T as the B operand: lane holds Q[row n][16 ks + 8 hl .. +8]
  bf16x8 qf[8];
  {
    const bf16* qrow = q + ((b * dm.Tq + (rvalid ? r : 0)) * dm.Hq + h) * (int64_t)HD + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = rvalid ? *(const bf16x8*)(qrow + 16 * ks) : zero8();
  }

  const int64_t stride = (int64_t)dm.Hkv * HD;
  const int64_t base = (b * dm.Nc * dm.Hkv + g) * (int64_t)HD;
  auto arr = [&](int bufi, int a) { return buf0 + (bufi * NARR + a) * TILE; };
  auto stage_k = [&](int tile, int bufi) {
    stage_tile64(arr(bufi, 0), kh + base, stride, (int64_t)tile * CK, dm.Nc, w, G, l);
    if constexpr (SPLIT) stage_tile64(arr(bufi, 1), kl + base, stride, (int64_t)tile * CK, dm.Nc, w, G, l);
  };
  auto stage_v = [&](int tile, int bufi) {
    stage_tile64(arr(bufi, SPLIT ? 2 : 1), vh + base, stride, (int64_t)tile * CK, dm.Nc, w, G, l);
    if constexpr (SPLIT) stage_tile64(arr(bufi, 3), vl + base, stride, (int64_t)tile * CK, dm.Nc, w, G, l);
  };
  // S^T block kb (32 keys) of the staged tile
  auto scores = [&](int bufi, int kb) {
    f32x16 s = {};
    const int row = kb * 32 + n;
    const bf16* khs = arr(bufi, 0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int off = swz128(row, 2 * ks + hl);
      s = mfma32(lds_read8(khs + off), qf[ks], s);
      if constexpr (SPLIT) s = mfma32(lds_read8(arr(bufi, 1) + off), qf[ks], s);
    }
    return s;
  };

  // ---- sweep 1: log-sum-exp per (row, head) column, log2 domain
  float m2 = -INFINITY, lsum = 0.f;
  const int nt1 = (int)((nvmax + CK - 1) / CK);
  if (nt1 > 0) {
    stage_k(0, 0);
    wait_loads();
  }
  __syncthreads();
  for (int tile = 0; tile < nt1; ++tile) {
    const int bufi = tile & 1;
    if (tile + 1 < nt1) stage_k(tile + 1, bufi ^ 1);
    float x[32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x16 s = scores(bufi, kb);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t key = (int64_t)tile * CK + kb * 32 + 8 * (j >> 2) + 4 * hl + (j & 3);
        x[kb * 16 + j] = key < nv ? s[j] * c2 : -INFINITY;
      }
    }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) mx = fmaxf(mx, x[j]);
    const float mnew = fmaxf(m2, mx);
    if (mnew > -INFINITY) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) acc += fexp2(x[j] - mnew);
      lsum = lsum * fexp2(m2 - mnew) + acc;
      m2 = mnew;
    }
    wait_loads();
    __syncthreads();
  }
  float L2;
  {
    const float mo = __shfl_xor(m2, 32, 64);
    const float lo = __shfl_xor(lsum, 32, 64);
    const float M = fmaxf(m2, mo);
    if (M > -INFINITY) {
      const float tot = (m2 > -INFINITY ? lsum * fexp2(m2 - M) : 0.f) + (mo > -INFINITY ? lo * fexp2(mo - M) : 0.f);
      L2 = M + flog2(tot);
    } else {
      L2 = INFINITY;  // no visible block: every probability is zero
    }
  }

  // ---- sweep 2: probabilities, value sum, importance
  f32x16 oacc[4] = {};
  float carry = 0.f;  // half share of the previous run's last compressed block (hl == 0 lanes)
  const int nt2 = nvmax > 0 ? (int)(nvmax / CK) + 1 : 0;
  const int g16 = l >> 4, i16 = l & 15;
  if (nt2 > 0) {
    stage_k(0, 0);
    stage_v(0, 0);
    wait_loads();
  }
  __syncthreads();
  for (int tile = 0; tile < nt2; ++tile) {
    const int bufi = tile & 1;
    if (tile + 1 < nt2) {
      stage_k(tile + 1, bufi ^ 1);
      stage_v(tile + 1, bufi ^ 1);
    }
    float* ipb = ipart + bufi * G * CQ * 16;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x16 s = scores(bufi, kb);
      float p[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t key = (int64_t)tile * CK + kb * 32 + 8 * (j >> 2) + 4 * hl + (j & 3);
        p[j] = key < nv ? fexp2(fmaf(s[j], c2, -L2)) : 0.f;
      }
      // importance of the four selection blocks this lane covers in this 32-key run
      float a[4], oth[4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        a[qq] = p[4 * qq] + p[4 * qq + 1] + p[4 * qq + 2] + 0.5f * p[4 * qq + 3];
        oth[qq] = __shfl_xor(0.5f * p[4 * qq + 3], 32, 64);
      }
      if (hl == 0) {
        a[0] += carry;
        a[1] += oth[0];
        a[2] += oth[1];
        a[3] += oth[2];
        carry = oth[3];
      } else {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) a[qq] += oth[qq];
      }
      float* ip = ipb + (w * CQ + n) * 16 + kb * 8 + hl;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) ip[2 * qq] = a[qq];
      // O^T += Vc^T P^T in two 16-key steps
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (bf16)p[8 * st + e];
        const int vr = kb * 32 + 16 * st + 4 * (g16 >> 1) + (i16 >> 2);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int col = 32 * db + (g16 & 1) * 16 + 4 * (i16 & 3);
          const int o0 = swz128(vr, col >> 3) + (col & 7);
          const int o1 = swz128(vr + 8, col >> 3) + (col & 7);
          const bf16* vhs = arr(bufi, SPLIT ? 2 : 1);
          oacc[db] = mfma32(cat(lds_read_tr(vhs + o0), lds_read_tr(vhs + o1)), pb, oacc[db]);
          if constexpr (SPLIT) {
            const bf16* vls = arr(bufi, 3);
            oacc[db] = mfma32(cat(lds_read_tr(vls + o0), lds_read_tr(vls + o1)), pb, oacc[db]);
          }
        }
      }
    }
    wait_loads();
    __syncthreads();
    // sum the group's heads in a fixed order; write the tile's 16 selection blocks
    for (int idx = tid; idx < CQ * 16; idx += nthr) {
      const int nn = idx >> 4, jj = idx & 15;
      const int64_t rr = rt0 + nn;
      if (rr >= dm.Tq || (vid && !vid[b * dm.Tq + rr])) continue;
      const int64_t J = (int64_t)tile * 16 + jj;
      if (J > (dm.q0 + rr) / dm.ls || J >= dm.Ns) continue;
      float sum = 0.f;
      for (int ww = 0; ww < G; ++ww) sum += ipb[(ww * CQ + nn) * 16 + jj];
      imp[((b * dm.Tq + rr) * dm.Hkv + g) * dm.Ns + J] = sum;
    }
  }
  // blocks up to the row's own block that no compressed block reaches
  for (int idx = tid; idx < CQ * 16; idx += nthr) {
    const int nn = idx >> 4, jj = idx & 15;
    const int64_t rr = rt0 + nn;
    if (rr >= dm.Tq || (vid && !vid[b * dm.Tq + rr])) continue;
    const int64_t J = (int64_t)nt2 * 16 + jj;
    if (J <= (dm.q0 + rr) / dm.ls && J < dm.Ns) imp[((b * dm.Tq + rr) * dm.Hkv + g) * dm.Ns + J] = 0.f;
  }

  if (!isv) return;
  const int64_t orow = ((b * dm.Tq + r) * dm.Hq + h) * (int64_t)HD;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = 32 * db + 8 * j4 + 4 * hl;
      if (o_f32)
        *(float4*)(o_f32 + orow + d0) =
            make_float4(oacc[db][4 * j4], oacc[db][4 * j4 + 1], oacc[db][4 * j4 + 2], oacc[db][4 * j4 + 3]);
      if (o_bf) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)oacc[db][4 * j4 + e];
        *(bf16x4*)(o_bf + orow + d0) = v4;
      }
    }
  }
  if (lse && hl == 0) lse[(b * dm.Tq + r) * dm.Hq + h] = nv > 0 ? L2 * LN2_F : -INFINITY;
}

size_t cmp_fast_smem(const Dims& dm, bool split) {
  return (size_t)2 * (split ? 4 : 2) * TILE * 2 + (size_t)2 * dm.G * CQ * 16 * 4;
}

hipError_t launch_cmp_fast(const Dims& dm, const void* q, const void* kh, const void* kl, const void* vh,
                           const void* vl, const uint8_t* vid, void* o, float* o32, float* lse, float* imp,
                           hipStream_t s) {
  if (dm.Tq <= 0 || dm.B <= 0) return hipSuccess;
  const int ntq = (int)((dm.Tq + CQ - 1) / CQ);
  const int units = (int)(dm.B * dm.Hkv);
  dim3 grid(xcd_grid(units, ntq)), block(dm.G * 64);
  const bool split = kl != nullptr;
  const size_t shm = cmp_fast_smem(dm, split);
  hipError_t e;
  if (split) {
    e = hipFuncSetAttribute((const void*)cmp_fast_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    cmp_fast_kernel<true><<<grid, block, shm, s>>>((const bf16*)q, (const bf16*)kh, (const bf16*)kl,
                                                   (const bf16*)vh, (const bf16*)vl, vid, (bf16*)o, o32, lse, imp,
                                                   dm, ntq);
  } else {
    e = hipFuncSetAttribute((const void*)cmp_fast_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)shm);
    if (e != hipSuccess) return e;
    cmp_fast_kernel<false><<<grid, block, shm, s>>>((const bf16*)q, (const bf16*)kh, nullptr, (const bf16*)vh,
                                                    nullptr, vid, (bf16*)o, o32, lse, imp, dm, ntq);
  }
  return hipGetLastError();
}
