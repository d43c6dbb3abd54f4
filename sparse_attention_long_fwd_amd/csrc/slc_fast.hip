// Selection branch with the gated combine, bf16 MFMA on gfx950.
//
// Selection (top168.com digest of VideoNSA, section 一; csdn page
// "VideoNSA：重新定义视频理解的稀疏注意力机制", section 2.2): a video row t attends
// at full resolution to the tokens u <= t of the blocks chosen for its KV group.
// Gated combine (same digest, section 一; csdn page, section 3.1): the three
// branch outputs are mixed per head with the given gate values,
//   out = g_cmp o_cmp + g_slc o_slc + g_swa o_swa.
//
// Every row has its own blocks, so the work unit is one (row, KV group): one
// wave gathers the row's blocks and serves all G query heads of the group from
// each block it loads (the heads share the KV head).  Scores are S^T = K Q^T
// with v_mfma_f32_16x16x32_bf16: 16 keys on M, the G heads (padded to 16) on
// N.  K fragments are read from global memory straight into A layout; V
// blocks go global -> LDS (one 16 KB tile per wave, XOR-swizzled rows) and
// come back transposed through ds_read_b64_tr_b16.  The next block's K is in
// flight while the current block's softmax and value product run.
//
// The kernel is bound by the gather of 64-token blocks: 32 KB of K and V per
// block, read once per (row, group).
#include "fast_common.hpp"

namespace {
constexpr int SW = 4;     // waves (rows) per workgroup
constexpr int HD = 128;
constexpr int SB = 64;    // selection block
constexpr float RESCALE_SLACK = 8.f;
}  // namespace

__device__ __forceinline__ void swait_all() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void swait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <bool OCMP_F32>
__global__ void __launch_bounds__(SW * 64) slc_fast_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                           const bf16* __restrict__ v, const int32_t* __restrict__ idx,
                                                           const uint8_t* __restrict__ vid,
                                                           const void* __restrict__ ocmp, const float* __restrict__ swa,
                                                           const float* __restrict__ gates, bf16* __restrict__ out,
                                                           bf16* __restrict__ o_slc, Dims dm, int nwg_per_unit,
                                                           int64_t tok_stride, int64_t head_stride, int group_seq) {
  __shared__ __attribute__((aligned(16))) bf16 vtile[SW][SB * HD];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int hn = l & 15, grp = l >> 4;  // head column, lane group (4 keys each)
  int unit, rank;
  if (group_seq) {  // one (batch, group) after another: its K/V is the whole working set
    unit = (int)(blockIdx.x / (unsigned)nwg_per_unit);
    rank = (int)(blockIdx.x % (unsigned)nwg_per_unit);
  } else if (!xcd_remap(blockIdx.x, (int)(dm.B * dm.Hkv), nwg_per_unit, &unit, &rank)) {
    return;
  }
  const int64_t b = unit / dm.Hkv;
  const int g = unit % dm.Hkv;
  const int64_t r = (int64_t)rank * SW + w;
  if (r >= dm.Tq) return;
  if (vid && !vid[b * dm.Tq + r]) return;
  const int G = dm.G;
  const int64_t t = dm.q0 + r;
  const int64_t jt = t / SB;
  const float c2 = dm.scale * LOG2E_F;
  const bool hvalid = hn < G;
  const int h = g * G + (hvalid ? hn : 0);

  // Q^T as the B operand: lane holds Q[head hn][32 ks + 8 grp .. +8]
  bf16x8 qf[4];
  {
    const bf16* qrow = q + ((b * dm.Tq + r) * dm.Hq + h) * (int64_t)HD + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = hvalid ? *(const bf16x8*)(qrow + 32 * ks) : zero8();
  }
  const int32_t* sel = idx + ((b * dm.Tq + r) * dm.Hkv + g) * dm.n;
  const int myj = l < dm.n ? sel[l] : -1;
  const int64_t stride = tok_stride;
  const bf16* kbase = k + b * dm.T * dm.Hkv * (int64_t)HD + g * head_stride;
  const bf16* vbase = v + b * dm.T * dm.Hkv * (int64_t)HD + g * head_stride;
  bf16* vt = vtile[w];

  // K fragments of one block: A operand of S^T, lane holds K[16 kb + hn][32 ks + 8 grp .. +8]
  bf16x8 kf[4][4];
  auto load_k = [&](int64_t j) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      int64_t key = j * SB + 16 * kb + hn;
      if (key >= dm.T) key = dm.T - 1;
      const bf16* kr = kbase + key * stride + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[kb][ks] = *(const bf16x8*)(kr + 32 * ks);
    }
  };

  // the chosen blocks that hold tokens <= t, in order
  int next_c = 0;
  auto next_block = [&](int& c) -> int64_t {
    for (; c < dm.n; ++c) {
      const int j = __shfl(myj, c, 64);
      if (j >= 0 && j <= jt) return (int64_t)j;
    }
    return -1;
  };
  int64_t j = next_block(next_c);
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{};
  if (j >= 0) {
    load_k(j);
    stage_tile64(vt, vbase, stride, j * SB, dm.T, 0, 1, l);
  }
  while (j >= 0) {
    swait_all();
    __builtin_amdgcn_wave_barrier();
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) s[kb] = mfma16(kf[kb][ks], qf[ks], s[kb]);
    }
    ++next_c;
    const int64_t jn = next_block(next_c);
    if (jn >= 0) load_k(jn);  // overlaps the softmax and value product below
    float x[16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int64_t key = j * SB + 16 * kb + 4 * grp + jj;
        x[4 * kb + jj] = key <= t ? s[kb][jj] * c2 : -INFINITY;
      }
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (mx > m_run + RESCALE_SLACK) {
      const float corr = fexp2(m_run - mx);
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[db][e] *= corr;
      m_run = mx;
    }
    float p[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = fexp2(x[e] - m_run);
      l_run += p[e];
    }
    // O^T += V^T P^T: 32-key steps, key(kappa) = 32 st + (r < 4 ? 4 grp + r : 16 + 4 grp + r - 4)
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
        const bf16x4 a0 = lds_read_tr(vt + swz128(vr, col >> 3) + (col & 7));
        const bf16x4 a1 = lds_read_tr(vt + swz128(vr + 16, col >> 3) + (col & 7));
        oacc[db] = mfma16(cat(a0, a1), pb, oacc[db]);
      }
    }
    j = jn;
    if (j >= 0) {
      swait_lds();  // the transposing reads of this tile are complete
      __builtin_amdgcn_wave_barrier();
      stage_tile64(vt, vbase, stride, j * SB, dm.T, 0, 1, l);
    }
  }
  float lt = l_run + __shfl_xor(l_run, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (!hvalid) return;
  const int64_t orow = ((b * dm.Tq + r) * dm.Hq + h) * (int64_t)HD;
  const float* gg = gates ? gates + ((b * dm.Tq + r) * dm.Hq + h) * 3 : nullptr;
  const float g0 = gg ? gg[0] : 0.f, g1 = gg ? gg[1] : 0.f, g2 = gg ? gg[2] : 0.f;
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const int d0 = 16 * db + 4 * grp;
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = oacc[db][e] * inv;
    if (o_slc) {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (bf16)o[e];
      *(bf16x4*)(o_slc + orow + d0) = v4;
    }
    if (out) {
      float oc[4];
      if constexpr (OCMP_F32) {
        const float4 c4 = *(const float4*)((const float*)ocmp + orow + d0);
        oc[0] = c4.x, oc[1] = c4.y, oc[2] = c4.z, oc[3] = c4.w;
      } else {
        const bf16x4 c4 = *(const bf16x4*)((const bf16*)ocmp + orow + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) oc[e] = (float)c4[e];
      }
      const float4 s4 = *(const float4*)(swa + orow + d0);
      const float sw[4] = {s4.x, s4.y, s4.z, s4.w};
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (bf16)(g0 * oc[e] + g1 * o[e] + g2 * sw[e]);
      *(bf16x4*)(out + orow + d0) = v4;
    }
  }
}

// head_major: k/v are laid out [B, Hkv, T, D] instead of [B, T, Hkv, D].
hipError_t launch_slc_fast(const Dims& dm, const void* q, const void* k, const void* v, const int32_t* idx,
                           const uint8_t* vid, const void* ocmp, bool ocmp_f32, const float* swa32,
                           const float* gates, void* out, void* o_slc, hipStream_t s, bool head_major,
                           bool group_seq) {
  if (dm.Tq <= 0 || dm.B <= 0 || (!out && !o_slc)) return hipSuccess;
  const int per_unit = (int)((dm.Tq + SW - 1) / SW);
  const int units = (int)(dm.B * dm.Hkv);
  dim3 grid(group_seq ? (unsigned)(units * per_unit) : xcd_grid(units, per_unit)), block(SW * 64);
  const int64_t tok_stride = head_major ? HD : (int64_t)dm.Hkv * HD;
  const int64_t head_stride = head_major ? dm.T * (int64_t)HD : HD;
  if (ocmp_f32)
    slc_fast_kernel<true><<<grid, block, 0, s>>>((const bf16*)q, (const bf16*)k, (const bf16*)v, idx, vid, ocmp,
                                                 swa32, gates, (bf16*)out, (bf16*)o_slc, dm, per_unit, tok_stride, head_stride,
                                                 group_seq ? 1 : 0);
  else
    slc_fast_kernel<false><<<grid, block, 0, s>>>((const bf16*)q, (const bf16*)k, (const bf16*)v, idx, vid, ocmp,
                                                  swa32, gates, (bf16*)out, (bf16*)o_slc, dm, per_unit, tok_stride, head_stride,
                                                 group_seq ? 1 : 0);
  return hipGetLastError();
}
