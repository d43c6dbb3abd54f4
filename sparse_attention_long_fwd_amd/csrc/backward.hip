// Backward pass of the hybrid layer (generic VALU kernels, gfx950): gradients of
// sum(d_out * out) with respect to q, k, v, the gates and the compression weights.
//
// The forward is the layer of the other kernels (top168.com digest of VideoNSA,
// section 一; csdn page "VideoNSA：重新定义视频理解的稀疏注意力机制", sections 2.2
// and 3.1; shd-paper.top page, English abstract): for video rows out = g_c o_c +
// g_s o_s + g_w o_w over the compression, selection and window branches, for
// text rows dense causal attention.  The chosen blocks are an input and pass no
// gradient.  Per branch b of one (row, head), with P the probabilities over its
// keys and E_b = sum_u P_u <d_out, v_u>:
//   d g_b = E_b,   ds_u = g_b P_u (<d_out, v_u> - E_b),
//   dq += scale sum_u ds_u k_u,   dk_u += scale ds_u q,   dv_u += g_b P_u d_out
// (text rows: one branch, g = 1).  Compressed keys and values are positional
// weighted sums of k, v, so dk[i d + m] += w_k[m] dkc[i] and
// dw_k[m] = sum_i <dkc[i], k[i d + m]> (likewise v).
//
// Three stages, no atomics on the gradients of k and v:
//  1. bwd_row_kernel (one workgroup per (batch, row, KV group)): per head and
//     branch, the log-sum-exp and E_b over the branch's keys, dq and d gates;
//     the statistics go to the workspace.
//  2. bwd_key_kernel (one workgroup per (batch, 32 keys, KV group)): walks the
//     rows that can see its keys and accumulates dk, dv in registers from the
//     stored statistics (window, selection and text rows); bwd_ckey_kernel does
//     the same for 32 compressed keys (dkc, dvc).
//  3. bwd_compress_kernel adds the compression's share to dk, dv;
//     bwd_dw_kernel reduces dw_k, dw_v.
#include "common.hpp"

#define BWD_THREADS 256

namespace {
constexpr int KB = 32;        // keys per workgroup of the key kernels
constexpr int LPK = 8;        // lanes per key
}  // namespace

__device__ __forceinline__ float bwd_block_sum(float x, float* red) { return block_sum(x, red); }

// 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32) widened to float
__device__ __forceinline__ void ld8(const bf16* p, float* f) {
  typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 v8;
  const v8 u = *(const v8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)u[i];
}
__device__ __forceinline__ void ld8(const float* p, float* f) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
// <x, y> over D channels, x in LDS (fp32), y in global memory (8 at a time)
template <typename TK>
__device__ __forceinline__ float dot_lds(const float* x, const TK* y, int D) {
  float acc = 0.f;
  for (int e = 0; e < D; e += 8) {
    float f[8];
    ld8(y + e, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(x[e + i], f[i], acc);
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Stage 1.  Up to HB heads of one KV group at once over one key list, so each key row is read
// once for all of them.  qs, dos: [HB][D] query and upstream gradient (LDS); thread e < D owns
// channel e of dqs [HB][D] (LDS), to which g_h scale (sum P dpv k - E sum P k) is added.  On
// return L[h], E[h] (uniform) are each head's log-sum-exp (-inf for an empty list) and E.
constexpr int HB = 8;

template <typename TK, typename KeyFn>
__device__ void bwd_branch_rows(const float* qs, const float* dos, const TK* kb, const TK* vb, int64_t kstride,
                                int D, int64_t nslots, KeyFn key_of, float scale, const float* gate, int nh,
                                float* dqs, float* ps, float* pds, int64_t* us, float* wred, float* L, float* E) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  float m_run[HB], l_run[HB];
#pragma unroll
  for (int h = 0; h < HB; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
  }
  // reduce x[h] over the workgroup (op: 0 max, 1 sum); uniform result in x
  auto reduce = [&](float* x, int op) {
#pragma unroll
    for (int h = 0; h < HB; ++h) x[h] = op ? wave_sum(x[h]) : wave_max(x[h]);
    __syncthreads();  // earlier readers of wred are done
    if (lane == 0)
#pragma unroll
      for (int h = 0; h < HB; ++h) wred[wv * HB + h] = x[h];
    __syncthreads();
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      float r = wred[h];
      for (int w2 = 1; w2 < BWD_THREADS / 64; ++w2) r = op ? r + wred[w2 * HB + h] : fmaxf(r, wred[w2 * HB + h]);
      x[h] = r;
    }
  };
  // pass A: log-sum-exp per head (online over chunks of 256 slots)
  for (int64_t a0 = 0; a0 < nslots; a0 += BWD_THREADS) {
    const int64_t a = a0 + tid;
    const int64_t u = a < nslots ? key_of(a) : -1;
    float z[HB];
#pragma unroll
    for (int h = 0; h < HB; ++h) z[h] = -INFINITY;
    if (u >= 0) {
      const TK* kr = kb + u * kstride;
      float acc[HB];
#pragma unroll
      for (int h = 0; h < HB; ++h) acc[h] = 0.f;
      for (int e = 0; e < D; e += 8) {
        float f[8];
        ld8(kr + e, f);
#pragma unroll
        for (int h = 0; h < HB; ++h)
          if (h < nh)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[h] = fmaf(qs[h * D + e + i], f[i], acc[h]);
      }
#pragma unroll
      for (int h = 0; h < HB; ++h)
        if (h < nh) z[h] = acc[h] * scale;
    }
    float mx[HB], p[HB];
#pragma unroll
    for (int h = 0; h < HB; ++h) mx[h] = z[h];
    reduce(mx, 0);
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      mx[h] = fmaxf(m_run[h], mx[h]);
      p[h] = (u >= 0 && mx[h] > -INFINITY) ? expf(z[h] - mx[h]) : 0.f;
    }
    reduce(p, 1);
#pragma unroll
    for (int h = 0; h < HB; ++h)
      if (mx[h] > -INFINITY) {
        l_run[h] = (m_run[h] == -INFINITY ? 0.f : l_run[h] * expf(m_run[h] - mx[h])) + p[h];
        m_run[h] = mx[h];
      }
  }
#pragma unroll
  for (int h = 0; h < HB; ++h) {
    L[h] = l_run[h] > 0.f ? m_run[h] + logf(l_run[h]) : -INFINITY;
    E[h] = 0.f;
  }
  // pass B: E = sum P dpv, and per channel A1 = sum P dpv k, A2 = sum P k
  float a1[HB], a2[HB];
#pragma unroll
  for (int h = 0; h < HB; ++h) a1[h] = a2[h] = 0.f;
  for (int64_t a0 = 0; a0 < nslots; a0 += BWD_THREADS) {
    const int64_t a = a0 + tid;
    const int64_t u = a < nslots ? key_of(a) : -1;
    float p[HB], pd[HB];
#pragma unroll
    for (int h = 0; h < HB; ++h) p[h] = pd[h] = 0.f;
    if (u >= 0) {
      const TK* kr = kb + u * kstride;
      const TK* vr = vb + u * kstride;
      float aq[HB], ad[HB];
#pragma unroll
      for (int h = 0; h < HB; ++h) aq[h] = ad[h] = 0.f;
      for (int e = 0; e < D; e += 8) {
        float fk[8], fv[8];
        ld8(kr + e, fk);
        ld8(vr + e, fv);
#pragma unroll
        for (int h = 0; h < HB; ++h)
          if (h < nh)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              aq[h] = fmaf(qs[h * D + e + i], fk[i], aq[h]);
              ad[h] = fmaf(dos[h * D + e + i], fv[i], ad[h]);
            }
      }
#pragma unroll
      for (int h = 0; h < HB; ++h)
        if (h < nh && L[h] > -INFINITY) {
          p[h] = expf(aq[h] * scale - L[h]);
          pd[h] = p[h] * ad[h];
        }
    }
    float es[HB];
#pragma unroll
    for (int h = 0; h < HB; ++h) es[h] = wave_sum(pd[h]);
    __syncthreads();  // the previous chunk's readers of ps, pds, us and wred are done
    if (lane == 0)
#pragma unroll
      for (int h = 0; h < HB; ++h) wred[wv * HB + h] = es[h];
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      ps[h * BWD_THREADS + tid] = p[h];
      pds[h * BWD_THREADS + tid] = pd[h];
    }
    us[tid] = u;
    __syncthreads();
#pragma unroll
    for (int h = 0; h < HB; ++h)
      for (int w2 = 0; w2 < BWD_THREADS / 64; ++w2) E[h] += wred[w2 * HB + h];
    if (tid < D) {
      const int64_t cnt = (nslots - a0 < BWD_THREADS) ? nslots - a0 : BWD_THREADS;
      for (int c = 0; c < cnt; ++c)
        if (us[c] >= 0) {
          const float kv = to_f32(kb[us[c] * kstride + tid]);
#pragma unroll
          for (int h = 0; h < HB; ++h) {
            a1[h] = fmaf(pds[h * BWD_THREADS + c], kv, a1[h]);
            a2[h] = fmaf(ps[h * BWD_THREADS + c], kv, a2[h]);
          }
        }
    }
  }
  if (tid < D)
#pragma unroll
    for (int h = 0; h < HB; ++h)
      if (h < nh) dqs[h * D + tid] += gate[h] * scale * (a1[h] - E[h] * a2[h]);
}

template <typename T>
__global__ void __launch_bounds__(BWD_THREADS)
    bwd_row_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   const float* __restrict__ kc, const float* __restrict__ vc, const int32_t* __restrict__ idx,
                   const uint8_t* __restrict__ vid, const float* __restrict__ gates, const T* __restrict__ dout,
                   float* __restrict__ dq, float* __restrict__ dgates, float* __restrict__ st_l,
                   float* __restrict__ st_e, Dims dm) {
  __shared__ float qs[HB * 256], dos[HB * 256], dqs[HB * 256];
  __shared__ float ps[HB * BWD_THREADS], pds[HB * BWD_THREADS];
  __shared__ int64_t us[BWD_THREADS];
  __shared__ float wred[(BWD_THREADS / 64) * HB];
  const int64_t r = blockIdx.x;
  const int g = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  const int D = dm.D;
  const int64_t t = dm.q0 + r;
  const bool is_vid = vid ? (vid[b * dm.Tq + r] != 0) : true;
  const int64_t kstride = (int64_t)dm.Hkv * D;
  const T* kb = k + (b * dm.T * dm.Hkv + g) * (int64_t)D;
  const T* vb = v + (b * dm.T * dm.Hkv + g) * (int64_t)D;
  const float* kcb = kc + (b * dm.Nc * dm.Hkv + g) * (int64_t)D;
  const float* vcb = vc + (b * dm.Nc * dm.Hkv + g) * (int64_t)D;
  const int32_t* sel = idx ? idx + ((b * dm.Tq + r) * dm.Hkv + g) * dm.n : nullptr;
  const int ls = dm.ls;
  const int64_t row0 = (b * dm.Tq + r) * dm.Hq + (int64_t)g * dm.G;  // the group's first head's row
  for (int hb = 0; hb < dm.G; hb += HB) {
    const int nh = dm.G - hb < HB ? dm.G - hb : HB;
    __syncthreads();
    for (int x = tid; x < nh * D; x += BWD_THREADS) {
      const int64_t o = (row0 + hb) * D + x;
      qs[x] = to_f32(q[o]);
      dos[x] = to_f32(dout[o]);
      dqs[x] = 0.f;
    }
    __syncthreads();
    float L0[HB], E0[HB], L1[HB], E1[HB], L2[HB], E2[HB], gt[HB];
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      L1[h] = L2[h] = -INFINITY;
      E1[h] = E2[h] = 0.f;
    }
    if (!is_vid) {
#pragma unroll
      for (int h = 0; h < HB; ++h) gt[h] = 1.f;
      bwd_branch_rows(qs, dos, kb, vb, kstride, D, t + 1, [=](int64_t a) { return a; }, dm.scale, gt, nh, dqs, ps,
                      pds, us, wred, L0, E0);
    } else {
      const float* gg = gates + (row0 + hb) * 3;
#pragma unroll
      for (int h = 0; h < HB; ++h) gt[h] = h < nh ? gg[3 * h] : 0.f;
      const int64_t nvis = cmp_visible(t, dm.l, dm.d, dm.Nc);
      bwd_branch_rows(qs, dos, kcb, vcb, kstride, D, nvis, [=](int64_t a) { return a; }, dm.scale, gt, nh, dqs, ps,
                      pds, us, wred, L0, E0);
      auto slc_key = [=](int64_t a) -> int64_t {
        const int32_t j = sel[a / ls];
        if (j < 0) return -1;
        const int64_t u = (int64_t)j * ls + (a % ls);
        return (u <= t && u < dm.T) ? u : -1;
      };
#pragma unroll
      for (int h = 0; h < HB; ++h) gt[h] = h < nh ? gg[3 * h + 1] : 0.f;
      bwd_branch_rows(qs, dos, kb, vb, kstride, D, (int64_t)dm.n * ls, slc_key, dm.scale, gt, nh, dqs, ps, pds, us,
                      wred, L1, E1);
      const int64_t lo = t - dm.w + 1 > 0 ? t - dm.w + 1 : 0;
#pragma unroll
      for (int h = 0; h < HB; ++h) gt[h] = h < nh ? gg[3 * h + 2] : 0.f;
      bwd_branch_rows(qs, dos, kb, vb, kstride, D, t - lo + 1, [=](int64_t a) { return lo + a; }, dm.scale, gt, nh,
                      dqs, ps, pds, us, wred, L2, E2);
    }
    __syncthreads();
    for (int x = tid; x < nh * D; x += BWD_THREADS) dq[(row0 + hb) * D + x] = dqs[x];
#pragma unroll
    for (int h = 0; h < HB; ++h)
      if (tid == h && h < nh) {
        const int64_t row = row0 + hb + h;
        st_l[row * 3 + 0] = L0[h];
        st_l[row * 3 + 1] = L1[h];
        st_l[row * 3 + 2] = L2[h];
        st_e[row * 3 + 0] = E0[h];
        st_e[row * 3 + 1] = E1[h];
        st_e[row * 3 + 2] = E2[h];
        dgates[row * 3 + 0] = is_vid ? E0[h] : 0.f;
        dgates[row * 3 + 1] = is_vid ? E1[h] : 0.f;
        dgates[row * 3 + 2] = is_vid ? E2[h] : 0.f;
      }
  }
}

// ---------------------------------------------------------------------------
// Stage 2.  Lane c8 = tid % 8 of key kk = tid / 8 owns channels [c8 nc, c8 nc + nc), nc = D / 8.
// One (row, head, branch) term: P = exp(scale <q, k> - L), ds = g P (<d_out, v> - E);
// dk += scale ds q, dv += g P d_out on the lane's channels.  `on` masks the key.
template <int MAXC, typename TQ>
__device__ __forceinline__ void bwd_key_term(const float* kf, const float* vf, const TQ* qr, const TQ* dr, int nc,
                                             float scale, float L, float E, float gate, bool on, float* ak,
                                             float* av) {
  float qf[MAXC], df[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; c += 8)
    if (c < nc) {
      ld8(qr + c, qf + c);
      ld8(dr + c, df + c);
    }
  float zq = 0.f, zd = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
    if (c < nc) {
      zq = fmaf(qf[c], kf[c], zq);
      zd = fmaf(df[c], vf[c], zd);
    }
#pragma unroll
  for (int o = LPK / 2; o >= 1; o >>= 1) {
    zq += __shfl_xor(zq, o, 64);
    zd += __shfl_xor(zd, o, 64);
  }
  if (!on) return;
  const float p = expf(zq * scale - L);
  const float ds = gate * p * (zd - E);
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
    if (c < nc) {
      ak[c] = fmaf(scale * ds, qf[c], ak[c]);
      av[c] = fmaf(gate * p, df[c], av[c]);
    }
}

// The lane's nc channels of one key row, widened once.
template <int MAXC, typename TK>
__device__ __forceinline__ void load_key(const TK* kr, const TK* vr, int nc, float* kf, float* vf) {
#pragma unroll
  for (int c = 0; c < MAXC; c += 8)
    if (c < nc) {
      ld8(kr + c, kf + c);
      ld8(vr + c, vf + c);
    }
}

// Full-resolution keys [u0, u0 + 32) of KV head g: window and selection terms of video rows,
// dense terms of text rows.
template <typename T, int MAXC>
__global__ void __launch_bounds__(BWD_THREADS)
    bwd_key_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   const int32_t* __restrict__ idx, const uint8_t* __restrict__ vid, const float* __restrict__ gates,
                   const T* __restrict__ dout, const float* __restrict__ st_l, const float* __restrict__ st_e,
                   float* __restrict__ dk, float* __restrict__ dv, Dims dm) {
  const int tid = threadIdx.x, kk = tid / LPK, c8 = tid % LPK;
  const int g = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int64_t u0 = (int64_t)blockIdx.x * KB, u = u0 + kk;
  const int D = dm.D, nc = D / LPK;
  const bool kvalid = u < dm.T;
  const int64_t ur = kvalid ? u : dm.T - 1;
  const int64_t kstride = (int64_t)dm.Hkv * D;
  const T* kr = k + (b * dm.T + ur) * kstride + (int64_t)g * D + c8 * nc;
  const T* vr = v + (b * dm.T + ur) * kstride + (int64_t)g * D + c8 * nc;
  float ak[MAXC], av[MAXC], kf[MAXC], vf[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) ak[c] = av[c] = kf[c] = vf[c] = 0.f;
  load_key<MAXC>(kr, vr, nc, kf, vf);
  const int64_t ulast = (u0 + KB - 1 < dm.T - 1) ? u0 + KB - 1 : dm.T - 1;
  // rows that can see a key of the block: t >= u0 (causal), among the query rows
  int64_t r0 = u0 - dm.q0;
  if (r0 < 0) r0 = 0;
  for (int64_t r = r0; r < dm.Tq; ++r) {
    const int64_t t = dm.q0 + r;
    const bool is_vid = vid ? (vid[b * dm.Tq + r] != 0) : true;
    const int32_t* sel = idx ? idx + ((b * dm.Tq + r) * dm.Hkv + g) * dm.n : nullptr;
    // branch membership of this key for this row (uniform checks first)
    bool in_swa = false, in_slc = false, in_txt = false;
    if (!is_vid) {
      in_txt = kvalid && u <= t;
    } else {
      const int64_t lo = t - dm.w + 1;
      if (ulast >= (lo > 0 ? lo : 0) && u0 <= t) in_swa = kvalid && u <= t && u >= lo;
      bool any = false;
      for (int c = 0; c < dm.n; ++c) {
        const int32_t j = sel[c];
        if (j >= 0 && (int64_t)j * dm.ls <= ulast && ((int64_t)j + 1) * dm.ls > u0) any = true;
      }
      if (any && kvalid && u <= t) {
        const int64_t ju = u / dm.ls;
        for (int c = 0; c < dm.n; ++c) in_slc |= sel[c] == ju;
      }
      // skip rows where no key of the block takes part (uniform over the workgroup)
      if (!any && !(ulast >= (lo > 0 ? lo : 0) && u0 <= t)) continue;
    }
    for (int hh = 0; hh < dm.G; ++hh) {
      const int h = g * dm.G + hh;
      const int64_t row = (b * dm.Tq + r) * dm.Hq + h;
      const T* qr = q + row * D + c8 * nc;
      const T* dr = dout + row * D + c8 * nc;
      if (!is_vid) {
        bwd_key_term<MAXC>(kf, vf, qr, dr, nc, dm.scale, st_l[row * 3], st_e[row * 3], 1.f, in_txt, ak, av);
      } else {
        const float* gg = gates + row * 3;
        bwd_key_term<MAXC>(kf, vf, qr, dr, nc, dm.scale, st_l[row * 3 + 1], st_e[row * 3 + 1], gg[1], in_slc, ak, av);
        bwd_key_term<MAXC>(kf, vf, qr, dr, nc, dm.scale, st_l[row * 3 + 2], st_e[row * 3 + 2], gg[2], in_swa, ak, av);
      }
    }
  }
  if (!kvalid) return;
  float* dko = dk + (b * dm.T + u) * kstride + (int64_t)g * D + c8 * nc;
  float* dvo = dv + (b * dm.T + u) * kstride + (int64_t)g * D + c8 * nc;
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
    if (c < nc) {
      dko[c] = ak[c];
      dvo[c] = av[c];
    }
}

// Compressed keys [i0, i0 + 32) of KV head g: compression-branch terms of video rows.
template <typename T, int MAXC>
__global__ void __launch_bounds__(BWD_THREADS)
    bwd_ckey_kernel(const T* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
                    const uint8_t* __restrict__ vid, const float* __restrict__ gates, const T* __restrict__ dout,
                    const float* __restrict__ st_l, const float* __restrict__ st_e, float* __restrict__ dkc,
                    float* __restrict__ dvc, Dims dm) {
  const int tid = threadIdx.x, kk = tid / LPK, c8 = tid % LPK;
  const int g = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int64_t i0 = (int64_t)blockIdx.x * KB, i = i0 + kk;
  const int D = dm.D, nc = D / LPK;
  const bool kvalid = i < dm.Nc;
  const int64_t ir = kvalid ? i : dm.Nc - 1;
  const int64_t kstride = (int64_t)dm.Hkv * D;
  const float* kr = kc + (b * dm.Nc + ir) * kstride + (int64_t)g * D + c8 * nc;
  const float* vr = vc + (b * dm.Nc + ir) * kstride + (int64_t)g * D + c8 * nc;
  float ak[MAXC], av[MAXC], kf[MAXC], vf[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) ak[c] = av[c] = kf[c] = vf[c] = 0.f;
  load_key<MAXC>(kr, vr, nc, kf, vf);
  const int64_t end_i = i * dm.d + dm.l - 1;  // the key is visible from this position on
  int64_t r0 = i0 * dm.d + dm.l - 1 - dm.q0;
  if (r0 < 0) r0 = 0;
  for (int64_t r = r0; r < dm.Tq; ++r) {
    const int64_t t = dm.q0 + r;
    if (vid && !vid[b * dm.Tq + r]) continue;
    const bool on = kvalid && end_i <= t;
    for (int hh = 0; hh < dm.G; ++hh) {
      const int h = g * dm.G + hh;
      const int64_t row = (b * dm.Tq + r) * dm.Hq + h;
      bwd_key_term<MAXC>(kf, vf, q + row * D + c8 * nc, dout + row * D + c8 * nc, nc, dm.scale, st_l[row * 3],
                   st_e[row * 3], gates[row * 3], on, ak, av);
    }
  }
  if (!kvalid) return;
  float* dko = dkc + (b * dm.Nc + i) * kstride + (int64_t)g * D + c8 * nc;
  float* dvo = dvc + (b * dm.Nc + i) * kstride + (int64_t)g * D + c8 * nc;
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
    if (c < nc) {
      dko[c] = ak[c];
      dvo[c] = av[c];
    }
}

// ---------------------------------------------------------------------------
// Stage 3.  dk[u] += sum over the compressed blocks i that hold u of w_k[u - i d] dkc[i];
// one thread per (batch, token, KV head, channel).
__global__ void __launch_bounds__(BWD_THREADS)
    bwd_compress_kernel(const float* __restrict__ dkc, const float* __restrict__ dvc, const float* __restrict__ w_k,
                        const float* __restrict__ w_v, float* __restrict__ dk, float* __restrict__ dv, Dims dm) {
  const int64_t x = (int64_t)blockIdx.x * BWD_THREADS + threadIdx.x;
  const int64_t per = (int64_t)dm.Hkv * dm.D;
  if (x >= dm.B * dm.T * per) return;
  const int64_t b = x / (dm.T * per), u = (x / per) % dm.T, c = x % per;
  // i d <= u <= i d + l - 1
  int64_t ilo = u - dm.l + 1;
  ilo = ilo > 0 ? (ilo + dm.d - 1) / dm.d : 0;
  int64_t ihi = u / dm.d;
  if (ihi > dm.Nc - 1) ihi = dm.Nc - 1;
  float gk = 0.f, gv = 0.f;
  for (int64_t i = ilo; i <= ihi; ++i) {
    const int m = (int)(u - i * dm.d);
    const int64_t o = (b * dm.Nc + i) * per + c;
    gk = fmaf(w_k[m], dkc[o], gk);
    gv = fmaf(w_v[m], dvc[o], gv);
  }
  dk[x] += gk;
  dv[x] += gv;
}

// dw_k[m] = sum_{b, i, h, e} dkc[b, i, h, e] k[b, i d + m, h, e]: one workgroup per (batch, 16
// compressed blocks), partial sums per m reduced in the workgroup and added atomically.
template <typename T>
__global__ void __launch_bounds__(BWD_THREADS)
    bwd_dw_kernel(const float* __restrict__ dkc, const float* __restrict__ dvc, const T* __restrict__ k,
                  const T* __restrict__ v, float* __restrict__ dw_k, float* __restrict__ dw_v, Dims dm) {
  __shared__ float red[16];
  const int64_t b = blockIdx.y;
  const int64_t i0 = (int64_t)blockIdx.x * 16;
  const int64_t per = (int64_t)dm.Hkv * dm.D;
  const int64_t ni = (dm.Nc - i0 < 16) ? dm.Nc - i0 : 16;
  for (int m = 0; m < dm.l; ++m) {
    float sk = 0.f, sv = 0.f;
    for (int64_t x = threadIdx.x; x < ni * per; x += BWD_THREADS) {
      const int64_t i = i0 + x / per, c = x % per;
      const int64_t o = (b * dm.Nc + i) * per + c;
      const int64_t src = (b * dm.T + i * dm.d + m) * per + c;
      sk = fmaf(dkc[o], to_f32(k[src]), sk);
      sv = fmaf(dvc[o], to_f32(v[src]), sv);
    }
    sk = block_sum(sk, red);
    sv = block_sum(sv, red);
    if (threadIdx.x == 0) {
      atomicAdd(dw_k + m, sk);
      atomicAdd(dw_v + m, sv);
    }
  }
}

__global__ void bwd_fill_kernel(float* __restrict__ p, int64_t n) {
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (x < n) p[x] = 0.f;
}

// Each lane of a key takes D / 8 channels in runs of 8: head_dim a multiple of 64, at most 256.
bool bwd_supported(const Dims& dm) { return dm.D <= 256 && dm.D % (8 * LPK) == 0; }

static size_t brup(size_t x) { return (x + 255) & ~(size_t)255; }

size_t bwd_workspace(const Dims& dm) {
  const size_t ckv = brup((size_t)dm.B * dm.Nc * dm.Hkv * dm.D * 4);
  return 4 * ckv + 2 * brup((size_t)dm.B * dm.Tq * dm.Hq * 3 * 4);
}

template <typename T>
static hipError_t launch_bwd_t(const Dims& dm, const void* q, const void* k, const void* v, const float* w_k,
                               const float* w_v, const float* gates, const uint8_t* vid, const int32_t* idx,
                               const void* dout, float* dq, float* dk, float* dv, float* dgates, float* dw_k,
                               float* dw_v, void* ws, hipStream_t s) {
  const size_t ckv = brup((size_t)dm.B * dm.Nc * dm.Hkv * dm.D * 4);
  char* p = (char*)ws;
  float* kc = (float*)p;
  float* vc = (float*)(p + ckv);
  float* dkc = (float*)(p + 2 * ckv);
  float* dvc = (float*)(p + 3 * ckv);
  float* st_l = (float*)(p + 4 * ckv);
  float* st_e = (float*)(p + 4 * ckv + brup((size_t)dm.B * dm.Tq * dm.Hq * 3 * 4));
  const int dt = sizeof(T) == 2 ? 1 : 0;
  hipError_t e = hipSuccess;
  if (dm.Nc > 0) {
    e = launch_compress(dt, 1, k, w_k, kc, nullptr, dm.B, dm.T, dm.Hkv, dm.D, dm.l, dm.d, dm.Nc, s);
    if (e == hipSuccess) e = launch_compress(dt, 1, v, w_v, vc, nullptr, dm.B, dm.T, dm.Hkv, dm.D, dm.l, dm.d, dm.Nc, s);
    if (e != hipSuccess) return e;
  }
  bwd_fill_kernel<<<dim3((unsigned)((dm.l + 255) / 256)), dim3(256), 0, s>>>(dw_k, dm.l);
  bwd_fill_kernel<<<dim3((unsigned)((dm.l + 255) / 256)), dim3(256), 0, s>>>(dw_v, dm.l);
  bwd_row_kernel<T><<<dim3((unsigned)dm.Tq, (unsigned)dm.Hkv, (unsigned)dm.B), dim3(BWD_THREADS), 0, s>>>(
      (const T*)q, (const T*)k, (const T*)v, kc, vc, idx, vid, gates, (const T*)dout, dq, dgates, st_l, st_e, dm);
  // channels per lane: 16 (head_dim <= 128) or 32 (<= 256)
  const dim3 gk((unsigned)((dm.T + KB - 1) / KB), (unsigned)dm.Hkv, (unsigned)dm.B);
  if (dm.D <= 128)
    bwd_key_kernel<T, 16><<<gk, dim3(BWD_THREADS), 0, s>>>((const T*)q, (const T*)k, (const T*)v, idx, vid, gates,
                                                          (const T*)dout, st_l, st_e, dk, dv, dm);
  else
    bwd_key_kernel<T, 32><<<gk, dim3(BWD_THREADS), 0, s>>>((const T*)q, (const T*)k, (const T*)v, idx, vid, gates,
                                                          (const T*)dout, st_l, st_e, dk, dv, dm);
  if (dm.Nc > 0) {
    const dim3 gc((unsigned)((dm.Nc + KB - 1) / KB), (unsigned)dm.Hkv, (unsigned)dm.B);
    if (dm.D <= 128)
      bwd_ckey_kernel<T, 16><<<gc, dim3(BWD_THREADS), 0, s>>>((const T*)q, kc, vc, vid, gates, (const T*)dout, st_l,
                                                             st_e, dkc, dvc, dm);
    else
      bwd_ckey_kernel<T, 32><<<gc, dim3(BWD_THREADS), 0, s>>>((const T*)q, kc, vc, vid, gates, (const T*)dout, st_l,
                                                             st_e, dkc, dvc, dm);
    const int64_t tot = dm.B * dm.T * dm.Hkv * dm.D;
    bwd_compress_kernel<<<dim3((unsigned)((tot + BWD_THREADS - 1) / BWD_THREADS)), dim3(BWD_THREADS), 0, s>>>(
        dkc, dvc, w_k, w_v, dk, dv, dm);
    bwd_dw_kernel<T><<<dim3((unsigned)((dm.Nc + 15) / 16), (unsigned)dm.B), dim3(BWD_THREADS), 0, s>>>(
        dkc, dvc, (const T*)k, (const T*)v, dw_k, dw_v, dm);
  }
  return hipGetLastError();
}

hipError_t launch_layer_bwd(int dtype, const Dims& dm, const void* q, const void* k, const void* v, const float* w_k,
                            const float* w_v, const float* gates, const uint8_t* vid, const int32_t* idx,
                            const void* dout, float* dq, float* dk, float* dv, float* dgates, float* dw_k,
                            float* dw_v, void* ws, hipStream_t s) {
  if (dm.B <= 0 || dm.Tq <= 0) return hipSuccess;
  if (!bwd_supported(dm)) return hipErrorInvalidValue;
  return dtype == 1 ? launch_bwd_t<bf16>(dm, q, k, v, w_k, w_v, gates, vid, idx, dout, dq, dk, dv, dgates, dw_k,
                                         dw_v, ws, s)
                    : launch_bwd_t<float>(dm, q, k, v, w_k, w_v, gates, vid, idx, dout, dq, dk, dv, dgates, dw_k,
                                          dw_v, ws, s);
}
