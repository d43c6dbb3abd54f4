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
#include "backward.hpp"

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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// acc + <x, y> over 8 bf16 channels: v_dot2_f32_bf16 takes two exact products per instruction
// into an fp32 sum.
__device__ __forceinline__ float dot8_bf16(bf16x8 x, bf16x8 y, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), __builtin_shufflevector(y, y, 0, 1),
                                        acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), __builtin_shufflevector(y, y, 2, 3),
                                        acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), __builtin_shufflevector(y, y, 4, 5),
                                        acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), __builtin_shufflevector(y, y, 6, 7),
                                         acc, false);
}

// ---------------------------------------------------------------------------
// Stage 1.  Up to HB heads of one KV group at once over one key list, so each key row is read
// once for all of them.  qs, dos: [HB][D] query and upstream gradient (LDS); thread e < D owns
// channel e of dqs [HB][D] (LDS), to which g_h scale (sum P dpv k - E sum P k) is added.  On
// return L[h], E[h] (uniform) are each head's log-sum-exp (-inf for an empty list) and E.
constexpr int HB = 8;

template <typename TK, typename KeyFn>
__device__ void bwd_branch_rows(const float* qs, const float* dos, const bf16* qh, const bf16* dh, const TK* kb,
                                const TK* vb, int64_t kstride,
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
      if constexpr (sizeof(TK) == 2) {
        for (int e = 0; e < D; e += 8) {
          const bf16x8 f = *(const bf16x8*)(kr + e);
#pragma unroll
          for (int h = 0; h < HB; ++h)
            if (h < nh) acc[h] = dot8_bf16(*(const bf16x8*)(qh + h * D + e), f, acc[h]);
        }
      } else {
        for (int e = 0; e < D; e += 8) {
          float f[8];
          ld8(kr + e, f);
#pragma unroll
          for (int h = 0; h < HB; ++h)
            if (h < nh)
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[h] = fmaf(qs[h * D + e + i], f[i], acc[h]);
        }
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
  const int np = BWD_THREADS / D, ch = tid % D, pt = tid / D;
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
      if constexpr (sizeof(TK) == 2) {
        for (int e = 0; e < D; e += 8) {
          const bf16x8 fk = *(const bf16x8*)(kr + e), fv = *(const bf16x8*)(vr + e);
#pragma unroll
          for (int h = 0; h < HB; ++h)
            if (h < nh) {
              aq[h] = dot8_bf16(*(const bf16x8*)(qh + h * D + e), fk, aq[h]);
              ad[h] = dot8_bf16(*(const bf16x8*)(dh + h * D + e), fv, ad[h]);
            }
        }
      } else {
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
    if (pt < np) {
      // thread = (channel e, part): part pt of the np = 256 / D parts takes the slots c = pt mod np,
      // 8 at a time with their loads issued together (a slot without a key has P = 0)
      const int64_t cnt = (nslots - a0 < BWD_THREADS) ? nslots - a0 : BWD_THREADS;
      for (int c0 = pt; c0 < cnt; c0 += 8 * np) {
        float kv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = c0 + i * np;
          const int64_t uu = c < cnt ? us[c] : -1;
          const float x = to_f32(kb[(uu >= 0 ? uu : 0) * kstride + ch]);
          kv[i] = uu >= 0 ? x : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = c0 + i * np < BWD_THREADS ? c0 + i * np : BWD_THREADS - 1;
#pragma unroll
          for (int h = 0; h < HB; ++h) {
            a1[h] = fmaf(pds[h * BWD_THREADS + c], kv[i], a1[h]);
            a2[h] = fmaf(ps[h * BWD_THREADS + c], kv[i], a2[h]);
          }
        }
      }
    }
  }
  // the parts' sums, in part order
  __syncthreads();
#pragma unroll
  for (int h = 0; h < HB; ++h) {
    ps[h * BWD_THREADS + tid] = a1[h];
    pds[h * BWD_THREADS + tid] = a2[h];
  }
  __syncthreads();
  if (tid < D)
#pragma unroll
    for (int h = 0; h < HB; ++h)
      if (h < nh) {
        float s1 = 0.f, s2 = 0.f;
        for (int q2 = 0; q2 < np; ++q2) {
          s1 += ps[h * BWD_THREADS + q2 * D + tid];
          s2 += pds[h * BWD_THREADS + q2 * D + tid];
        }
        dqs[h * D + tid] += gate[h] * scale * (s1 - E[h] * s2);
      }
}

template <typename T>
__global__ void __launch_bounds__(BWD_THREADS) __attribute__((amdgpu_waves_per_eu(2)))
    bwd_row_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   const float* __restrict__ kc, const float* __restrict__ vc, const int32_t* __restrict__ idx,
                   const uint8_t* __restrict__ vid, const float* __restrict__ gates, const T* __restrict__ dout,
                   float* __restrict__ dq, float* __restrict__ dgates, float* __restrict__ st_l,
                   float* __restrict__ st_e, Dims dm) {
  __shared__ float qs[HB * 256], dos[HB * 256], dqs[HB * 256];
  __shared__ __attribute__((aligned(16))) bf16 qh[sizeof(T) == 2 ? HB * 256 : 8], dh[sizeof(T) == 2 ? HB * 256 : 8];
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
      if constexpr (sizeof(T) == 2) {
        qh[x] = q[o];
        dh[x] = dout[o];
      }
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
      bwd_branch_rows(qs, dos, qh, dh, kb, vb, kstride, D, t + 1, [=](int64_t a) { return a; }, dm.scale, gt, nh, dqs, ps,
                      pds, us, wred, L0, E0);
    } else {
      const float* gg = gates + (row0 + hb) * 3;
#pragma unroll
      for (int h = 0; h < HB; ++h) gt[h] = h < nh ? gg[3 * h] : 0.f;
      const int64_t nvis = cmp_visible(t, dm.l, dm.d, dm.Nc);
      bwd_branch_rows(qs, dos, qh, dh, kcb, vcb, kstride, D, nvis, [=](int64_t a) { return a; }, dm.scale, gt, nh, dqs, ps,
                      pds, us, wred, L0, E0);
      auto slc_key = [=](int64_t a) -> int64_t {
        const int32_t j = sel[a / ls];
        if (j < 0) return -1;
        const int64_t u = (int64_t)j * ls + (a % ls);
        return (u <= t && u < dm.T) ? u : -1;
      };
#pragma unroll
      for (int h = 0; h < HB; ++h) gt[h] = h < nh ? gg[3 * h + 1] : 0.f;
      bwd_branch_rows(qs, dos, qh, dh, kb, vb, kstride, D, (int64_t)dm.n * ls, slc_key, dm.scale, gt, nh, dqs, ps, pds, us,
                      wred, L1, E1);
      const int64_t lo = t - dm.w + 1 > 0 ? t - dm.w + 1 : 0;
#pragma unroll
      for (int h = 0; h < HB; ++h) gt[h] = h < nh ? gg[3 * h + 2] : 0.f;
      bwd_branch_rows(qs, dos, qh, dh, kb, vb, kstride, D, t - lo + 1, [=](int64_t a) { return lo + a; }, dm.scale, gt, nh,
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

// Rows are split into chunks of rc rows (a multiple of 32), so that keys seen by nearly every row
// (the forced first selection block, the first compressed blocks) are shared by several
// workgroups.  Chunk c < n - 1 holds the keys [0, keys[c]) its rows can see in a slab
// [B, keys[c], Hkv, D] of its own at off[c] (the dv slabs follow at `half`); the last chunk writes
// the gradients themselves, and bwd_chunk_sum_kernel adds the slabs to them in chunk order, so
// the sums do not depend on scheduling.
constexpr int MAXCH = 32;
struct RowChunks {
  int64_t rc, half;
  int n;
  int64_t keys[MAXCH], off[MAXCH];
};

// At most max_chunks chunks of at least min_rows rows; compressed: the keys are compressed blocks.
static RowChunks make_chunks(const Dims& dm, int max_chunks, int64_t min_rows, bool compressed) {
  RowChunks ch{};
  int64_t r = (dm.Tq + max_chunks - 1) / max_chunks;
  if (r < min_rows) r = min_rows;
  r = (r + 31) / 32 * 32;
  ch.rc = r;
  ch.n = (int)((dm.Tq + r - 1) / r);
  const int64_t N = compressed ? dm.Nc : dm.T;
  int64_t o = 0;
  for (int c = 0; c < ch.n; ++c) {
    int64_t kc = N;
    if (c < ch.n - 1) {
      const int64_t t = dm.q0 + (c + 1) * r - 1;  // the chunk's last position
      kc = compressed ? (t + 1 >= dm.l ? (t + 1 - dm.l) / dm.d + 1 : 0) : t + 1;
      if (kc > N) kc = N;
    }
    ch.keys[c] = kc;
    ch.off[c] = o;
    if (c < ch.n - 1) o += kc * dm.B * dm.Hkv * dm.D;
  }
  ch.half = o;
  return ch;
}

// One query row's terms for the lane's key over the G heads of the group, HG heads at a time with
// their q and d_out loaded together.  Branch 1 takes statistics slot s1 and gate slot gs1 (gate 1
// when gs1 < 0); branch 2, when TWO, the window's slot 2.  Per head and branch b:
//   P_b = exp(scale <q, k> - L_b),  ds = sum_b g_b P_b (<d_out, v> - E_b),
//   dk += scale ds q,  dv += (sum_b g_b P_b) d_out,
// the branches sharing the loads and the dot products.  K8: the key's channels also come packed
// as bf16 (k8, v8; bf16 q and d_out), and the dot products run on v_dot2_f32_bf16.
template <typename T, int MAXC, bool TWO, bool K8>
__device__ __forceinline__ void bwd_row_terms(const T* __restrict__ q, const T* __restrict__ dout,
                                              const float* __restrict__ st_l, const float* __restrict__ st_e,
                                              const float* __restrict__ gates, int64_t row0, const Dims& dm,
                                              int c8, int s1, int gs1, bool on1, bool on2, const float* kf,
                                              const float* vf, const bf16x8* k8, const bf16x8* v8, float* ak,
                                              float* av) {
  constexpr int E = 16 / (int)sizeof(T);  // elements per 16-byte load
  constexpr int NV = MAXC / E;
  constexpr int HG = 128 / (MAXC * (int)sizeof(T)) > 1 ? 128 / (MAXC * (int)sizeof(T)) : 1;
  typedef T rawv __attribute__((ext_vector_type(E)));
  const int D = dm.D, nc = D / LPK;
  for (int h0 = 0; h0 < dm.G; h0 += HG) {
    rawv qv[HG][NV], dw[HG][NV];
    float L1[HG], E1[HG], G1[HG], L2[HG], E2[HG], G2[HG];
#pragma unroll
    for (int i = 0; i < HG; ++i) {
      const int hh = h0 + i < dm.G ? h0 + i : dm.G - 1;
      const int64_t row = row0 + hh;
      const T* qr = q + row * D + c8 * nc;
      const T* dr = dout + row * D + c8 * nc;
#pragma unroll
      for (int j = 0; j < NV; ++j)
        if (j * E < nc) {
          qv[i][j] = *(const rawv*)(qr + j * E);
          dw[i][j] = *(const rawv*)(dr + j * E);
        }
      L1[i] = st_l[row * 3 + s1];
      E1[i] = st_e[row * 3 + s1];
      G1[i] = gs1 >= 0 ? gates[row * 3 + gs1] : 1.f;
      if (TWO) {
        L2[i] = st_l[row * 3 + 2];
        E2[i] = st_e[row * 3 + 2];
        G2[i] = gates[row * 3 + 2];
      }
    }
#pragma unroll
    for (int i = 0; i < HG; ++i) {
      float zq = 0.f, zd = 0.f;
      if constexpr (K8) {
#pragma unroll
        for (int j = 0; j < NV; ++j)
          if (j * E < nc) {
            zq = dot8_bf16(qv[i][j], k8[j], zq);
            zd = dot8_bf16(dw[i][j], v8[j], zd);
          }
      } else {
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (j * E + e < nc) {
              zq = fmaf(to_f32(qv[i][j][e]), kf[j * E + e], zq);
              zd = fmaf(to_f32(dw[i][j][e]), vf[j * E + e], zd);
            }
      }
#pragma unroll
      for (int o = LPK / 2; o >= 1; o >>= 1) {
        zq += __shfl_xor(zq, o, 64);
        zd += __shfl_xor(zd, o, 64);
      }
      const bool hv = h0 + i < dm.G;
      const float a1 = hv && on1 ? G1[i] * expf(zq * dm.scale - L1[i]) : 0.f;
      float sds = a1 * (zd - E1[i]), pa = a1;
      if (TWO) {
        const float a2 = hv && on2 ? G2[i] * expf(zq * dm.scale - L2[i]) : 0.f;
        sds += a2 * (zd - E2[i]);
        pa += a2;
      }
      sds *= dm.scale;
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (j * E + e < nc) {
            ak[j * E + e] = fmaf(sds, to_f32(qv[i][j][e]), ak[j * E + e]);
            av[j * E + e] = fmaf(pa, to_f32(dw[i][j][e]), av[j * E + e]);
          }
    }
  }
}

// Bits [lo, hi) of 32-row word `base` (lo, hi relative to the chunk's rows [ra, rb)).
__device__ __forceinline__ uint32_t word_range(int64_t base, int64_t ra, int64_t rb, uint32_t m) {
  if (base < ra) m &= ~((1u << (ra - base)) - 1u);
  if (base + 32 > rb) m &= (1u << (rb - base)) - 1u;
  return m;
}

// The lane's accumulated gradients: the gradient rows themselves for the last chunk, else the
// chunk's slab.
template <int MAXC>
__device__ __forceinline__ void store_key_grads(const float* ak, const float* av, float* gk, float* gv,
                                                float* part, const RowChunks& ch, int c, int64_t b, int64_t u,
                                                int64_t N, int g, const Dims& dm, int c8) {
  const int nc = dm.D / LPK;
  const int64_t kstride = (int64_t)dm.Hkv * dm.D;
  float *dko, *dvo;
  if (c == ch.n - 1) {
    dko = gk + (b * N + u) * kstride + (int64_t)g * dm.D + c8 * nc;
    dvo = gv + (b * N + u) * kstride + (int64_t)g * dm.D + c8 * nc;
  } else {
    const int64_t o = ch.off[c] + (b * ch.keys[c] + u) * kstride + (int64_t)g * dm.D + c8 * nc;
    dko = part + o;
    dvo = part + ch.half + o;
  }
#pragma unroll
  for (int i = 0; i < MAXC; ++i)
    if (i < nc) {
      dko[i] = ak[i];
      dvo[i] = av[i];
    }
}

// Full-resolution keys [u0, u0 + 32) of KV head g, the rows of chunk c: window and selection
// terms of video rows, dense terms of text rows.
template <typename T, int MAXC>
__global__ void __launch_bounds__(BWD_THREADS)
    bwd_key_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   const int32_t* __restrict__ idx, const uint8_t* __restrict__ vid, const float* __restrict__ gates,
                   const T* __restrict__ dout, const float* __restrict__ st_l, const float* __restrict__ st_e,
                   const uint32_t* __restrict__ sbits, const uint32_t* __restrict__ tbits, float* __restrict__ dk,
                   float* __restrict__ dv, float* __restrict__ part, Dims dm, RowChunks ch) {
  const int tid = threadIdx.x, kk = tid / LPK, c8 = tid % LPK, lane = tid & 63;
  const int g = blockIdx.y;
  const int64_t b = blockIdx.z / ch.n;
  const int c = (int)(blockIdx.z % ch.n);
  const int64_t u0 = (int64_t)blockIdx.x * KB, u = u0 + kk;
  if (u0 >= ch.keys[c]) return;  // no row of the chunk sees these keys, and the chunk stores none of them
  const int D = dm.D, nc = D / LPK;
  const bool kvalid = u < dm.T;
  const int64_t ur = kvalid ? u : dm.T - 1;
  const int64_t kstride = (int64_t)dm.Hkv * D;
  float ak[MAXC], av[MAXC], kf[MAXC], vf[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) ak[i] = av[i] = kf[i] = vf[i] = 0.f;
  load_key<MAXC>(k + (b * dm.T + ur) * kstride + (int64_t)g * D + c8 * nc,
                 v + (b * dm.T + ur) * kstride + (int64_t)g * D + c8 * nc, nc, kf, vf);
  constexpr bool K8 = sizeof(T) == 2;
  bf16x8 k8[MAXC / 8], v8[MAXC / 8];  // bf16 keys: the same channels packed (exact)
#pragma unroll
  for (int j = 0; j < MAXC / 8; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      k8[j][e] = (bf16)kf[8 * j + e];
      v8[j][e] = (bf16)vf[8 * j + e];
    }
  const int64_t ulast = (u0 + KB - 1 < dm.T - 1) ? u0 + KB - 1 : dm.T - 1;
  // Rows that can see a key of the block (t >= u0) among the chunk's rows [ra, rb).  Only rows
  // that can take part are visited, 32 at a time from bit masks: text rows, the window range of
  // the block's keys, and the rows that chose a selection block overlapping the keys.
  int64_t ra = u0 - dm.q0;
  if (ra < c * ch.rc) ra = c * ch.rc;
  if (ra < 0) ra = 0;
  const int64_t rb = (c + 1) * ch.rc < dm.Tq ? (c + 1) * ch.rc : dm.Tq;
  const int64_t nw = (dm.Tq + 31) / 32;
  const int64_t rw1 = ulast + dm.w - 1 - dm.q0;  // last row whose window reaches a key of the block
  const int64_t j0 = u0 / dm.ls, j1 = ulast / dm.ls, ju = ur / dm.ls;
  const uint32_t* sb = sbits + ((b * dm.Hkv + g) * dm.Ns) * nw;
  for (int64_t wi = ra / 32; wi * 32 < rb; ++wi) {
    const int64_t base = wi * 32;
    uint32_t m = tbits[b * nw + wi];
    for (int64_t j = j0; j <= j1; ++j) m |= sb[j * nw + wi];
    const int64_t wa = base > ra ? base : ra, wb = base + 31 < rw1 ? base + 31 : rw1;
    if (wa <= wb) {  // rows wa .. wb of the window range
      const uint32_t hi = (wb - base) == 31 ? 0xffffffffu : ((1u << (wb - base + 1)) - 1u);
      m |= hi & ~((1u << (wa - base)) - 1u);
    }
    for (m = word_range(base, ra, rb, m); m; m &= m - 1) {
      const int64_t r = base + __builtin_ctz(m);
      const int64_t t = dm.q0 + r;
      // the row's top-n list, one entry per lane (n <= 32), loaded beside the row's video flag
      const int32_t sj = lane < dm.n ? idx[((b * dm.Tq + r) * dm.Hkv + g) * dm.n + lane] : -1;
      const bool is_vid = vid ? (vid[b * dm.Tq + r] != 0) : true;
      // branch membership of this key for this row: on1 (text, or selection) and on2 (window)
      bool on1 = false, on2 = false;
      if (!is_vid) {
        on1 = kvalid && u <= t;
      } else {
        on2 = kvalid && u <= t && u >= t - dm.w + 1;
        for (int64_t j = j0; j <= j1; ++j)
          if (__any(sj == (int32_t)j) && j == ju) on1 = kvalid && u <= t;
      }
      if (!__any(on1 || on2)) continue;  // no key of this wave takes part
      bwd_row_terms<T, MAXC, true, K8>(q, dout, st_l, st_e, gates, (b * dm.Tq + r) * dm.Hq + (int64_t)g * dm.G,
                                       dm, c8, is_vid ? 1 : 0, is_vid ? 1 : -1, on1, on2, kf, vf, k8, v8, ak, av);
    }
  }
  if (kvalid && u < ch.keys[c]) store_key_grads<MAXC>(ak, av, dk, dv, part, ch, c, b, u, dm.T, g, dm, c8);
}

// Compressed keys [i0, i0 + 32) of KV head g, the video rows of chunk c: compression-branch terms.
template <typename T, int MAXC>
__global__ void __launch_bounds__(BWD_THREADS)
    bwd_ckey_kernel(const T* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
                    const float* __restrict__ gates, const T* __restrict__ dout, const float* __restrict__ st_l,
                    const float* __restrict__ st_e, const uint32_t* __restrict__ tbits, float* __restrict__ dkc,
                    float* __restrict__ dvc, float* __restrict__ part, Dims dm, RowChunks ch) {
  const int tid = threadIdx.x, kk = tid / LPK, c8 = tid % LPK;
  const int g = blockIdx.y;
  const int64_t b = blockIdx.z / ch.n;
  const int c = (int)(blockIdx.z % ch.n);
  const int64_t i0 = (int64_t)blockIdx.x * KB, i = i0 + kk;
  if (i0 >= ch.keys[c]) return;
  const int D = dm.D, nc = D / LPK;
  const bool kvalid = i < dm.Nc;
  const int64_t ir = kvalid ? i : dm.Nc - 1;
  const int64_t kstride = (int64_t)dm.Hkv * D;
  float ak[MAXC], av[MAXC], kf[MAXC], vf[MAXC];
#pragma unroll
  for (int x = 0; x < MAXC; ++x) ak[x] = av[x] = kf[x] = vf[x] = 0.f;
  load_key<MAXC>(kc + (b * dm.Nc + ir) * kstride + (int64_t)g * D + c8 * nc,
                 vc + (b * dm.Nc + ir) * kstride + (int64_t)g * D + c8 * nc, nc, kf, vf);
  const int64_t end_i = i * dm.d + dm.l - 1;  // the key is visible from this position on
  int64_t ra = i0 * dm.d + dm.l - 1 - dm.q0;
  if (ra < c * ch.rc) ra = c * ch.rc;
  if (ra < 0) ra = 0;
  const int64_t rb = (c + 1) * ch.rc < dm.Tq ? (c + 1) * ch.rc : dm.Tq;
  const int64_t nw = (dm.Tq + 31) / 32;
  for (int64_t wi = ra / 32; wi * 32 < rb; ++wi) {
    const int64_t base = wi * 32;
    for (uint32_t m = word_range(base, ra, rb, ~tbits[b * nw + wi]); m; m &= m - 1) {  // video rows
      const int64_t r = base + __builtin_ctz(m);
      const bool on = kvalid && end_i <= dm.q0 + r;
      if (!__any(on)) continue;
      bwd_row_terms<T, MAXC, false, false>(q, dout, st_l, st_e, gates, (b * dm.Tq + r) * dm.Hq + (int64_t)g * dm.G,
                                           dm, c8, 0, 0, on, false, kf, vf, nullptr, nullptr, ak, av);
    }
  }
  if (kvalid && i < ch.keys[c]) store_key_grads<MAXC>(ak, av, dkc, dvc, part, ch, c, b, i, dm.Nc, g, dm, c8);
}

// gk, gv [B, N, Hkv, D] (the last chunk's sums) += the slabs of the other chunks, in chunk order.
__global__ void bwd_chunk_sum_kernel(const float* __restrict__ part, float* __restrict__ gk, float* __restrict__ gv,
                                     int64_t N, Dims dm, RowChunks ch) {
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t hd = (int64_t)dm.Hkv * dm.D;
  if (x >= dm.B * N * hd) return;
  const int64_t b = x / (N * hd), u = (x / hd) % N, e = x % hd;
  float sk = 0.f, sv = 0.f;
  for (int c = 0; c < ch.n - 1; ++c)
    if (u < ch.keys[c]) {
      const int64_t o = ch.off[c] + (b * ch.keys[c] + u) * hd + e;
      sk += part[o];
      sv += part[ch.half + o];
    }
  gk[x] += sk;
  gv[x] += sv;
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

// Row bit masks for the key kernel: sbits [B, Hkv, Ns, nw] marks the video rows that chose each
// block, tbits [B, nw] the text rows (nw = 32-row words).  One thread per (batch, row, group, slot);
// the masks start at zero.  OR is order-free, so the masks are deterministic.
__global__ void bwd_bits_kernel(const int32_t* __restrict__ idx, const uint8_t* __restrict__ vid,
                                uint32_t* __restrict__ sbits, uint32_t* __restrict__ tbits, Dims dm) {
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= dm.B * dm.Tq * dm.Hkv * dm.n) return;
  const int s = (int)(x % dm.n);
  const int g = (int)((x / dm.n) % dm.Hkv);
  const int64_t br = x / ((int64_t)dm.n * dm.Hkv);  // b * Tq + r
  const int64_t b = br / dm.Tq, r = br % dm.Tq;
  const int64_t nw = (dm.Tq + 31) / 32;
  const uint32_t bit = 1u << (r % 32);
  if (vid && !vid[br]) {
    if (g == 0 && s == 0) atomicOr(tbits + b * nw + r / 32, bit);
    return;
  }
  const int j = idx[x];
  if (j >= 0 && j < dm.Ns) atomicOr(sbits + ((b * dm.Hkv + g) * dm.Ns + j) * nw + r / 32, bit);
}

// Each lane of a key takes D / 8 channels in runs of 8: head_dim a multiple of 64, at most 256.
bool bwd_supported(const Dims& dm) { return dm.D <= 256 && dm.D % (8 * LPK) == 0; }

static size_t brup(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t bits_bytes(const Dims& dm) {
  const size_t nw = (size_t)(dm.Tq + 31) / 32;
  return brup((size_t)dm.B * dm.Hkv * dm.Ns * nw * 4) + brup((size_t)dm.B * nw * 4);
}

// chunking of the key kernel's rows (at most 4 chunks) and of the compressed-key kernel's (at most 32)
static RowChunks key_rows(const Dims& dm) { return make_chunks(dm, 4, 2048, false); }
static RowChunks ckey_rows(const Dims& dm) { return make_chunks(dm, MAXCH, 1024, true); }

static size_t part_bytes(const Dims& dm) {
  const size_t a = (size_t)key_rows(dm).half, c = dm.Nc > 0 ? (size_t)ckey_rows(dm).half : 0;
  return brup((a > c ? a : c) * 2 * 4);
}

size_t bwd_workspace(const Dims& dm) {
  const size_t ckv = brup((size_t)dm.B * dm.Nc * dm.Hkv * dm.D * 4);
  return 4 * ckv + 2 * brup((size_t)dm.B * dm.Tq * dm.Hq * 3 * 4) + bits_bytes(dm) + part_bytes(dm);
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
  uint32_t* sbits = (uint32_t*)(p + 4 * ckv + 2 * brup((size_t)dm.B * dm.Tq * dm.Hq * 3 * 4));
  const size_t nw = (size_t)(dm.Tq + 31) / 32;
  uint32_t* tbits = sbits + brup((size_t)dm.B * dm.Hkv * dm.Ns * nw * 4) / 4;
  float* part = (float*)((char*)sbits + bits_bytes(dm));
  const RowChunks kch = key_rows(dm);
  const int dt = sizeof(T) == 2 ? 1 : 0;
  hipError_t e = hipSuccess;
  if (dm.Nc > 0) {
    e = launch_compress(dt, 1, k, w_k, kc, nullptr, dm.B, dm.T, dm.Hkv, dm.D, dm.l, dm.d, dm.Nc, s);
    if (e == hipSuccess) e = launch_compress(dt, 1, v, w_v, vc, nullptr, dm.B, dm.T, dm.Hkv, dm.D, dm.l, dm.d, dm.Nc, s);
    if (e != hipSuccess) return e;
  }
  const int64_t nbits = (int64_t)(bits_bytes(dm) / 4);
  bwd_fill_kernel<<<dim3((unsigned)((nbits + 255) / 256)), dim3(256), 0, s>>>((float*)sbits, nbits);
  const int64_t npairs = dm.B * dm.Tq * dm.Hkv * dm.n;
  bwd_bits_kernel<<<dim3((unsigned)((npairs + 255) / 256)), dim3(256), 0, s>>>(idx, vid, sbits, tbits, dm);
  bwd_fill_kernel<<<dim3((unsigned)((dm.l + 255) / 256)), dim3(256), 0, s>>>(dw_k, dm.l);
  bwd_fill_kernel<<<dim3((unsigned)((dm.l + 255) / 256)), dim3(256), 0, s>>>(dw_v, dm.l);
  bwd_row_kernel<T><<<dim3((unsigned)dm.Tq, (unsigned)dm.Hkv, (unsigned)dm.B), dim3(BWD_THREADS), 0, s>>>(
      (const T*)q, (const T*)k, (const T*)v, kc, vc, idx, vid, gates, (const T*)dout, dq, dgates, st_l, st_e, dm);
  // channels per lane: 16 (head_dim <= 128) or 32 (<= 256)
  const dim3 gk((unsigned)((dm.T + KB - 1) / KB), (unsigned)dm.Hkv, (unsigned)(dm.B * kch.n));
  if (dm.D <= 128)
    bwd_key_kernel<T, 16><<<gk, dim3(BWD_THREADS), 0, s>>>((const T*)q, (const T*)k, (const T*)v, idx, vid, gates,
                                                          (const T*)dout, st_l, st_e, sbits, tbits, dk, dv, part,
                                                          dm, kch);
  else
    bwd_key_kernel<T, 32><<<gk, dim3(BWD_THREADS), 0, s>>>((const T*)q, (const T*)k, (const T*)v, idx, vid, gates,
                                                          (const T*)dout, st_l, st_e, sbits, tbits, dk, dv, part,
                                                          dm, kch);
  const int64_t tot = dm.B * dm.T * dm.Hkv * dm.D;
  if (kch.n > 1)
    bwd_chunk_sum_kernel<<<dim3((unsigned)((tot + BWD_THREADS - 1) / BWD_THREADS)), dim3(BWD_THREADS), 0, s>>>(
        part, dk, dv, dm.T, dm, kch);
  if (dm.Nc > 0) {
    const RowChunks cch = ckey_rows(dm);
    const dim3 gc((unsigned)((dm.Nc + KB - 1) / KB), (unsigned)dm.Hkv, (unsigned)(dm.B * cch.n));
    if (dm.D <= 128)
      bwd_ckey_kernel<T, 16><<<gc, dim3(BWD_THREADS), 0, s>>>((const T*)q, kc, vc, gates, (const T*)dout, st_l,
                                                             st_e, tbits, dkc, dvc, part, dm, cch);
    else
      bwd_ckey_kernel<T, 32><<<gc, dim3(BWD_THREADS), 0, s>>>((const T*)q, kc, vc, gates, (const T*)dout, st_l,
                                                             st_e, tbits, dkc, dvc, part, dm, cch);
    const int64_t ctot = dm.B * dm.Nc * dm.Hkv * dm.D;
    if (cch.n > 1)
      bwd_chunk_sum_kernel<<<dim3((unsigned)((ctot + BWD_THREADS - 1) / BWD_THREADS)), dim3(BWD_THREADS), 0, s>>>(
          part, dkc, dvc, dm.Nc, dm, cch);
    bwd_compress_kernel<<<dim3((unsigned)((tot + BWD_THREADS - 1) / BWD_THREADS)), dim3(BWD_THREADS), 0, s>>>(
        dkc, dvc, w_k, w_v, dk, dv, dm);
    bwd_dw_kernel<T><<<dim3((unsigned)((dm.Nc + 15) / 16), (unsigned)dm.B), dim3(BWD_THREADS), 0, s>>>(
        dkc, dvc, (const T*)k, (const T*)v, dw_k, dw_v, dm);
  }
  return hipGetLastError();
}

// The compression's share of dk, dv (dk[u] += sum_i w_k[u - i d] dkc[i], likewise v) and the
// compression weight gradients dw_k, dw_v (cleared here, then summed over the batch) from the
// gradients dkc, dvc of the compressed keys and values.
hipError_t launch_bwd_compress_grads(int dtype, const Dims& dm, const float* dkc, const float* dvc, const float* w_k,
                                     const float* w_v, const void* k, const void* v, float* dk, float* dv,
                                     float* dw_k, float* dw_v, hipStream_t s) {
  bwd_fill_kernel<<<dim3((unsigned)((dm.l + 255) / 256)), dim3(256), 0, s>>>(dw_k, dm.l);
  bwd_fill_kernel<<<dim3((unsigned)((dm.l + 255) / 256)), dim3(256), 0, s>>>(dw_v, dm.l);
  if (dm.Nc <= 0) return hipGetLastError();
  const int64_t tot = dm.B * dm.T * dm.Hkv * dm.D;
  bwd_compress_kernel<<<dim3((unsigned)((tot + BWD_THREADS - 1) / BWD_THREADS)), dim3(BWD_THREADS), 0, s>>>(
      dkc, dvc, w_k, w_v, dk, dv, dm);
  const dim3 gd((unsigned)((dm.Nc + 15) / 16), (unsigned)dm.B);
  if (dtype == 1)
    bwd_dw_kernel<bf16><<<gd, dim3(BWD_THREADS), 0, s>>>(dkc, dvc, (const bf16*)k, (const bf16*)v, dw_k, dw_v, dm);
  else
    bwd_dw_kernel<float><<<gd, dim3(BWD_THREADS), 0, s>>>(dkc, dvc, (const float*)k, (const float*)v, dw_k, dw_v,
                                                          dm);
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
