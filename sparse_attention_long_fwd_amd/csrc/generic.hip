// Generic (VALU) kernels of the hybrid layer: any head_dim <= 256 (multiple of
// 8), fp32 or bf16.  They are the path for fp32 inputs and for shapes the MFMA
// kernels do not cover.  One workgroup owns one (batch, query row, KV group)
// and walks the group's heads; scores are plain fp32 dot products.
//
// Definitions (pages cited by title and section):
//  - compression branch over block tokens, importance from its probabilities,
//    selection of blocks, sliding window, per-head gates: top168.com digest of
//    VideoNSA, section 一; csdn page "VideoNSA：重新定义视频理解的稀疏注意力机制",
//    sections 2.2 and 3.1;
//  - text rows keep dense causal attention: shd-paper.top page, English
//    abstract.
#include "common.hpp"

#define GEN_THREADS 256

// ---------------------------------------------------------------------------
// Compression-branch attention + block importance.
// Dynamic shared memory: q [D] + p [256] + importance [Ns] floats.
template <typename T, typename TC>
__global__ void __launch_bounds__(GEN_THREADS)
    cmp_generic_kernel(const T* __restrict__ q, const TC* __restrict__ kc, const TC* __restrict__ vc,
                       const uint8_t* __restrict__ vid, T* __restrict__ o, float* __restrict__ lse,
                       float* __restrict__ imp, Dims dm) {
  extern __shared__ float sm[];
  __shared__ float red[16];
  const int64_t r = blockIdx.x;
  const int g = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  if (vid && !vid[b * dm.Tq + r]) return;
  const int D = dm.D;
  float* qs = sm;
  float* ps = sm + D;
  float* is = ps + GEN_THREADS;
  const int64_t t = dm.q0 + r;
  const int64_t nvis = cmp_visible(t, dm.l, dm.d, dm.Nc);
  for (int64_t j = tid; j < dm.Ns; j += GEN_THREADS) is[j] = 0.f;
  const int64_t kstride = (int64_t)dm.Hkv * D;
  const TC* kbase = kc + (b * dm.Nc * dm.Hkv + g) * (int64_t)D;
  const TC* vbase = vc + (b * dm.Nc * dm.Hkv + g) * (int64_t)D;
  for (int hh = 0; hh < dm.G; ++hh) {
    const int h = g * dm.G + hh;
    const int64_t row = (b * dm.Tq + r) * dm.Hq + h;
    __syncthreads();
    for (int e = tid; e < D; e += GEN_THREADS) qs[e] = to_f32(q[row * D + e]);
    __syncthreads();
    // pass 1: maximum, then sum of exponentials
    float mloc = -INFINITY;
    for (int64_t i = tid; i < nvis; i += GEN_THREADS) {
      const TC* kr = kbase + i * kstride;
      float z = 0.f;
      for (int e = 0; e < D; ++e) z = fmaf(qs[e], to_f32(kr[e]), z);
      mloc = fmaxf(mloc, z * dm.scale);
    }
    const float M = block_max(mloc, red);
    float sloc = 0.f;
    for (int64_t i = tid; i < nvis; i += GEN_THREADS) {
      const TC* kr = kbase + i * kstride;
      float z = 0.f;
      for (int e = 0; e < D; ++e) z = fmaf(qs[e], to_f32(kr[e]), z);
      sloc += expf(z * dm.scale - M);
    }
    const float S = block_sum(sloc, red);
    const float L = nvis > 0 ? M + logf(S) : -INFINITY;
    if (lse && tid == 0) lse[row] = L;
    // pass 2: probabilities, value sum and importance, in chunks of 256 keys
    float oacc = 0.f;
    for (int64_t i0 = 0; i0 < nvis; i0 += GEN_THREADS) {
      const int64_t i = i0 + tid;
      float p = 0.f;
      if (i < nvis) {
        const TC* kr = kbase + i * kstride;
        float z = 0.f;
        for (int e = 0; e < D; ++e) z = fmaf(qs[e], to_f32(kr[e]), z);
        p = expf(z * dm.scale - L);
      }
      __syncthreads();
      ps[tid] = p;
      __syncthreads();
      const int64_t iend = (i0 + GEN_THREADS < nvis) ? i0 + GEN_THREADS : nvis;
      if (tid < D) {
        for (int64_t ii = i0; ii < iend; ++ii) oacc = fmaf(ps[ii - i0], to_f32(vbase[ii * kstride + tid]), oacc);
      }
      // importance: thread owns selection block j, adds frac(i, j) * p_i over this chunk's blocks
      const int64_t jlo = (i0 * dm.d) / dm.ls;
      const int64_t jhi = ((iend - 1) * dm.d + dm.l - 1) / dm.ls;
      for (int64_t j = jlo + tid; j <= jhi && j < dm.Ns; j += GEN_THREADS) {
        const int64_t b0 = j * dm.ls, b1 = j * dm.ls + dm.ls - 1;
        // compressed blocks overlapping [b0, b1]: i*d <= b1 and i*d + l - 1 >= b0
        int64_t ilo = (b0 - dm.l + 1 + dm.d - 1);
        ilo = ilo > 0 ? ilo / dm.d : 0;
        int64_t ihi = b1 / dm.d;
        if (ilo < i0) ilo = i0;
        if (ihi > iend - 1) ihi = iend - 1;
        float acc = 0.f;
        for (int64_t ii = ilo; ii <= ihi; ++ii) {
          const int64_t a0 = ii * dm.d, a1 = ii * dm.d + dm.l - 1;
          const int64_t lo = a0 > b0 ? a0 : b0, hi = a1 < b1 ? a1 : b1;
          if (hi >= lo) acc = fmaf((float)(hi - lo + 1) / (float)dm.l, ps[ii - i0], acc);
        }
        is[j] += acc;
      }
    }
    if (o && tid < D) o[row * D + tid] = from_f32<T>(oacc);
  }
  __syncthreads();
  if (imp) {
    float* dst = imp + ((b * dm.Tq + r) * dm.Hkv + g) * dm.Ns;
    for (int64_t j = tid; j < dm.Ns; j += GEN_THREADS) dst[j] = is[j];
  }
}

hipError_t launch_cmp_generic(int dtype, int cdtype, const Dims& dm, const void* q, const void* kc, const void* vc,
                              const uint8_t* vid, void* o, float* lse, float* imp, hipStream_t s) {
  if (dm.Tq <= 0 || dm.B <= 0) return hipSuccess;
  dim3 grid((unsigned)dm.Tq, (unsigned)dm.Hkv, (unsigned)dm.B);
  size_t shm = sizeof(float) * (size_t)(dm.D + GEN_THREADS + dm.Ns);
  if (dtype == 1 && cdtype == 1)
    cmp_generic_kernel<bf16, bf16><<<grid, GEN_THREADS, shm, s>>>((const bf16*)q, (const bf16*)kc, (const bf16*)vc,
                                                                   vid, (bf16*)o, lse, imp, dm);
  else if (dtype == 1)
    cmp_generic_kernel<bf16, float><<<grid, GEN_THREADS, shm, s>>>((const bf16*)q, (const float*)kc,
                                                                    (const float*)vc, vid, (bf16*)o, lse, imp, dm);
  else
    cmp_generic_kernel<float, float><<<grid, GEN_THREADS, shm, s>>>((const float*)q, (const float*)kc,
                                                                     (const float*)vc, vid, (float*)o, lse, imp, dm);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Online-softmax attention of one head over a key list, 256 key slots per step.
// key_of(a) maps slot a to a token position or -1 (masked).  Thread e < D
// returns output channel e.
template <typename T, typename KeyFn>
__device__ float attend_list(const float* qs, const T* kb, const T* vb, int64_t kstride, int D, int64_t nslots,
                             KeyFn key_of, float scale, float* ps, int64_t* us, float* red) {
  const int tid = threadIdx.x;
  float m_run = -INFINITY, l_run = 0.f, oacc = 0.f;
  for (int64_t a0 = 0; a0 < nslots; a0 += GEN_THREADS) {
    const int64_t a = a0 + tid;
    const int64_t u = a < nslots ? key_of(a) : -1;
    float z = -INFINITY;
    if (u >= 0) {
      const T* kr = kb + u * kstride;
      float acc = 0.f;
      for (int e = 0; e < D; ++e) acc = fmaf(qs[e], to_f32(kr[e]), acc);
      z = acc * scale;
    }
    const float mc = block_max(z, red);
    const float m_new = fmaxf(m_run, mc);
    float p = 0.f;
    if (u >= 0) p = expf(z - m_new);
    const float lc = block_sum(p, red);
    if (m_new == -INFINITY) continue;  // nothing seen yet (uniform across the block)
    const float corr = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
    __syncthreads();
    ps[tid] = p;
    us[tid] = u;
    __syncthreads();
    l_run = l_run * corr + lc;
    if (tid < D) {
      float acc = 0.f;
      const int64_t cnt = (nslots - a0 < GEN_THREADS) ? nslots - a0 : GEN_THREADS;
      for (int c = 0; c < cnt; ++c)
        if (us[c] >= 0) acc = fmaf(ps[c], to_f32(vb[us[c] * kstride + tid]), acc);
      oacc = oacc * corr + acc;
    }
    m_run = m_new;
  }
  return l_run > 0.f ? oacc / l_run : 0.f;
}

template <typename T>
__global__ void __launch_bounds__(GEN_THREADS)
    sparse_generic_kernel(const T* __restrict__ q, const T* __restrict__ ks, const T* __restrict__ vs,
                          const T* __restrict__ kw, const T* __restrict__ vw, const int32_t* __restrict__ idx, const uint8_t* __restrict__ vid,
                          const T* __restrict__ o_cmp, const float* __restrict__ gates, T* __restrict__ out,
                          T* __restrict__ o_slc, T* __restrict__ o_swa, Dims dm) {
  __shared__ float qs[256];
  __shared__ float ps[GEN_THREADS];
  __shared__ int64_t us[GEN_THREADS];
  __shared__ float red[16];
  const int64_t r = blockIdx.x;
  const int g = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  const int D = dm.D;
  const int64_t t = dm.q0 + r;
  const bool is_vid = vid ? (vid[b * dm.Tq + r] != 0) : true;
  const int64_t kstride = (int64_t)dm.Hkv * D;
  // selection keys / values, and those of the window branch and text rows
  const T* ksb = ks + (b * dm.T * dm.Hkv + g) * (int64_t)D;
  const T* vsb = vs + (b * dm.T * dm.Hkv + g) * (int64_t)D;
  const T* kb = kw + (b * dm.T * dm.Hkv + g) * (int64_t)D;
  const T* vb = vw + (b * dm.T * dm.Hkv + g) * (int64_t)D;
  const int32_t* sel = idx ? idx + ((b * dm.Tq + r) * dm.Hkv + g) * dm.n : nullptr;
  const int ls = dm.ls;
  for (int hh = 0; hh < dm.G; ++hh) {
    const int h = g * dm.G + hh;
    const int64_t row = (b * dm.Tq + r) * dm.Hq + h;
    __syncthreads();
    for (int e = tid; e < D; e += GEN_THREADS) qs[e] = to_f32(q[row * D + e]);
    __syncthreads();
    if (!is_vid) {
      if (!out) continue;
      float o = attend_list(qs, kb, vb, kstride, D, t + 1, [=](int64_t a) { return a; }, dm.scale, ps, us, red);
      if (tid < D) out[row * D + tid] = from_f32<T>(o);
      continue;
    }
    float os = 0.f, ow = 0.f;
    if (o_slc || out) {
      auto slc_key = [=](int64_t a) -> int64_t {
        const int c = (int)(a / ls);
        const int32_t j = sel[c];
        if (j < 0) return -1;
        const int64_t u = (int64_t)j * ls + (a % ls);
        return (u <= t && u < dm.T) ? u : -1;
      };
      os = attend_list(qs, ksb, vsb, kstride, D, (int64_t)dm.n * ls, slc_key, dm.scale, ps, us, red);
      if (o_slc && tid < D) o_slc[row * D + tid] = from_f32<T>(os);
    }
    if (o_swa || out) {
      const int64_t lo = t - dm.w + 1 > 0 ? t - dm.w + 1 : 0;
      ow = attend_list(qs, kb, vb, kstride, D, t - lo + 1, [=](int64_t a) { return lo + a; }, dm.scale, ps, us,
                       red);
      if (o_swa && tid < D) o_swa[row * D + tid] = from_f32<T>(ow);
    }
    if (out && tid < D) {
      const float* gg = gates + row * 3;
      out[row * D + tid] = from_f32<T>(gg[0] * to_f32(o_cmp[row * D + tid]) + gg[1] * os + gg[2] * ow);
    }
  }
}

hipError_t launch_sparse_generic(int dtype, const Dims& dm, const void* q, const void* ks, const void* vs,
                                 const void* kw, const void* vw, const int32_t* idx, const uint8_t* vid, const void* o_cmp, const float* gates,
                                 void* out, void* o_slc, void* o_swa, hipStream_t s) {
  if (dm.Tq <= 0 || dm.B <= 0) return hipSuccess;
  dim3 grid((unsigned)dm.Tq, (unsigned)dm.Hkv, (unsigned)dm.B);
  if (dtype == 1)
    sparse_generic_kernel<bf16><<<grid, GEN_THREADS, 0, s>>>(
        (const bf16*)q, (const bf16*)ks, (const bf16*)vs, (const bf16*)kw, (const bf16*)vw, idx, vid, (const bf16*)o_cmp, gates, (bf16*)out,
        (bf16*)o_slc, (bf16*)o_swa, dm);
  else
    sparse_generic_kernel<float><<<grid, GEN_THREADS, 0, s>>>(
        (const float*)q, (const float*)ks, (const float*)vs, (const float*)kw, (const float*)vw, idx, vid, (const float*)o_cmp, gates, (float*)out,
        (float*)o_slc, (float*)o_swa, dm);
  return hipGetLastError();
}
