// Gate values of the three branches from each token's hidden state, gfx950.
//
// A learned weighting mixes the compression, selection and window outputs per
// head (top168.com digest of VideoNSA, section 一; csdn page
// "VideoNSA：重新定义视频理解的稀疏注意力机制", section 3.1: three gate values
// per head from the token's features).  Per token t and output f = 3 h + c:
//   g[t][f] = 1 / (1 + exp(-(b[f] + sum_k x[t][k] w[f][k])))
// with x [R, K] bf16 hidden states, w [N, K] bf16, b [N] fp32 (optional),
// g [R, N] fp32 — the [B, T, Hq, 3] gate tensor the layer reads.
//
// HBM-bound: the hidden states (K = 3584 channels, 7 KB a token) are read once;
// w (N <= 96 rows) is staged through LDS in 64-channel chunks and shared by the
// 128 tokens of a workgroup.  The product runs on the matrix cores with
// the gate outputs on M (three 32-row blocks) and tokens on N, so each lane ends
// with 4-float runs of one token's gates for 16-byte stores.  The reduction
// index is permuted per chunk: lane half h and step s of a 64-channel chunk take
// channels 32 h + 8 s .. +8, so each lane reads 64 contiguous bytes of its
// token's row and the two halves of a wave cover 128 contiguous bytes.
#include "fast_common.hpp"

namespace {
constexpr int GK = 64;            // hidden channels per chunk
constexpr int GF = 96;            // gate outputs per workgroup pass (3 x 32)
constexpr int GW_UNITS = GF * GK / 8;  // 16-byte units of one staged chunk of w
}  // namespace

// Element offset of (output row f, logical 16-byte chunk c) in a staged [GF][GK] chunk of w,
// chunks XOR-swizzled by the row so that 8 consecutive rows reading one chunk hit 8 positions.
__device__ __forceinline__ int gswz(int f, int c) { return f * GK + ((c ^ (f & 7)) << 3); }

// TB token blocks of 32 per wave, 4 waves: 128 TB tokens per workgroup.
template <int TB>
__global__ void __launch_bounds__(256) gate_proj_kernel(const bf16* __restrict__ x, const bf16* __restrict__ w,
                                                        const float* __restrict__ bias, float* __restrict__ g,
                                                        int64_t R, int K, int N) {
  __shared__ __attribute__((aligned(16))) bf16 s_w[2][GF * GK];
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, c = l & 31;
  const int64_t t0 = ((int64_t)blockIdx.x * 4 + wv) * (32 * TB);
  const bf16* xr[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    int64_t t = t0 + 32 * tb + c;
    if (t >= R) t = R - 1;  // rows past the end repeat the last row; their gates are not stored
    xr[tb] = x + t * K + 32 * h;
  }
  // chunk kc of w into LDS buffer `buf` (rows past N repeat row N - 1; never stored)
  auto stage = [&](int buf, int kc) {
    for (int ins = wv; ins < GW_UNITS / 64; ins += 4) {
      const int p = ins * 64 + l, f = p >> 3, cc = (p & 7) ^ (f & 7);
      const bf16* gp = w + (int64_t)(f < N ? f : N - 1) * K + kc + cc * 8;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gp,
                                       (__attribute__((address_space(3))) void*)(s_w[buf] + ins * 512), 16, 0, 0);
    }
  };
  bf16x8 xa[TB][4], xb[TB][4];
  f32x16 acc[TB][3];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int fb = 0; fb < 3; ++fb) acc[tb][fb] = f32x16{};
  const int nch = K / GK;
  // chunk ch: its w chunk is in LDS buffer ch & 1 and its x fragments in `cur`; the next chunk's
  // loads (w by DMA into the other buffer, x into `nxt`) are issued before the products
  auto chunk = [&](int ch, bf16x8 (&cur)[TB][4], bf16x8 (&nxt)[TB][4]) {
    const int buf = ch & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's share of chunk ch has landed
    __syncthreads();                                    // every share has; buf ^ 1 is no longer read
    bf16x8 wf[3][4];
#pragma unroll
    for (int fb = 0; fb < 3; ++fb)
#pragma unroll
      for (int s = 0; s < 4; ++s) wf[fb][s] = lds_read8(s_w[buf] + gswz(fb * 32 + c, 4 * h + s));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // w fragments in registers before the next DMA
    if (ch + 1 < nch) {
      stage(buf ^ 1, (ch + 1) * GK);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int s = 0; s < 4; ++s) nxt[tb][s] = *(const bf16x8*)(xr[tb] + (ch + 1) * GK + 8 * s);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int fb = 0; fb < 3; ++fb) acc[tb][fb] = mfma32(wf[fb][s], cur[tb][s], acc[tb][fb]);
  };
  stage(0, 0);
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int s = 0; s < 4; ++s) xa[tb][s] = *(const bf16x8*)(xr[tb] + 8 * s);
  for (int ch = 0; ch < nch; ch += 2) {
    chunk(ch, xa, xb);
    if (ch + 1 < nch) chunk(ch + 1, xb, xa);
  }
  // lane (h, c) holds token t0 + 32 tb + c, outputs 32 fb + 8 q + 4 h + i in acc[tb][fb][4 q + i]
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int64_t t = t0 + 32 * tb + c;
    if (t >= R) continue;
    float* gr = g + t * N;
#pragma unroll
    for (int fb = 0; fb < 3; ++fb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = 32 * fb + 8 * q + 4 * h;
        if (f >= N) continue;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float z = acc[tb][fb][4 * q + i] + (bias && f + i < N ? bias[f + i] : 0.f);
          v[i] = 1.f / (1.f + fexp2(-z * LOG2E_F));
        }
        if (vec) {
          *(float4*)(gr + f) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (f + i < N) gr[f + i] = v[i];
        }
      }
  }
}

bool gate_proj_supported(int64_t K, int N) { return K > 0 && K % GK == 0 && N > 0 && N <= GF; }

hipError_t launch_gate_proj(const void* x, const void* w, const float* bias, float* g, int64_t R, int64_t K, int N,
                            hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (!gate_proj_supported(K, N)) return hipErrorInvalidValue;
  // one 32-token block a wave (192 VGPRs: two waves a SIMD); two blocks a wave need 324
  const int64_t nblk = (R + 127) / 128;
  gate_proj_kernel<1><<<dim3((unsigned)nblk), dim3(256), 0, s>>>((const bf16*)x, (const bf16*)w, bias, g, R,
                                                                  (int)K, N);
  return hipGetLastError();
}
