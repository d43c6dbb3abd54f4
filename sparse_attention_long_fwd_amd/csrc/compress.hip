// K/V block compressor: each compressed token is the positional weighted sum of
// the cmp_block consecutive tokens of its block (top168.com digest of VideoNSA,
// section 一: the compression branch merges neighbouring content; csdn page
// "VideoNSA：重新定义视频理解的稀疏注意力机制", section 2.2).
//
// HBM-bound: one thread owns 8 consecutive channels of one (block, KV head) and
// streams the block's tokens with 16-byte loads; neighbouring threads cover the
// rest of the token row, so every load instruction of a wave reads whole
// contiguous rows.  Blocks overlap by cmp_block - cmp_stride tokens; the second
// read of a token hits in L2.  Sums are fp32; the result is stored in the input
// type, in fp32, or as a bf16 high part plus a bf16 low part (hi + lo carries
// the fp32 sum to within 2^-16 relative), as the caller asks.
#include "common.hpp"

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;

__device__ __forceinline__ void load8(const bf16* p, float* f) {
  bf16x8_t u = *(const bf16x8_t*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)u[i];
}
__device__ __forceinline__ void load8(const float* p, float* f) {
  float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void store8(bf16* p, const float* f) {
  bf16x8_t u;
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = (bf16)f[i];
  *(bf16x8_t*)p = u;
}
__device__ __forceinline__ void store8(float* p, const float* f) {
  *(float4*)p = make_float4(f[0], f[1], f[2], f[3]);
  *(float4*)(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

// MODE 0: output in TO; MODE 2: bf16 high part to out, low part to out_lo.
template <typename T, typename TO, int MODE>
__global__ void __launch_bounds__(256) compress_kernel(const T* __restrict__ x, const float* __restrict__ w,
                                                       TO* __restrict__ out, bf16* __restrict__ out_lo, int64_t T_len,
                                                       int H, int D, int l, int d, int64_t Nc, int64_t total) {
  extern __shared__ float ws[];
  for (int m = threadIdx.x; m < l; m += blockDim.x) ws[m] = w[m];
  __syncthreads();
  int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  int chunks = D >> 3;
  int c = (int)(gid % chunks);
  int64_t rest = gid / chunks;
  int h = (int)(rest % H);
  rest /= H;
  int64_t i = rest % Nc;
  int64_t b = rest / Nc;
  const T* src = x + ((b * T_len + i * d) * H + h) * (int64_t)D + c * 8;
  int64_t tok_stride = (int64_t)H * D;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int m = 0; m < l; ++m) {
    float f[8];
    load8(src + m * tok_stride, f);
    float wm = ws[m];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(wm, f[e], acc[e]);
  }
  const int64_t o = ((b * Nc + i) * H + h) * (int64_t)D + c * 8;
  if constexpr (MODE == 2) {
    bf16x8_t hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = (bf16)acc[e];
      lo[e] = (bf16)(acc[e] - (float)hi[e]);
    }
    *(bf16x8_t*)((bf16*)out + o) = hi;
    *(bf16x8_t*)(out_lo + o) = lo;
  } else {
    store8(out + o, acc);
  }
}

hipError_t launch_compress(int dtype, int out_mode, const void* x, const float* w, void* out, void* out_lo,
                           int64_t B, int64_t T, int H, int D, int l, int d, int64_t Nc, hipStream_t s) {
  if (Nc <= 0 || B <= 0) return hipSuccess;
  int64_t total = B * Nc * H * (D / 8);
  dim3 grid((unsigned)((total + 255) / 256)), block(256);
  size_t shm = sizeof(float) * (size_t)l;
  if (dtype == 1) {
    const bf16* xi = (const bf16*)x;
    if (out_mode == 2)
      compress_kernel<bf16, bf16, 2><<<grid, block, shm, s>>>(xi, w, (bf16*)out, (bf16*)out_lo, T, H, D, l, d, Nc,
                                                             total);
    else if (out_mode == 1)
      compress_kernel<bf16, float, 0><<<grid, block, shm, s>>>(xi, w, (float*)out, nullptr, T, H, D, l, d, Nc, total);
    else
      compress_kernel<bf16, bf16, 0><<<grid, block, shm, s>>>(xi, w, (bf16*)out, nullptr, T, H, D, l, d, Nc, total);
  } else {
    compress_kernel<float, float, 0><<<grid, block, shm, s>>>((const float*)x, w, (float*)out, nullptr, T, H, D, l,
                                                              d, Nc, total);
  }
  return hipGetLastError();
}
