// Shared device helpers and launcher declarations of the NSA library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define NSA_WAVE 64

typedef __bf16 bf16;

// Problem dimensions shared by every launcher (validated on the host).
struct Dims {
  int64_t B, Tq, T, q0;   // batch, query rows, kv tokens, position of query row 0
  int Hq, Hkv, D, G;      // heads, KV heads, head dim, heads per KV group
  int l, d, ls;           // compressed block, stride, selection block
  int n, n_init, n_local; // top-n and forced blocks
  int w;                  // window
  float scale;            // softmax scale
  int64_t Nc, Ns;         // compressed / selection block counts
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Number of compressed blocks visible from absolute position t (whole block <= t).
__device__ __forceinline__ int64_t cmp_visible(int64_t t, int l, int d, int64_t Nc) {
  int64_t v = (t + 1 >= l) ? (t + 1 - l) / d + 1 : 0;
  return v < Nc ? v : Nc;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Block-wide reductions for blockDim.x a multiple of 64; scratch holds >= 16 floats.
__device__ __forceinline__ float block_max(float x, float* scratch) {
  x = wave_max(x);
  int wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[wv] = x;
  __syncthreads();
  float r = scratch[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, scratch[i]);
  return r;
}
__device__ __forceinline__ float block_sum(float x, float* scratch) {
  x = wave_sum(x);
  int wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[wv] = x;
  __syncthreads();
  float r = scratch[0];
  for (int i = 1; i < nw; ++i) r += scratch[i];
  return r;
}

// ---------------------------------------------------------------------------
// Launchers (host side), one per kernel family.  dtype: 0 = fp32, 1 = bf16.
// out_mode: 0 = the input's type, 1 = fp32, 2 = bf16 high part (out) + low part (out_lo).
hipError_t launch_compress(int dtype, int out_mode, const void* x, const float* w, void* out, void* out_lo,
                           int64_t B, int64_t T, int H, int D, int l, int d, int64_t Nc, hipStream_t s);

// Backward pass of the layer (generic kernels): gradients of sum(dout * out); outputs fp32.
size_t bwd_workspace(const Dims& dm);
bool bwd_supported(const Dims& dm);
hipError_t launch_layer_bwd(int dtype, const Dims& dm, const void* q, const void* k, const void* v, const float* w_k,
                            const float* w_v, const float* gates, const uint8_t* vid, const int32_t* idx,
                            const void* dout, float* dq, float* dk, float* dv, float* dgates, float* dw_k,
                            float* dw_v, void* ws, hipStream_t s);

// cdtype: element type of the compressed keys / values (dtype or fp32).
hipError_t launch_cmp_generic(int dtype, int cdtype, const Dims& dm, const void* q, const void* kc, const void* vc,
                              const uint8_t* vid, void* o, float* lse, float* imp, hipStream_t s);

hipError_t launch_topk(const Dims& dm, const float* imp, const uint8_t* vid, int32_t* idx, hipStream_t s);

// Generic selection / window / text-row kernel.  Writes whichever outputs are non-null.
// ks / vs: keys and values of the selection branch; kw / vw: of the window branch and text rows.
hipError_t launch_sparse_generic(int dtype, const Dims& dm, const void* q, const void* ks, const void* vs,
                                 const void* kw, const void* vw, const int32_t* idx, const uint8_t* vid, const void* o_cmp, const float* gates,
                                 void* out, void* o_slc, void* o_swa, hipStream_t s);
