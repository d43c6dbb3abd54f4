// Backward pass of the layer: launchers shared by the generic and the matrix-core kernels.
#pragma once
#include "common.hpp"

hipError_t launch_bwd_compress_grads(int dtype, const Dims& dm, const float* dkc, const float* dvc, const float* w_k,
                                     const float* w_v, const void* k, const void* v, float* dk, float* dv,
                                     float* dw_k, float* dw_v, hipStream_t s);
// The same backward on the matrix cores (bf16, head_dim 128, 1..8 heads per KV group, selection blocks
// of 32, 64 or 128 tokens); bwd_fast_supported says when it applies.
bool bwd_fast_supported(int32_t dtype, const Dims& dm);
size_t bwd_fast_workspace(const Dims& dm);
hipError_t launch_layer_bwd_fast(const Dims& dm, const void* q, const void* k, const void* v, const float* w_k,
                                 const float* w_v, const float* gates, const uint8_t* vid, const int32_t* idx,
                                 const void* dout, float* dq, float* dk, float* dv, float* dgates, float* dw_k,
                                 float* dw_v, void* ws, hipStream_t s);
