// MFMA (bf16, gfx950) kernels of the hybrid layer: declarations.
#pragma once
#include "common.hpp"

// True when the MFMA kernels cover this problem (bf16, head_dim 128, ...).
bool fast_supported(int32_t dtype, const Dims& dm);

// Scratch bytes the MFMA selection/window path needs.
size_t fast_sparse_workspace(const Dims& dm);

// cdtype: element type of the compressed keys / values (bf16 or fp32).
hipError_t launch_cmp_fast(int cdtype, const Dims& dm, const void* q, const void* kc, const void* vc, const uint8_t* vid,
                           void* o, float* lse, float* imp, hipStream_t s);

hipError_t launch_sparse_fast(const Dims& dm, const void* q, const void* k, const void* v, const int32_t* idx,
                              const uint8_t* vid, const void* o_cmp, const float* gates, void* out, void* o_slc,
                              void* o_swa, void* ws, hipStream_t s);
