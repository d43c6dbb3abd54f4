// gfx950 matrix-core helpers: bf16 MFMA wrappers, LDS transpose reads, packing.
//
// Operand layouts (per lane l of a 64-wide wave):
//  v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] B[16x32]
//    A: lane l holds A[l%32][8*(l/32) .. +8]      B: lane l holds B[8*(l/32) .. +8][l%32]
//    D: lane l holds D[8*(j/4) + 4*(l/32) + j%4][l%32], j = 0..15
//  v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] B[32x16]
//    A: lane l holds A[l%16][8*(l/16) .. +8]      B: lane l holds B[8*(l/16) .. +8][l%16]
//    D: lane l holds D[4*(l/16) + j][l%16], j = 0..3
//  ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
//    (i % 4) of the 4-element chunk addressed by lane 4*e + i/4, for e = 0..3.
//    With lane j of the group pointing at row r0 + j/4, columns c0 + 4*(j%4),
//    lane i gets column c0 + i of rows r0 .. r0+3: a transposed 4 x 16 tile.
#pragma once
#include "common.hpp"

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
// v_mfma_f32_16x16x32_f16: the same layout and rate as the bf16 form, 10 mantissa bits
__device__ __forceinline__ f32x4 mfma16h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Transposed read of 4 bf16 (see the layout note above).  p points into LDS.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, const_cast<bf16*>(p)));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 lds_read8(const bf16* p) { return *(const bf16x8*)p; }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (bf16)0.f;
  return z;
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return log2f(x); }

#define LOG2E_F 1.4426950408889634f
#define LN2_F 0.6931471805599453f
