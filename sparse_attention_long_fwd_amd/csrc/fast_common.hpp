// Helpers shared by the MFMA kernels: XCD-aware work mapping.
#pragma once
#include "fast.hpp"
#include "mfma.hpp"

// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2.  Work is made of `units` independent (batch, KV group)
// streams of `per_unit` items; the remap sends every XCD the items of as few
// units as possible (a unit's compressed K/V stays in that XCD's L2) and keeps
// each XCD's items in rank order, so rank 0 (the heaviest tile, by convention
// of the callers) starts first everywhere.
__host__ __device__ inline unsigned xcd_grid(int units, int per_unit) {
  if (units <= 8 && 8 % units == 0) {
    const int P = 8 / units;
    return 8u * (unsigned)((per_unit + P - 1) / P);
  }
  return (unsigned)units * (unsigned)per_unit;
}

__device__ __forceinline__ bool xcd_remap(unsigned id, int units, int per_unit, int* unit, int* rank) {
  const int xcd = (int)(id & 7u), k = (int)(id >> 3);
  if (units <= 8 && 8 % units == 0) {
    const int P = 8 / units;
    *unit = xcd / P;
    *rank = k * P + xcd % P;
  } else if (units % 8 == 0) {
    const int per = units / 8;
    *unit = xcd * per + k % per;
    *rank = k / per;
  } else {
    *unit = (int)(id % (unsigned)units);
    *rank = (int)(id / (unsigned)units);
  }
  return *rank < per_unit;
}

// Element offset of (row, 16-byte chunk c) in an LDS tile of 128-element bf16
// rows whose chunks are XOR-swizzled by the row: 16 consecutive rows reading
// the same logical chunk land on 16 different chunk positions (banks).
__device__ __forceinline__ int swz128(int row, int c) { return row * 128 + ((c ^ (row & 15)) << 3); }

// Stage rows [key0, key0 + 64) of a [*, 128] bf16 array (row stride `stride`
// elements) into a swizzled 64 x 128 LDS tile with direct global -> LDS loads
// (16 bytes a lane, lane i of an instruction lands at base + 16 i).  Rows at or
// past `nrows` repeat row nrows - 1: finite data that the callers' masks never
// weight.  Instruction m of wave w covers LDS chunks [64 (w + nw m), +64), i.e.
// four rows.  The caller waits (s_waitcnt vmcnt) and synchronises before use.
__device__ __forceinline__ void stage_tile64(bf16* lds_tile, const bf16* src, int64_t stride, int64_t key0,
                                             int64_t nrows, int w, int nw, int lane) {
  for (int ins = w; ins < 16; ins += nw) {
    const int p = ins * 64 + lane;  // LDS chunk position
    const int row = p >> 4, cpos = p & 15;
    const int c = cpos ^ (row & 15);  // logical chunk stored at this position
    int64_t key = key0 + row;
    if (key >= nrows) key = nrows - 1;
    const bf16* gp = src + key * stride + c * 8;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gp,
                                     (__attribute__((address_space(3))) void*)(lds_tile + ins * 512), 16, 0, 0);
  }
}

// Copy a contiguous 16 KB run global -> LDS with the direct-to-LDS load: 16 instructions of
// 64 lanes x 16 bytes, spread over the nw waves of the workgroup (wave w, lane `lane`).
__device__ __forceinline__ void stage_lin16k(bf16* lds_tile, const bf16* src, int w, int nw, int lane) {
  for (int ins = w; ins < 16; ins += nw)
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + (ins * 64 + lane) * 8),
                                     (__attribute__((address_space(3))) void*)(lds_tile + ins * 512), 16, 0, 0);
}

// Operand bytes of the scaled fp8 MFMAs (v_mfma_scale_f32_32x32x64_f8f6f4, ..._16x16x128_...).
// Measured on gfx950: with n lane groups (2 halves of 32 lanes, or 4 groups of 16), lane group g's
// 32 bytes are two 16-byte pieces, K = [16 g, 16 g + 16) and [16 g + 16 n, +16), and the scale
// of the 32-wide K block s is the scale byte of lane group s.  So a lane reads the two 16-channel
// pieces [16 g, +16) and [16 g + 16 n, +16) of an fp8 row (relative to the product's first
// channel) and supplies the scale of channels [32 g, 32 g + 32).

// fp8 (e4m3) pieces of one query row for the B operand: the 32 bf16 values v (two 16-channel
// pieces, as loaded by the caller) times 2^(8 - E), E the exponent of the row's largest magnitude
// rmax (frexp convention, so every scaled value stays below 256, inside e4m3's range), and the
// E8M0 scale byte 119 + E that undoes it (127, a factor 1, for an all-zero row).  One scale for the
// whole row: every lane sharing the row supplies the same byte.  Four bytes per register, in order.
__device__ __forceinline__ void fp8_pieces(const bf16x8 (&v)[4], float rmax, i32x8& out, int& sbyte) {
  int E = 0;
  (void)frexpf(rmax, &E);
  const bool ok = rmax > 0.f && 119 + E >= 1;
  sbyte = ok ? 119 + E : 127;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const float f0 = ok ? ldexpf((float)v[i][4 * e2 + 0], 8 - E) : 0.f;
      const float f1 = ok ? ldexpf((float)v[i][4 * e2 + 1], 8 - E) : 0.f;
      const float f2 = ok ? ldexpf((float)v[i][4 * e2 + 2], 8 - E) : 0.f;
      const float f3 = ok ? ldexpf((float)v[i][4 * e2 + 3], 8 - E) : 0.f;
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, wd, true);
      out[2 * i + e2] = wd;
    }
}

// Loads the two 16-channel pieces [o0, o0 + 16) and [o1, o1 + 16) of a bf16 row (zeros when !valid)
// and returns their largest magnitude.
__device__ __forceinline__ float load_pieces(const bf16* __restrict__ x, int o0, int o1, bool valid, bf16x8 (&v)[4]) {
  v[0] = valid ? *(const bf16x8*)(x + o0) : zero8();
  v[1] = valid ? *(const bf16x8*)(x + o0 + 8) : zero8();
  v[2] = valid ? *(const bf16x8*)(x + o1) : zero8();
  v[3] = valid ? *(const bf16x8*)(x + o1 + 8) : zero8();
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)v[i][e]));
  return m;
}
