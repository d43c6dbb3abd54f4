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

// Selection partial records (the value sum of one (row, slot, head) partial) in a block
// floating-point form: 128 signed 12-bit integers X sharing one power-of-two step, 192 bytes (a
// quarter fewer than fp16, for the same 11 bits of magnitude relative to the record's largest
// value).  The step 2^(e - 11) is not stored: it is folded into the partial's (max, sum) pair as
// (m + e - 11, l 2^(11 - e)), which leaves the merge weights 2^(m - M) l / L unchanged and scales
// the value weights by exactly the step (see rec12_ml).  e is held to [-20, 128]: records whose
// largest magnitude is below 2^-20 round to a step of 2^-31.
//
// Lane (row, hl) of an O^T accumulator owns dims 32 db + 8 j4 + 4 hl + e (db, j4, e in 0..3) as
// acc[db][4 j4 + e].  It writes 8 packs of 8 values at bytes [96 hl + 12 p, +12): pack p = 2 db + c
// holds acc[db][8 c .. 8 c + 7], i.e. dims 32 db + 16 c + 4 hl + {0..3} and the same + 8, as a
// little-endian 96-bit string with value i at bit 12 i.
constexpr int SLC_REC_BYTES = 192;

__host__ __device__ inline int rec12_exp(float amax) {
  int e = 0;
  (void)frexpf(amax * 1.00048828125f, &e);  // amax (1 + 2^-11) < 2^e: scaled values round to |X| <= 2047
  return e < -20 ? -20 : (e > 128 ? 128 : e);
}

// (max, sum) of a partial whose values were stored with exponent e.
__host__ __device__ inline float2 rec12_ml(float m, float l, int e) {
  return make_float2(m + (float)(e - 11), ldexpf(l, 11 - e));
}

// Eight values times `scale` (2^(11 - e)) rounded to the nearest integer, packed into three words.
__host__ __device__ inline void rec12_pack8(const float* x, float scale, uint32_t* w3) {
  uint32_t u[8];
  for (int i = 0; i < 8; ++i) {
    // adding 1.5 * 2^23 rounds to an integer held in the low mantissa bits (two's complement mod 2^12)
    const float f = fmaf(x[i], scale, 12582912.0f);
    uint32_t b;
    __builtin_memcpy(&b, &f, 4);
    u[i] = b & 0xFFFu;
  }
  w3[0] = u[0] | (u[1] << 12) | (u[2] << 24);
  w3[1] = (u[2] >> 8) | (u[3] << 4) | (u[4] << 16) | (u[5] << 28);
  w3[2] = (u[5] >> 4) | (u[6] << 8) | (u[7] << 20);
}

__host__ __device__ inline int rec12_sx(uint32_t w, int bit) { return (int)(w << (20 - bit)) >> 20; }

// The eight integers of a pack, as floats.
__host__ __device__ inline void rec12_unpack8(uint32_t a, uint32_t b, uint32_t c, float* x) {
  x[0] = (float)rec12_sx(a, 0);
  x[1] = (float)rec12_sx(a, 12);
  x[2] = (float)rec12_sx((a >> 24) | (b << 8), 0);
  x[3] = (float)rec12_sx(b, 4);
  x[4] = (float)rec12_sx(b, 16);
  x[5] = (float)rec12_sx((b >> 28) | (c << 4), 0);
  x[6] = (float)rec12_sx(c, 8);
  x[7] = (float)rec12_sx(c, 20);
}

// Writes lane (row, hl)'s half of a record from its accumulators acc[4][16] times `mul`, with the
// record's exponent e (both halves must use the same e).
template <typename Acc>
__device__ __forceinline__ void rec12_store_half(unsigned char* rec, int hl, const Acc (&acc)[4], float mul, int e) {
  const float scale = ldexpf(mul, 11 - e);
  uint32_t w[24];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = acc[db][8 * c + i];
      rec12_pack8(x, scale, w + 3 * (2 * db + c));
    }
  uint4* dst = (uint4*)(rec + 96 * hl);
#pragma unroll
  for (int i = 0; i < 6; ++i) dst[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
}
