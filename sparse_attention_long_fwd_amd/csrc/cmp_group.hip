// Compression-branch attention fused with block importance, one wave per 16 query rows x the
// whole GQA group (gfx950, MFMA 16x16x32).
//
// What it computes (top168.com digest of VideoNSA, section 一: the selection branch scores
// segments by importance, read here from the compression branch's probabilities): for each
// video row t and head h,
//   p_i = softmax_i(scale * <q_t,h, kc_i>) over the compressed blocks i whose tokens all lie at
//         or before t,  o_cmp = sum_i p_i vc_i,
//   imp[t, g, j] = sum_{h in group g} sum_i frac(i, j) p_{h,i},
// with compressed block 32 / stride 16 and selection block 64, so block j takes compressed
// blocks 4j .. 4j+2 whole and half of 4j-1 and 4j+3.
//
// Layout on the chip.  A workgroup is 64 consecutive query rows of one KV group on four waves,
// one wave per SIMD; a wave owns 16 rows and all G heads of the group.  Scores are formed
// transposed per head, S^T = Kc Q^T with v_mfma_f32_16x16x32_bf16 (16 keys on M, the wave's 16
// rows on N): every key fragment read from LDS feeds G matrix products, and a lane holds four
// consecutive compressed keys of one row for each head -- exactly one selection block's aligned
// run of four -- so the importance is summed over the heads in registers and the half-block
// shares cross to the next lane group with one lane shuffle per 16 keys.  Values enter through
// O^T += Vc^T P^T (dims on M, 32 keys per step) from pre-transposed tiles whose key order matches
// the score registers, so P needs no shuffles; the G x 128 x 16 fp32 accumulators (224 registers
// for G = 7) stay in the accumulation registers for the whole sweep.
//
// The importance needs the final softmax normaliser, hence two sweeps over the keys: the first
// forms each (row, head)'s log-sum-exp, the second the exact probabilities, the value sum and the
// importance; both form the same scores.  All matrix products take fp16 operands: the compressed
// keys and values are fp32 block sums, and fp16's 10 mantissa bits keep the block importances
// within about 2e-4 of exact (bf16 keys move them by up to about 1e-3, which can reorder blocks
// that the top-n must keep apart), and the value sum within a few 1e-3 (with bf16 probabilities
// and values, whose roundings are 2^-9 relative each, rows dominated by one compressed value lose
// up to 0.013).  fp16's range is kept by power-of-two scales: one per query row and one per
// 64-key tile of compressed keys, which bring the largest magnitude to [2^14, 2^15) and
// [2^13, 2^14) (so the scores' precision does not depend on the inputs' magnitude), and one per
// 64-key value tile, zero unless the tile's largest magnitude reaches 2^14.  The query and key
// scales enter the score factor; against the largest value-tile scale s_ref of the sequence and
// KV head, a tile's probabilities are scaled by 2^(s_tile - s_ref) and the output by 2^s_ref.
//
// Compressed K / V tiles of 64 keys are written by compress_kv16_kernel in their LDS image, so
// they go global -> LDS as linear 16 KB runs (global_load_lds, 16 bytes a lane), double-buffered.
#include "fast_common.hpp"

namespace {
constexpr int WR = 16;        // query rows per wave
constexpr int NWV = 4;        // waves per workgroup of the second sweep (one per SIMD)
constexpr int RQ = WR * NWV;  // query rows per workgroup of the second sweep
constexpr int NWA = 8;        // waves per workgroup of the first sweep (two per SIMD)
constexpr int RA = WR * NWA;  // query rows per workgroup of the first sweep
constexpr int CK = 64;        // compressed keys per tile
constexpr int HD = 128;       // head dim
constexpr int TILE = CK * HD;
// One LDS staging buffer (bytes): the key tile (64 rows of 128 fp16, 16-byte chunks swizzled as
// swz128) and the value tile (V^T, 128 dims x 64 keys, fp16).
constexpr int L_KT = 0;
constexpr int L_VT = L_KT + TILE * 2;
constexpr int L_BUF = L_VT + TILE * 2;
}  // namespace

// Key and value tiles (written by compress_kv16_kernel): per (b, KV head) ceil(Nc / 64) tiles of
// 64 compressed keys, 8192 fp16 each (the block sums times 2^-s of the tile's scale s, a signed
// byte per tile), keys past Nc zero.
//  key tile:   row = key, 16-byte chunk c of the row at position c ^ (key & 15) (the swz128 image);
//  value tile: V^T, [128 dims][64 key slots]: in each 32-key half the slot of key offset o is
//              8 ((o & 15) >> 2) + 4 (o >> 4) + (o & 3), so lane group gi's 8 slots are the keys
//              4 gi .. 4 gi + 3 and 16 + 4 gi .. +3 of the half, the order its score registers of
//              the half's two 16-key M-blocks hold them in; 16-byte chunks XOR-swizzled by (dim & 7).
// Buffer: all key tiles, all value tiles, the key tiles' scale bytes, the value tiles' scale bytes.
__host__ __device__ __forceinline__ int kt16_pos(int key, int dim) {
  return key * HD + ((((dim >> 3) ^ (key & 15))) << 3) + (dim & 7);
}
__host__ __device__ __forceinline__ int vt16_slot(int dim, int key) {
  const int h = key >> 5, o = key & 31;
  const int s = 32 * h + 8 * ((o & 15) >> 2) + 4 * (o >> 4) + (o & 3);
  return dim * CK + (((s >> 3) ^ (dim & 7)) << 3) + (s & 7);
}

struct Kv16Layout {
  size_t ntiles;  // tiles of one kind: B * Hkv * ceil(Nc / 64)
  __host__ __device__ size_t kt() const { return 0; }
  __host__ __device__ size_t vt() const { return ntiles * TILE * 2; }
  __host__ __device__ size_t ks() const { return 2 * ntiles * TILE * 2; }
  __host__ __device__ size_t vs() const { return ks() + ntiles; }
  __host__ __device__ size_t bytes() const { return vs() + ntiles; }
};

// Power-of-two range scale of fp16 data whose largest magnitude is m: s with m 2^-s in
// [2^(lim - 1), 2^lim) (for m = 0: -lim), clamped to [-127, 127]; with nonneg, at least 0.
__device__ __forceinline__ int f16_range_scale(float m, int lim, bool nonneg) {
  int E = 0;
  (void)frexpf(m, &E);  // m in [2^(E - 1), 2^E)
  int s = E - lim;
  s = s < -127 ? -127 : (s > 127 ? 127 : s);
  return nonneg && s < 0 ? 0 : s;
}

__device__ __forceinline__ void gwait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The tiles of one (sequence b, KV head g) in the kv16 buffer.
struct GroupTiles {
  const _Float16* kt;  // key tiles
  const _Float16* vt;  // value tiles
  const uint8_t* ksc;  // key tile scales (signed bytes)
  const uint8_t* vsc;  // value tile scales
  int ntv;             // tiles
  __device__ GroupTiles(const unsigned char* kv16, const Dims& dm, int64_t b, int g) {
    ntv = (int)((dm.Nc + CK - 1) / CK);
    const Kv16Layout ly{(size_t)dm.B * dm.Hkv * ntv};
    const int64_t t0 = (b * dm.Hkv + g) * ntv;
    kt = (const _Float16*)(kv16 + ly.kt()) + t0 * TILE;
    vt = (const _Float16*)(kv16 + ly.vt()) + t0 * TILE;
    ksc = kv16 + ly.ks() + t0;
    vsc = kv16 + ly.vs() + t0;
  }
  // past the last tile (only importances of blocks no compressed key reaches are flushed there,
  // every probability is 0): the last one
  __device__ int clamp(int tile) const { return tile < ntv ? tile : ntv - 1; }
};

// Q of one row for every head of the group as B operands of the score products (step ks:
// Q[row][32 ks + 8 gi .. +8]), in fp16 times 2^-eq, eq the row's range scale (the four lane groups
// of a row share it); returns eq.
template <int G>
__device__ __forceinline__ int load_q16(const bf16* qrow, bool rvalid, int gi, f16x8 (&qf)[G][4]) {
  // two passes over the row (the second from cache), so that the bf16 and fp16 copies are never
  // live together
  float m = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 x = rvalid ? *(const bf16x8*)(qrow + h * HD + 32 * ks + 8 * gi) : zero8();
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)x[e]));
    }
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  const int eq = f16_range_scale(m, 15, false);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 x = rvalid ? *(const bf16x8*)(qrow + h * HD + 32 * ks + 8 * gi) : zero8();
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[h][ks][e] = (_Float16)ldexpf((float)x[e], -eq);
    }
  return eq;
}

// Scores S^T of 16-key M-block mb (keys 16 mb .. +16 of the staged key tile kts) for every head:
// each key fragment read from LDS feeds the G heads' products.  Lane (gi, c) gets the scores of
// keys 16 mb + 4 gi + j, j = 0..3, for row c.
template <int G>
__device__ __forceinline__ void scores16(const _Float16* kts, int mb, int c, int gi, const f16x8 (&qf)[G][4],
                                         f32x4 (&S)[G]) {
#pragma unroll
  for (int h = 0; h < G; ++h) S[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const f16x8 kf = *(const f16x8*)(kts + swz128(16 * mb + c, 4 * ks + gi));
#pragma unroll
    for (int h = 0; h < G; ++h) S[h] = mfma16h(kf, qf[h][ks], S[h]);
  }
}

// 4 x 4 transpose among a row's four lanes (lanes c, c + 16, c + 32, c + 48): on entry lane group
// gi holds items (mb, gi) in v0..v3 (mb = 0..3); on exit it holds items (gi, k) in w0..w3 (k = 0..3).
// Two exchange steps of gfx950's lane swaps (no LDS round trip): v_permlane32_swap trades the upper
// 32 lanes of its first operand with the lower 32 of its second (lane groups gi and gi ^ 2: v0 with
// v2, v1 with v3), v_permlane16_swap the odd 16-lane rows of its first operand with the even rows of
// its second (lane groups gi and gi ^ 1).
__device__ __forceinline__ void row_transpose4(float v0, float v1, float v2, float v3, float& w0, float& w1,
                                               float& w2, float& w3) {
  const auto a02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v2), false, false);
  const auto a13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v1), __float_as_uint(v3), false, false);
  const auto b01 = __builtin_amdgcn_permlane16_swap(a02[0], a13[0], false, false);
  const auto b23 = __builtin_amdgcn_permlane16_swap(a02[1], a13[1], false, false);
  w0 = __uint_as_float(b01[0]);
  w1 = __uint_as_float(b01[1]);
  w2 = __uint_as_float(b23[0]);
  w3 = __uint_as_float(b23[1]);
}

// The value of lane group gi - 1 (group 3 for gi = 0) of the same row, by lane swaps: odd lane
// groups take their even neighbour directly, even ones the neighbour of their opposite group.
__device__ __forceinline__ float row_rotate1(float x) {
  const int gi = (threadIdx.x & 63) >> 4;
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // odd groups: a[0] = group gi - 1
  const auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned y = gi < 2 ? b[1] : b[0];                              // group gi ^ 2
  const auto d = __builtin_amdgcn_permlane16_swap(y, y, false, false);  // even groups: d[1] = y of gi + 1
  return __uint_as_float((gi & 1) ? a[0] : d[1]);
}

// Stores the importance of one row for a tile's 32 selection blocks of 32 tokens, j0 .. j0 + 31
// (blocks after jmax are not written): on entry lane group gi holds blocks j0 + 8 mb + 2 gi in
// a0..a3 and j0 + 8 mb + 2 gi + 1 in b0..b3; after two transposes it holds blocks j0 + 8 gi .. +7
// and stores them as 32 contiguous bytes.
__device__ __forceinline__ void store_imp_tile32(float* __restrict__ imp_row, int64_t j0, int64_t jmax, float a0,
                                                 float a1, float a2, float a3, float b0, float b1, float b2,
                                                 float b3) {
  const int gi = (threadIdx.x & 63) >> 4;
  float w[8];
  row_transpose4(a0, a1, a2, a3, w[0], w[2], w[4], w[6]);
  row_transpose4(b0, b1, b2, b3, w[1], w[3], w[5], w[7]);
  const int64_t j = j0 + 8 * gi;  // w[0..7] are blocks j .. j + 7
  if (j + 7 <= jmax && (((uintptr_t)(imp_row + j)) & 15) == 0) {
    *(float4*)(imp_row + j) = make_float4(w[0], w[1], w[2], w[3]);
    *(float4*)(imp_row + j + 4) = make_float4(w[4], w[5], w[6], w[7]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (j + e <= jmax) imp_row[j + e] = w[e];
  }
}

// ---------------------------------------------------------------------------
// First sweep: the log-sum-exp of every (video row, head), written to lse (natural log; -inf for a
// row with no visible compressed block).  Eight waves of 16 rows each (two per SIMD: no value
// accumulators here, so a wave fits in half the register file), the key tiles staged once for 128
// rows.  Each lane sums over its own keys in log2 units y = score c2: the sum of 2^(y - mr) against
// a whole-number reference mr, the largest floor(y) so far (updated per 32 keys).  When mr moves the
// sum is rescaled by an exact power of two (ldexp), so every term is below 2 and no step branches (the two waves on a
// SIMD overlap one's products with the other's exponentials).  The four lanes of a row are merged
// at the end.
template <int G>
__global__ void __attribute__((amdgpu_flat_work_group_size(NWA * 64, NWA * 64), amdgpu_waves_per_eu(2, 2)))
cmp_lse_kernel(const bf16* __restrict__ q, const unsigned char* __restrict__ kv16, const uint8_t* __restrict__ vid,
               float* __restrict__ lse, Dims dm, int ntiles) {
  __shared__ __attribute__((aligned(16))) _Float16 kbuf[2][TILE];
  __shared__ int s_any;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, gi = l >> 4, c = l & 15;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  int unit, rank;
  if (!xcd_remap(blockIdx.x, (int)(dm.B * dm.Hkv), ntiles, &unit, &rank)) return;
  const int64_t b = unit / dm.Hkv;
  const int g = unit % dm.Hkv;
  const int64_t rt0 = (int64_t)(ntiles - 1 - rank) * RA;  // heaviest row tiles first
  const GroupTiles gt(kv16, dm, b, g);
  if (tid == 0) s_any = 0;
  __syncthreads();
  if (tid < RA) {
    const int64_t rr = rt0 + tid;
    if (rr < dm.Tq && (!vid || vid[b * dm.Tq + rr])) s_any = 1;
  }
  __syncthreads();
  if (!s_any) return;

  const int64_t r = rt0 + WR * w + c;  // this lane's query row
  const bool rvalid = r < dm.Tq;
  const bool isv = rvalid && (!vid || vid[b * dm.Tq + r]);
  const int nv = rvalid ? (int)cmp_visible(dm.q0 + r, dm.l, dm.d, dm.Nc) : 0;
  const int64_t rlast = (rt0 + RA < dm.Tq ? rt0 + RA : dm.Tq) - 1;
  const int nvmax = (int)cmp_visible(dm.q0 + rlast, dm.l, dm.d, dm.Nc);
  const int nvmin = (int)cmp_visible(dm.q0 + rt0, dm.l, dm.d, dm.Nc);
  const float c2 = dm.scale * LOG2E_F;
  f16x8 qf[G][4];
  const int eq = load_q16<G>(q + ((b * dm.Tq + (rvalid ? r : 0)) * dm.Hq + (int64_t)g * G) * HD, rvalid, gi, qf);
  auto stage_k = [&](int tile, int bi) {
    stage_lin16k((bf16*)kbuf[bi], (const bf16*)(gt.kt + (int64_t)gt.clamp(tile) * TILE), wu, NWA, l);
  };

  constexpr float kNoKey = -1e30f;  // reference before the first visible key (below every score)
  float mr[G], ls[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mr[h] = kNoKey;
    ls[h] = 0.f;
  }
  // one 16-key M-block's scores; MASK: register j counts only when j < lm (else -inf)
  // two 16-key M-blocks' scores (keys 16 mb .. +32); MASK: register j of block a counts only when
  // j < lm[a] (else -inf)
  auto lse_pair = [&](const f32x4 (&Sa)[G], const f32x4 (&Sb)[G], float ct, int lma, int lmb, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = (MASK && j >= lma) ? -INFINITY : Sa[h][j];
        v[4 + j] = (MASK && j >= lmb) ? -INFINITY : Sb[h][j];
      }
      const float bm = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
      const float mn = fmaxf(mr[h], floorf(bm * ct));
      float acc = ldexpf(ls[h], (int)fmaxf(mr[h] - mn, -256.f));
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += fexp2(fmaf(v[j], ct, -mn));
      ls[h] = acc;
      mr[h] = mn;
    }
  };
  // Score register j of M-block mb of tile `tile` holds compressed key 64 tile + 16 mb + 4 gi + j
  auto lim_of = [&](int tile, int mb) { return nv - (tile * CK + 16 * mb + 4 * gi); };
  auto lse_tile = [&](int tile, int bi, auto mask_c) {
    const float ct = ldexpf(c2, eq + (int)(int8_t)gt.ksc[gt.clamp(tile)]);  // log2 units per raw score
#pragma unroll
    for (int mb = 0; mb < 4; mb += 2) {
      f32x4 Sa[G], Sb[G];
      scores16<G>(kbuf[bi], mb, c, gi, qf, Sa);
      scores16<G>(kbuf[bi], mb + 1, c, gi, qf, Sb);
      lse_pair(Sa, Sb, ct, lim_of(tile, mb), lim_of(tile, mb + 1), mask_c);
    }
  };
  // A tile whose keys are all visible, after the first: the terms 2^(y - mr) against the reference
  // as it stands, without the per-block maxima.  Their sum over the tile must stay below 2^100 for
  // every lane (else false: the tile is redone by lse_tile from the unchanged state); then the
  // running sum is brought back below 2^32 by an exact power of two.  The reference stays within
  // 2^13 of the row's largest term (a sum of at most 2^13 terms only passes 2^32 with a term above
  // 2^19), so no term that matters underflows.
  auto lse_tile_fast = [&](int tile, int bi) -> bool {
    const float ct = ldexpf(c2, eq + (int)(int8_t)gt.ksc[gt.clamp(tile)]);
    float ts[G];
#pragma unroll
    for (int mb = 0; mb < 4; mb += 2) {
      // both M-blocks' key fragments read once; head by head, the next head's two score chains go
      // out before this head's exponentials
      f16x8 k0[4], k1[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        k0[ks] = *(const f16x8*)(kbuf[bi] + swz128(16 * mb + c, 4 * ks + gi));
        k1[ks] = *(const f16x8*)(kbuf[bi] + swz128(16 * (mb + 1) + c, 4 * ks + gi));
      }
      auto head_scores = [&](int h, f32x4& A, f32x4& B) {
        A = f32x4{0.f, 0.f, 0.f, 0.f};
        B = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          A = mfma16h(k0[ks], qf[h][ks], A);
          B = mfma16h(k1[ks], qf[h][ks], B);
        }
      };
      f32x4 Sa, Sb;
      head_scores(0, Sa, Sb);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        f32x4 Na, Nb;
        if (h + 1 < G) head_scores(h + 1, Na, Nb);
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) a += fexp2(fmaf(Sa[j], ct, -mr[h])) + fexp2(fmaf(Sb[j], ct, -mr[h]));
        ts[h] = mb ? ts[h] + a : a;
        if (h + 1 < G) {
          Sa = Na;
          Sb = Nb;
        }
      }
    }
    bool ok = true;
#pragma unroll
    for (int h = 0; h < G; ++h) ok = ok && ts[h] < 0x1p100f;  // false for inf and NaN
    if (__builtin_amdgcn_ballot_w64(!ok)) return false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float acc = ls[h] + ts[h];
      const int e = acc >= 0x1p32f ? __builtin_amdgcn_frexp_expf(acc) : 0;
      ls[h] = ldexpf(acc, -e);
      mr[h] += (float)e;
    }
    return true;
  };
  const int nt1 = (nvmax + CK - 1) / CK;
  if (nt1 > 0) {
    stage_k(0, 0);
    gwait_loads();
  }
  __syncthreads();
  for (int tile = 0; tile < nt1; ++tile) {
    const int bi = tile & 1;
    if (tile + 1 < nt1) stage_k(tile + 1, bi ^ 1);
    if ((tile + 1) * CK <= nvmin) {
      if (tile == 0 || !lse_tile_fast(tile, bi)) lse_tile(tile, bi, std::false_type{});
    } else {
      lse_tile(tile, bi, std::true_type{});
    }
    gwait_loads();
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = mr[h];
    M = fmaxf(M, __shfl_xor(M, 16, 64));
    M = fmaxf(M, __shfl_xor(M, 32, 64));
    float tot = ls[h] * fexp2(mr[h] - M);
    tot += __shfl_xor(tot, 16, 64);
    tot += __shfl_xor(tot, 32, 64);
    if (isv && gi == 0)
      lse[(b * dm.Tq + r) * dm.Hq + (int64_t)g * G + h] = M > kNoKey ? (M + flog2(tot)) * LN2_F : -INFINITY;
  }
}

// Second sweep: exact probabilities from the log-sum-exp, the value sum and the block importance.
// Four waves of 16 rows each, one per SIMD (the value accumulators of all G heads fill the
// accumulation registers).  LS: tokens per selection block (32, 64 or 128).  Compressed key i spans
// tokens [16 i, 16 i + 31], so block J takes half of its first straddling key, the keys inside it
// whole and half of its last straddling key: LS = 32: keys 2J - 1 (half), 2J, 2J + 1 (half);
// LS = 64: 4J - 1 (half) .. 4J + 3 (half); LS = 128: 8J - 1 (half) .. 8J + 7 (half).  A lane holds
// four consecutive keys 4k .. 4k + 3 of its row: with LS = 32 they make blocks 2k and 2k + 1, with
// LS = 64 block k, with LS = 128 half of block k / 2 (the lane groups gi, gi ^ 1 are joined with one
// lane exchange); the half share of a lane's first key comes from the previous lane group.
template <int G, int LS>
__global__ void __attribute__((amdgpu_flat_work_group_size(NWV * 64, NWV * 64), amdgpu_waves_per_eu(1, 1)))
cmp_group_kernel(const bf16* __restrict__ q, const unsigned char* __restrict__ kv16, const uint8_t* __restrict__ vid,
                 const float* __restrict__ lse, bf16* __restrict__ o_bf, float* __restrict__ o_f32,
                 float* __restrict__ imp, Dims dm, int ntiles) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_any, s_scale;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, gi = l >> 4, c = l & 15;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  int unit, rank;
  if (!xcd_remap(blockIdx.x, (int)(dm.B * dm.Hkv), ntiles, &unit, &rank)) return;
  const int64_t b = unit / dm.Hkv;
  const int g = unit % dm.Hkv;
  const int64_t rt0 = (int64_t)(ntiles - 1 - rank) * RQ;  // heaviest row tiles first
  const GroupTiles gt(kv16, dm, b, g);

  // skip row tiles without a video row; the largest value-tile scale of this (sequence, KV head)
  if (tid == 0) {
    s_any = 0;
    s_scale = 0;
  }
  __syncthreads();
  if (tid < RQ) {
    const int64_t rr = rt0 + tid;
    if (rr < dm.Tq && (!vid || vid[b * dm.Tq + rr])) s_any = 1;
  }
  for (int i = tid; i < gt.ntv; i += blockDim.x) {
    const int sc = gt.vsc[i];
    if (sc) atomicMax(&s_scale, sc);
  }
  __syncthreads();
  if (!s_any) return;
  const int s_ref = s_scale;  // the value accumulators hold O 2^-s_ref

  const int64_t r = rt0 + WR * w + c;  // this lane's query row
  const bool rvalid = r < dm.Tq;
  const bool isv = rvalid && (!vid || vid[b * dm.Tq + r]);
  const int nv = rvalid ? (int)cmp_visible(dm.q0 + r, dm.l, dm.d, dm.Nc) : 0;
  const int64_t rlast = (rt0 + RQ < dm.Tq ? rt0 + RQ : dm.Tq) - 1;
  const int nvmax = (int)cmp_visible(dm.q0 + rlast, dm.l, dm.d, dm.Nc);
  const int nvmin = (int)cmp_visible(dm.q0 + rt0, dm.l, dm.d, dm.Nc);
  const float c2 = dm.scale * LOG2E_F;

  f16x8 qf[G][4];
  const int eq = load_q16<G>(q + ((b * dm.Tq + (rvalid ? r : 0)) * dm.Hq + (int64_t)g * G) * HD, rvalid, gi, qf);

  auto lds_at = [&](int bi, int off) { return smem + bi * L_BUF + off; };
  auto stage_k = [&](int tile, int bi) {
    stage_lin16k((bf16*)lds_at(bi, L_KT), (const bf16*)(gt.kt + (int64_t)gt.clamp(tile) * TILE), wu, NWV, l);
  };
  auto stage_v = [&](int tile, int bi) {
    stage_lin16k((bf16*)lds_at(bi, L_VT), (const bf16*)(gt.vt + (int64_t)gt.clamp(tile) * TILE), wu, NWV, l);
  };
  // log2 units per raw score unit of tile `tile`
  auto c2_of = [&](int tile) { return ldexpf(c2, eq + (int)(int8_t)gt.ksc[gt.clamp(tile)]); };
  // Score register j of M-block mb of tile `tile` holds compressed key tile CK + 16 mb + 4 gi + j;
  // it is visible when j < lim
  auto lim_of = [&](int tile, int mb) { return nv - (tile * CK + 16 * mb + 4 * gi); };
  auto full = [&](int tile) { return (tile + 1) * CK <= nvmin; };

  // log2-domain normaliser of each head from the first sweep (+inf, every p zero, for rows with
  // no visible block and rows that are not computed)
  float L2[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    L2[h] = (isv && nv > 0) ? lse[(b * dm.Tq + r) * dm.Hq + (int64_t)g * G + h] * LOG2E_F : INFINITY;

  // ---- sweep 2: probabilities, value sum, importance
  int64_t jmax = -1;  // this lane's row's last candidate block (-1: text row or past the end)
  if (isv) {
    const int64_t jt = (dm.q0 + r) / dm.ls;
    jmax = jt < dm.Ns ? jt : dm.Ns - 1;
  }
  float* imp_row = imp ? imp + ((b * dm.Tq + (rvalid ? r : 0)) * dm.Hkv + g) * dm.Ns : nullptr;
  f32x4 O[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int db = 0; db < 8; ++db) O[h][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  int sh_prev = 0;    // the range scale shift folded into L2
  // half share of the last compressed key before this lane's first (64-token blocks: of the previous
  // tile's last block, in lane group 0; else of the previous M-block's, lane group 3's shifted)
  float rprev = 0.f;
  // one tile: per 32-key half, the scores and probabilities of its two M-blocks, the value product and
  // the importance of their two selection blocks per lane; MASK as in sweep 1.  The value
  // tile's range scale sh = s_tile - s_ref (<= 0) enters the probabilities' exponent; their sums
  // over the heads are scaled back by 2^-sh for the importance.
  auto pv_tile = [&](int tile, int bi, int sh, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    const float ct = c2_of(tile);
    const float unscale = ldexpf(1.f, -sh);
    // L2 - sh for this tile (L2 holds L2 - sh of the previous tile)
#pragma unroll
    for (int h = 0; h < G; ++h) L2[h] += (float)(sh_prev - sh);
    sh_prev = sh;
    // importance of this lane's row in the tile: block 16 tile + 4 mb + gi for mb = 0..3
    float im0 = 0.f, im1 = 0.f, im2 = 0.f, im3 = 0.f;
    // with 64-token blocks the carry-outs of the four M-blocks, with 32-token blocks the second block of each
    float jm0 = 0.f, jm1 = 0.f, jm2 = 0.f, jm3 = 0.f;
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      float P0[4], P1[4];  // sums over the heads
      const int lm0 = lim_of(tile, 2 * half), lm1 = lim_of(tile, 2 * half + 1);
      // key fragments of both M-blocks and the value fragments (dims 16 db + c, this lane group's
      // 8 key slots), read once for all heads
      const _Float16* kts = (const _Float16*)lds_at(bi, L_KT);
      const _Float16* vts = (const _Float16*)lds_at(bi, L_VT);
      f16x8 k0[4], k1[4], vr[8];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        k0[ks] = *(const f16x8*)(kts + swz128(16 * (2 * half) + c, 4 * ks + gi));
        k1[ks] = *(const f16x8*)(kts + swz128(16 * (2 * half + 1) + c, 4 * ks + gi));
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int dim = 16 * db + c;
        vr[db] = *(const f16x8*)(vts + dim * CK + (((4 * half + gi) ^ (dim & 7)) << 3));
      }
      // head by head: the next head's two score chains go out before this head's probabilities,
      // and this head's value products (O^T += Vc^T P^T over the half's 32 keys) right after
      // them, so the matrix products of one head run beside the exponentials of the next and only
      // two heads' scores are live at a time
      auto head_scores = [&](int h, f32x4& A, f32x4& B) {
        A = f32x4{0.f, 0.f, 0.f, 0.f};
        B = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          A = mfma16h(k0[ks], qf[h][ks], A);
          B = mfma16h(k1[ks], qf[h][ks], B);
        }
      };
      f32x4 Sa, Sb;
      head_scores(0, Sa, Sb);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        f32x4 Na, Nb;
        if (h + 1 < G) head_scores(h + 1, Na, Nb);
        f16x8 pb;  // P^T operand of the half's 32 keys: M-block 2 half in slots 0..3, the next in 4..7
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float pa = fexp2(fmaf(Sa[j], ct, -L2[h]));
          float pc = fexp2(fmaf(Sb[j], ct, -L2[h]));
          if constexpr (MASK) {
            pa = j < lm0 ? pa : 0.f;
            pc = j < lm1 ? pc : 0.f;
          }
          P0[j] = h ? P0[j] + pa : pa;
          P1[j] = h ? P1[j] + pc : pc;
          pb[j] = (_Float16)pa;
          pb[4 + j] = (_Float16)pc;
        }
#pragma unroll
        for (int db = 0; db < 8; ++db) O[h][db] = mfma16h(vr[db], pb, O[h][db]);
        if (h + 1 < G) {
          Sa = Na;
          Sb = Nb;
        }
      }
      // importance of this lane's row from M-blocks mb = 2 half, 2 half + 1 (keys 4k .. 4k + 3,
      // k = 16 tile + 4 mb + gi)
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const float* P = mi ? P1 : P0;
        const int64_t kq = (int64_t)tile * 16 + 4 * (2 * half + mi) + gi;
        const float t = 0.5f * P[3] * unscale;
        if constexpr (LS == 64) {
          // block k without the half of key 4k - 1 (x), and the half of key 4k + 3 that block k + 1
          // takes (t); the carries are added once per tile, after the transpose
          const float x = (P[0] + P[1] + P[2]) * unscale + t;
          if (mi == 0) {
            im0 = half ? im0 : x;
            im2 = half ? x : im2;
            jm0 = half ? jm0 : t;
            jm2 = half ? t : jm2;
          } else {
            im1 = half ? im1 : x;
            im3 = half ? x : im3;
            jm1 = half ? jm1 : t;
            jm3 = half ? t : jm3;
          }
          continue;
        }
        const float rc = row_rotate1(t);  // t of lane group gi - 1, or of group 3 for gi = 0
        const float carry = gi ? rc : rprev;   // half of the key before this lane's first
        rprev = rc;
        if constexpr (LS == 32) {
          const float hp1 = 0.5f * P[1] * unscale;
          const float b0 = carry + P[0] * unscale + hp1;  // block 2k
          const float b1 = hp1 + P[2] * unscale + t;      // block 2k + 1
          if (mi == 0) {
            im0 = half ? im0 : b0;
            im2 = half ? b0 : im2;
            jm0 = half ? jm0 : b1;
            jm2 = half ? b1 : jm2;
          } else {
            im1 = half ? im1 : b0;
            im3 = half ? b0 : im3;
            jm1 = half ? jm1 : b1;
            jm3 = half ? b1 : jm3;
          }
        } else {
          // lane groups 2m, 2m + 1 hold block k / 2: keys 8J .. 8J + 3 whole (and the half of 8J - 1),
          // keys 8J + 4 .. 8J + 6 whole and half of 8J + 7
          const float v = (gi & 1) ? (P[0] + P[1] + P[2]) * unscale + t
                                   : (P[0] + P[1] + P[2] + P[3]) * unscale + carry;
          const float blk = v + __shfl_xor(v, 16, 64);
          if (imp_row && !(gi & 1)) {
            const int64_t J = kq >> 1;
            if (J <= jmax) imp_row[J] = blk;
          }
        }
      }
    }
    if constexpr (LS == 64) {
      // lane group gi now holds blocks 16 tile + 4 gi + q (q = 0..3): X[q] and the carry-outs T[q];
      // block 4 gi + q takes T[q - 1], and for q = 0 the last carry-out of lane group gi - 1, or for
      // gi = 0 that of the previous tile's last block
      float X0, X1, X2, X3, T0, T1, T2, T3;
      row_transpose4(im0, im1, im2, im3, X0, X1, X2, X3);
      row_transpose4(jm0, jm1, jm2, jm3, T0, T1, T2, T3);
      const float R = row_rotate1(T3);
      const float cin = gi ? R : rprev;
      rprev = R;  // for lane group 0: this tile's block 15
      if (imp_row) {
        const int64_t j = (int64_t)tile * 16 + 4 * gi;
        const float w0 = X0 + cin, w1 = X1 + T0, w2 = X2 + T1, w3 = X3 + T2;
        if (j + 3 <= jmax && (((uintptr_t)(imp_row + j)) & 15) == 0) {
          *(float4*)(imp_row + j) = make_float4(w0, w1, w2, w3);
        } else {
          if (j <= jmax) imp_row[j] = w0;
          if (j + 1 <= jmax) imp_row[j + 1] = w1;
          if (j + 2 <= jmax) imp_row[j + 2] = w2;
          if (j + 3 <= jmax) imp_row[j + 3] = w3;
        }
      }
    } else if constexpr (LS == 32) {
      if (imp_row) store_imp_tile32(imp_row, (int64_t)tile * 32, jmax, im0, im1, im2, im3, jm0, jm1, jm2, jm3);
    }
  };
  const int nt2 = nvmax > 0 ? nvmax / CK + 1 : 0;
  if (nt2 > 0) {
    stage_k(0, 0);
    stage_v(0, 0);
    gwait_loads();
  }
  __syncthreads();
  for (int tile = 0; tile < nt2; ++tile) {
    const int bi = tile & 1;
    if (tile + 1 < nt2) {
      stage_k(tile + 1, bi ^ 1);
      stage_v(tile + 1, bi ^ 1);
    }
    // fp16 range of the value tile: its probabilities times 2^(s_tile - s_ref) <= 1
    const int sh = (int)gt.vsc[gt.clamp(tile)] - s_ref;
    if (full(tile))
      pv_tile(tile, bi, sh, std::false_type{});
    else
      pv_tile(tile, bi, sh, std::true_type{});
    gwait_loads();
    __syncthreads();
  }
  // blocks up to the row's own block that no compressed block reaches (1024 tokens a 64-key tile)
  if (imp_row) {
    for (int64_t J = (int64_t)nt2 * (1024 / LS) + gi; J <= jmax; J += 4) imp_row[J] = 0.f;
  }

  if (!isv) return;
  const int64_t orow = (b * dm.Tq + r) * dm.Hq + (int64_t)g * G;
  const float oscale = ldexpf(1.f, s_ref);
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d0 = 16 * db + 4 * gi;
      f32x4 o4 = O[h][db];
      if (s_ref) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] *= oscale;
      }
      if (o_f32) *(f32x4*)(o_f32 + (orow + h) * HD + d0) = o4;
      if (o_bf) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)o4[e];
        *(bf16x4*)(o_bf + (orow + h) * HD + d0) = v4;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Key and value tiles for cmp_group_kernel: the fp32 block sums of a 64-key tile (weights w over
// l tokens, stride d), their range scale s (keys: the largest magnitude times 2^-s lies in
// [2^13, 2^14); values: zero unless the largest magnitude reaches 2^14) and the sums times 2^-s in
// fp16, at kt16_pos (keys) or vt16_slot (values).  One workgroup per
// (b, KV head, 64-key tile) and kind: blocks [0, n) make key tiles, [n, 2n) value tiles.  A tile
// leaves as one contiguous 16 KB run.
__global__ void __launch_bounds__(256) compress_kv16_kernel(const bf16* __restrict__ k, const bf16* __restrict__ v,
                                                            const float* __restrict__ w_k,
                                                            const float* __restrict__ w_v,
                                                            unsigned char* __restrict__ out, int64_t T_len, int H,
                                                            int l, int d, int64_t Nc, int ntv) {
  __shared__ float ws[64];
  __shared__ float s_max[4];
  __shared__ __attribute__((aligned(16))) float s_v[CK * (HD + 1)];  // fp32 sums, padded rows
  __shared__ __attribute__((aligned(16))) _Float16 s_t[TILE];
  const Kv16Layout ly{(size_t)gridDim.x / 2};
  const bool is_v = blockIdx.x >= ly.ntiles;
  const int64_t id = is_v ? blockIdx.x - (int64_t)ly.ntiles : blockIdx.x;  // (b, h, tile) index
  const int tile = (int)(id % ntv);
  const int64_t bh = id / ntv;
  const int h = (int)(bh % H);
  const int64_t b = bh / H;
  const bf16* x = is_v ? v : k;
  const float* w = is_v ? w_v : w_k;
  for (int m = threadIdx.x; m < l; m += blockDim.x) ws[m] = w[m];
  __syncthreads();
  float mx = 0.f;
  for (int it = threadIdx.x; it < CK * (HD / 8); it += blockDim.x) {
    const int key = it >> 4, c8 = it & 15;
    const int64_t i = (int64_t)tile * CK + key;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (i < Nc) {
      const bf16* src = x + ((b * T_len + i * d) * H + h) * (int64_t)HD + c8 * 8;
      for (int m = 0; m < l; ++m) {
        const bf16x8 u = *(const bf16x8*)(src + (int64_t)m * H * HD);
        const float wm = ws[m];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(wm, (float)u[e], acc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s_v[key * (HD + 1) + c8 * 8 + e] = acc[e];
      mx = fmaxf(mx, fabsf(acc[e]));
    }
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = mx;
  __syncthreads();
  const int sc = f16_range_scale(fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3])), 14, is_v);
  for (int it = threadIdx.x; it < CK * HD; it += blockDim.x) {
    const int key = it >> 7, dim = it & 127;
    s_t[is_v ? vt16_slot(dim, key) : kt16_pos(key, dim)] = (_Float16)ldexpf(s_v[key * (HD + 1) + dim], -sc);
  }
  __syncthreads();
  unsigned char* dst = out + (is_v ? ly.vt() : ly.kt()) + (size_t)id * TILE * 2;
  for (int c = threadIdx.x; c < TILE / 8; c += blockDim.x) *(f16x8*)(dst + c * 16) = *(const f16x8*)(s_t + c * 8);
  if (threadIdx.x == 0) out[(is_v ? ly.vs() : ly.ks()) + id] = (unsigned char)(int8_t)sc;
}

static size_t kv16_ntiles(const Dims& dm) { return (size_t)dm.B * dm.Hkv * ((dm.Nc + CK - 1) / CK); }

size_t kv16_tiles_bytes(const Dims& dm) { return Kv16Layout{kv16_ntiles(dm)}.bytes(); }

hipError_t launch_compress_kv16(const Dims& dm, const void* k, const float* w_k, const void* v, const float* w_v,
                                void* out, hipStream_t s) {
  if (dm.Nc <= 0 || dm.B <= 0) return hipSuccess;
  if (dm.D != HD || dm.l > 64) return hipErrorInvalidValue;
  const size_t n = kv16_ntiles(dm);
  compress_kv16_kernel<<<(unsigned)(2 * n), 256, 0, s>>>((const bf16*)k, (const bf16*)v, w_k, w_v,
                                                        (unsigned char*)out, dm.T, dm.Hkv, dm.l, dm.d, dm.Nc,
                                                        (int)((dm.Nc + CK - 1) / CK));
  return hipGetLastError();
}

bool cmp_group_supported(const Dims& dm) {
  return dm.D == HD && dm.G >= 4 && dm.G <= 7 && dm.l == 32 && dm.d == 16 &&
         (dm.ls == 32 || dm.ls == 64 || dm.ls == 128);
}

hipError_t launch_cmp_group(const Dims& dm, const void* q, const void* kv16, const uint8_t* vid, void* o_bf,
                            float* o32, float* lse, float* imp, hipStream_t s) {
  if (dm.Tq <= 0 || dm.B <= 0) return hipSuccess;
  if (!cmp_group_supported(dm) || !kv16 || !lse) return hipErrorInvalidValue;
  const size_t shm = (size_t)2 * L_BUF;
  const int units = (int)(dm.B * dm.Hkv);
  const int ta = (int)((dm.Tq + RA - 1) / RA), tb = (int)((dm.Tq + RQ - 1) / RQ);
  auto go = [&](auto lse_kernel, auto kernel) -> hipError_t {
    lse_kernel<<<dim3(xcd_grid(units, ta)), dim3(NWA * 64), 0, s>>>((const bf16*)q, (const unsigned char*)kv16, vid,
                                                                    lse, dm, ta);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    kernel<<<dim3(xcd_grid(units, tb)), dim3(NWV * 64), shm, s>>>((const bf16*)q, (const unsigned char*)kv16, vid,
                                                                  lse, (bf16*)o_bf, o32, imp, dm, tb);
    return hipGetLastError();
  };
  auto by_ls = [&](auto lse_kernel, auto k32, auto k64, auto k128) -> hipError_t {
    return dm.ls == 32 ? go(lse_kernel, k32) : dm.ls == 128 ? go(lse_kernel, k128) : go(lse_kernel, k64);
  };
  switch (dm.G) {
    case 4: return by_ls(cmp_lse_kernel<4>, cmp_group_kernel<4, 32>, cmp_group_kernel<4, 64>, cmp_group_kernel<4, 128>);
    case 5: return by_ls(cmp_lse_kernel<5>, cmp_group_kernel<5, 32>, cmp_group_kernel<5, 64>, cmp_group_kernel<5, 128>);
    case 6: return by_ls(cmp_lse_kernel<6>, cmp_group_kernel<6, 32>, cmp_group_kernel<6, 64>, cmp_group_kernel<6, 128>);
    case 7: return by_ls(cmp_lse_kernel<7>, cmp_group_kernel<7, 32>, cmp_group_kernel<7, 64>, cmp_group_kernel<7, 128>);
    default: return hipErrorInvalidValue;
  }
}
