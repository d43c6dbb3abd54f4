// Compression-branch attention fused with block importance, bf16 MFMA on gfx950.
//
// What it computes (top168.com digest of VideoNSA, section 一: the selection
// branch scores segments by importance, read here from the compression
// branch's probabilities): for each video row t and head h,
//   p_i = softmax_i(scale * <q_t,h, kc_i>) over the compressed blocks i whose
//         tokens all lie at or before t,  o_cmp = sum_i p_i vc_i,
//   imp[t, g, j] = sum_{h in group g} sum_i frac(i, j) p_{h,i},
// with compressed block 32 / stride 16 and selection block 64, so that block j
// takes compressed blocks 4j .. 4j+2 whole and half of 4j-1 and 4j+3.
//
// This kernel serves 8 query heads per KV head and compressed keys / values that
// the caller passes in; with 4..7 heads per KV head the layer's own compression
// runs on cmp_group_kernel (fp16 key / value tiles, all heads of a group in one
// wave).
//
// Layout on the chip: one workgroup = 32 consecutive query rows x the G heads
// of one KV group, one wave per head.  Scores are formed transposed,
// S^T = Kc Q^T (v_mfma_f32_32x32x16_bf16, keys on M, the wave's 32 rows on N),
// so each lane owns one (row, head) column: its softmax statistics need one
// cross-half exchange, and the score registers are already the B operand of
// O^T += Vc^T P^T after a bf16 conversion.  Vc^T comes from LDS with the
// gfx950 transposing read (ds_read_b64_tr_b16); Kc is read in A layout.
// Compressed K/V tiles of 64 keys go global -> LDS directly (global_load_lds,
// 16 bytes a lane), double-buffered: the next tile streams in while the
// current one is consumed, without staging registers.  LDS rows are 256 bytes
// with their 16-byte chunks XOR-swizzled by the row index, so the A-layout and
// transposing reads of 16 consecutive rows hit distinct banks.
//
// The importance needs the final softmax normaliser, so the kernel makes two
// sweeps over the keys: the first forms the log-sum-exp (Q Kc^T only), the
// second exact probabilities, the value sum and the importance.  Each lane's
// probabilities come in aligned runs of 4 compressed blocks (one selection
// block); the half-block shares cross lanes with one xor-32 shuffle and a
// carry, the G heads are summed in a fixed order through LDS, so the result is
// deterministic.
//
// Compressed K and V may come split (compressed inside the layer from an fp32
// sum).  K then comes as a bf16 high part plus the remainder in fp8 (e4m3) with
// one power-of-two scale per 32 channels of a key (compress_k8_kernel); the
// remainder enters every score through the scaled fp8 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4) against an fp8 copy of Q with one scale
// per row.  The remainder is below 2^-8 of the key and its product carries an
// error near 2^-4 of itself, so the scores keep about 2^-12 relative precision
// instead of the 2^-8 of bf16 keys, at half the matrix-core time of a second
// bf16 product.  V comes as bf16 high + low parts; both enter the value
// sum for workgroups whose rows see fewer than kVloBelow compressed blocks,
// longer rows use the high part alone.
#include "fast_common.hpp"

namespace {
constexpr int CQ = 32;         // query rows per workgroup
constexpr int CK = 64;         // compressed keys per tile
constexpr int HD = 128;        // head dim
constexpr int TILE = CK * HD;  // bf16 elements of one staged array
// Rows that see fewer compressed blocks than this use the low parts of V too.  With few blocks
// one block's value dominates the output, so the bf16 rounding of Vc shows in it undamped; from
// a few hundred blocks on the softmax averages it down well below the bf16 output rounding.
// Scores always use both parts of K: the block importance that decides the top-n moves by
// up to a few 1e-3 with bf16 Kc.
constexpr int64_t kVloBelow = 256;

}  // namespace

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Instruction interleaving in the pipelined loop bodies: LLVM's AMDGPU scheduling groups (a
// group of n instructions of one kind, in order).
#define SG(kind, n) __builtin_amdgcn_sched_group_barrier(kind, n, 0)
constexpr int SG_VALU = 0x2, SG_MFMA = 0x8, SG_DSR = 0x100;

// Split keys, low part (compress_k8_kernel, launch_compress_k8): [B, Nc, Hkv, 128] bytes of fp8
// e4m3 in channel order plus [B, Nc, Hkv, 4] scale bytes (E8M0: 2^(byte - 127)), scale s for
// channels 32 s .. 32 s + 31.  Lane half hl of scaled MFMA c (32x32x64) reads channels
// [64 c + 16 hl, +16) and [64 c + 32 + 16 hl, +16) and supplies scale byte 2 c + hl (see the
// operand note in fast_common.hpp).
// Staged fp8 tile: 64 rows of 128 bytes, 16-byte chunk c of row r at chunk c ^ ((r >> 1) & 7), so
// the 16 lanes reading one chunk of 16 consecutive rows hit distinct banks.
__device__ __forceinline__ int swz8(int row, int c) { return row * 128 + ((c ^ ((row >> 1) & 7)) << 4); }

// Row stride (floats) of the per-head importance partials: 16 blocks + 1 pad, so 32 lanes
// writing one block of 32 rows and 16 lanes reading the 16 blocks of a row hit distinct banks.
constexpr int IPS = 17;

// The other lane half's value (lane l gets lane l ^ 32), with gfx950's v_permlane32_swap.
__device__ __forceinline__ float xchg32(float x, int hl) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(hl ? r[0] : r[1]);
}

// LDS image of one staging buffer (byte offsets): K high, [K low fp8, K scales,] V high[, V low]
template <bool SPLIT>
struct CmpLds {
  static constexpr int KH = 0;
  static constexpr int KL = TILE * 2;
  static constexpr int KS = KL + CK * HD;
  static constexpr int VH = SPLIT ? KS + CK * 4 : TILE * 2;
  static constexpr int VL = VH + TILE * 2;
  static constexpr int BUF = SPLIT ? VL + TILE * 2 : VH + TILE * 2;
};

// SPLIT: keys as bf16 high parts (kh) + fp8 low parts (kl8) with scales (ksc).
// ipart_bufs: 2 = importance partials double-buffered by tile parity, 1 = one buffer (one more
// barrier a tile; used where two do not fit in LDS).
template <bool SPLIT>
__global__ void __launch_bounds__(512) cmp_fast_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kh,
                                                       const uint8_t* __restrict__ kl8,
                                                       const uint8_t* __restrict__ ksc, const bf16* __restrict__ vh,
                                                       const bf16* __restrict__ vl, const uint8_t* __restrict__ vid,
                                                       bf16* __restrict__ o_bf, float* __restrict__ o_f32,
                                                       float* __restrict__ lse, float* __restrict__ imp, Dims dm,
                                                       int tile_lo, int ntiles, int ipart_bufs) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  using LY = CmpLds<SPLIT>;
  float* ipart0 = (float*)(smem + 2 * LY::BUF);  // [ipart_bufs][G][CQ][IPS]
  __shared__ int s_any;

  const int G = dm.G;
  const int nthr = G * 64;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, hl = l >> 5, n = l & 31;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index as a uniform value
  int unit, rank;
  if (!xcd_remap(blockIdx.x, (int)(dm.B * dm.Hkv), ntiles, &unit, &rank)) return;
  const int64_t b = unit / dm.Hkv;
  const int g = unit % dm.Hkv;
  const int64_t rt0 = (int64_t)(tile_lo + ntiles - 1 - rank) * CQ;  // row tiles [tile_lo, +ntiles), heaviest first

  if (tid == 0) s_any = 0;
  __syncthreads();
  if (tid < CQ) {
    const int64_t r = rt0 + tid;
    if (r < dm.Tq && (!vid || vid[b * dm.Tq + r])) s_any = 1;
  }
  __syncthreads();
  if (!s_any) return;

  // key counts fit in int: Nc < 2^27 for kv_len <= 2^31
  const int64_t rlast = (rt0 + CQ < dm.Tq ? rt0 + CQ : dm.Tq) - 1;
  const int nvmax = (int)cmp_visible(dm.q0 + rlast, dm.l, dm.d, dm.Nc);
  const int nvmin = (int)cmp_visible(dm.q0 + rt0, dm.l, dm.d, dm.Nc);  // row rt0 always exists
  const int64_t r = rt0 + n;
  const bool rvalid = r < dm.Tq;
  const bool isv = rvalid && (!vid || vid[b * dm.Tq + r]);
  const int64_t t = dm.q0 + r;
  const int nv = rvalid ? (int)cmp_visible(t, dm.l, dm.d, dm.Nc) : 0;
  const int h = g * G + w;
  const float c2 = dm.scale * LOG2E_F;

  // Q^T as the B operand: lane holds Q[row n][16 ks + 8 hl .. +8]
  bf16x8 qf[8];
  {
    const bf16* qrow = q + ((b * dm.Tq + (rvalid ? r : 0)) * dm.Hq + h) * (int64_t)HD + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = rvalid ? *(const bf16x8*)(qrow + 16 * ks) : zero8();
  }
  // fp8 copy of Q for the low parts of K: B operand of scaled MFMA c (channels 64 c .. 64 c + 63):
  // lane half hl holds the pieces [64 c + 16 hl, +16) and [64 c + 32 + 16 hl, +16) (the operand
  // byte order of fast_common.hpp), one power-of-two scale for the whole row
  i32x8 q8[2] = {};
  int q8s = 127;
  if constexpr (SPLIT) {
    const bf16* qn = q + ((b * dm.Tq + (rvalid ? r : 0)) * dm.Hq + h) * (int64_t)HD;
    bf16x8 pv[2][4];
    float m = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c) m = fmaxf(m, load_pieces(qn, 64 * c + 16 * hl, 64 * c + 32 + 16 * hl, rvalid, pv[c]));
    m = fmaxf(m, xchg32(m, hl));  // the row's other half
#pragma unroll
    for (int c = 0; c < 2; ++c) fp8_pieces(pv[c], m, q8[c], q8s);
  }

  // VLO: the low parts of V enter the value sum (see kVloBelow); a uniform choice per workgroup
  auto body = [&](auto vlo_c) {
  constexpr bool VLO = decltype(vlo_c)::value;
  const int64_t stride = (int64_t)dm.Hkv * HD;
  const int64_t base = (b * dm.Nc * dm.Hkv + g) * (int64_t)HD;
  auto lds_at = [&](int bufi, int off) { return smem + bufi * LY::BUF + off; };
  auto khs_of = [&](int bufi) { return (bf16*)lds_at(bufi, LY::KH); };
  auto vhs_of = [&](int bufi) { return (bf16*)lds_at(bufi, LY::VH); };
  auto vls_of = [&](int bufi) { return (bf16*)lds_at(bufi, LY::VL); };
  // Direct global -> LDS staging of the 64 rows [tile CK, +CK) of a [*, 128] bf16 array into a
  // swizzled tile (the swz128 layout): the tile takes 16 instructions of 64 lanes x 16 bytes,
  // instruction ins covers LDS chunks [64 ins, +64) (rows 4 ins .. 4 ins + 3) and goes to wave
  // ins mod G.  Rows at or past Nc repeat row Nc - 1 (finite data the masks never weight).
  auto stage64 = [&](bf16* lds, const bf16* src, int tile) {
    const bf16* st = src + (int64_t)tile * CK * stride;
    const int64_t left64 = dm.Nc - (int64_t)tile * CK;
    const int left = left64 < CK ? (int)left64 : CK;  // >= 0; 0 only for the flush tile past the end
    for (int ins = wu; ins < 16; ins += G) {
      const int row = ins * 4 + (l >> 4);
      const int c = (l & 15) ^ (row & 15);
      const int rr = row < left ? row : left - 1;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(st + (rr * (int)stride + c * 8)),
                                       (__attribute__((address_space(3))) void*)(lds + ins * 512), 16, 0, 0);
    }
  };
  // fp8 low parts: 8 instructions of 64 lanes x 16 bytes (rows 8 ins .. 8 ins + 7, the swz8
  // layout), then the 64 keys' scale words (one 4-byte load a lane) from the last wave
  auto stage_k = [&](int tile, int bufi, auto lo_c) {
    stage64(khs_of(bufi), kh + base, tile);
    if constexpr (decltype(lo_c)::value) {
      const int64_t left64 = dm.Nc - (int64_t)tile * CK;
      const int left = left64 < CK ? (int)left64 : CK;
      const int64_t key0 = (b * dm.Nc + (int64_t)tile * CK) * dm.Hkv + g;  // (key, head) row index
      unsigned char* lo = lds_at(bufi, LY::KL);
      for (int ins = wu; ins < 8; ins += G) {
        const int row = ins * 8 + (l >> 3);
        const int c = (l & 7) ^ ((row >> 1) & 7);
        const int rr = row < left ? row : left - 1;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(kl8 + (key0 + (int64_t)rr * dm.Hkv) * HD + c * 16),
            (__attribute__((address_space(3))) void*)(lo + ins * 1024), 16, 0, 0);
      }
      if (wu == G - 1) {
        const int rr = l < left ? l : left - 1;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(ksc + (key0 + (int64_t)rr * dm.Hkv) * 4),
            (__attribute__((address_space(3))) void*)lds_at(bufi, LY::KS), 4, 0, 0);
      }
    }
  };
  auto stage_v = [&](int tile, int bufi) {
    stage64(vhs_of(bufi), vh + base, tile);
    if constexpr (VLO) stage64(vls_of(bufi), vl + base, tile);
  };
  // S^T blocks 0 and 1 (32 keys each) of the staged tile; the two accumulation chains alternate
  auto scores2 = [&](int bufi, f32x16& s0, f32x16& s1, auto lo_c) {
    s0 = f32x16{};
    s1 = f32x16{};
    const bf16* khs = khs_of(bufi);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int off0 = swz128(n, 2 * ks + hl), off1 = swz128(32 + n, 2 * ks + hl);
      s0 = mfma32(lds_read8(khs + off0), qf[ks], s0);
      s1 = mfma32(lds_read8(khs + off1), qf[ks], s1);
    }
    if constexpr (decltype(lo_c)::value) {
      const unsigned char* lo = lds_at(bufi, LY::KL);
      const int* sc = (const int*)lds_at(bufi, LY::KS);
      // scale bytes 2c + hl of the lane's key row (channels [64 c + 32 hl, +32), the scale of K block
      // hl of MFMA c), moved so byte 2c belongs to this lane half
      const int sa0 = sc[n] >> (8 * hl), sa1 = sc[32 + n] >> (8 * hl);
      // A operand of MFMA c, lane half hl: the 16-byte chunks 4 c + hl and 4 c + 2 + hl of the key's
      // remainder row (channels [64 c + 16 hl, +16) and [64 c + 32 + 16 hl, +16))
      i32x8 a[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int row = kb * 32 + n;
          const i32x4 x0 = *(const i32x4*)(lo + swz8(row, 4 * c + hl));
          const i32x4 x1 = *(const i32x4*)(lo + swz8(row, 4 * c + 2 + hl));
          a[kb][c] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0][0], q8[0], s0, 0, 0, 0, sa0, 0, q8s);
      s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1][0], q8[0], s1, 0, 0, 0, sa1, 0, q8s);
      s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0][1], q8[1], s0, 0, 0, 2, sa0, 0, q8s);
      s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1][1], q8[1], s1, 0, 0, 2, sa1, 0, q8s);
    }
  };
  // Score register j of block kb in tile `tile` holds key tile CK + kb 32 + 4 hl + koff(j); it is
  // visible when koff(j) < lim(tile, kb)
  auto koff = [](int j) { return 8 * (j >> 2) + (j & 3); };
  auto lim = [&](int tile, int kb) { return nv - (tile * CK + kb * 32 + 4 * hl); };
  // tiles whose keys every row of the workgroup sees need no mask
  auto full = [&](int tile) { return (tile + 1) * CK <= nvmin; };

  // keys' low parts (split keys) in both sweeps
  constexpr std::integral_constant<bool, SPLIT> lo1{};
  constexpr std::integral_constant<bool, SPLIT> lo2{};
  // ---- sweep 1: log-sum-exp per (row, head) column.  mr: running maximum of the raw scores,
  // lsum: sum of 2^((s - mr) c2).  The scores of tile i are formed (MFMA) while the exponentials
  // of tile i - 1 run (VALU).
  float mr = -INFINITY, lsum = 0.f;
  auto lse_block = [&](f32x16 s, int tile, int kb, bool mask) {
    if (mask) {  // uniform
      const int lm = lim(tile, kb);
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (koff(j) >= lm) s[j] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[j]);
    const float mnew = fmaxf(mr, mx);
    const float mu = mnew > -INFINITY ? mnew : 0.f;  // nothing visible yet: every term is 0
    const float off = -mu * c2;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc += fexp2(fmaf(s[j], c2, off));
    lsum = lsum * fexp2((mr - mu) * c2) + acc;
    mr = mnew;
  };
  const int nt1 = (nvmax + CK - 1) / CK;
  if (nt1 > 0) {
    stage_k(0, 0, lo1);
    wait_loads();
  }
  __syncthreads();
  {
    // Tiles [0, nfull) are seen whole by every row of the workgroup.  Their loop forms the scores
    // of tile i (MFMA) while the exponentials of tile i - 1 run (VALU), interleaved by the
    // scheduling groups; the remaining tiles go one by one with masks.
    const int nfull = nvmin / CK;
    f32x16 p0, p1;  // formed scores not yet summed: those of tile t - 1
    int t = 0;
    if (nt1 > 0) {
      if (nt1 > 1) stage_k(1, 1, lo1);
      scores2(0, p0, p1, lo1);
      wait_loads();
      __syncthreads();
      t = 1;
      for (; t < nt1 && t <= nfull; ++t) {
        if (t + 1 < nt1) stage_k(t + 1, (t + 1) & 1, lo1);
        f32x16 s0, s1;
        scores2(t & 1, s0, s1, lo1);
        lse_block(p0, t - 1, 0, false);
        lse_block(p1, t - 1, 1, false);
        SG(SG_DSR, 8);
#pragma unroll
        for (int i = 0; i < 24; ++i) {
          SG(SG_MFMA, 1);
          SG(SG_DSR, 1);
          SG(SG_VALU, 4);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          SG(SG_MFMA, 1);
          SG(SG_VALU, 5);
        }
        p0 = s0;
        p1 = s1;
        wait_loads();
        __syncthreads();
      }
      lse_block(p0, t - 1, 0, !full(t - 1));
      lse_block(p1, t - 1, 1, !full(t - 1));
      for (; t < nt1; ++t) {
        if (t + 1 < nt1) stage_k(t + 1, (t + 1) & 1, lo1);
        scores2(t & 1, p0, p1, lo1);
        lse_block(p0, t, 0, !full(t));
        lse_block(p1, t, 1, !full(t));
        wait_loads();
        __syncthreads();
      }
    }
  }
  float L2;  // log2-domain normaliser: p = 2^(s c2 - L2)
  {
    const float mo = xchg32(mr, hl), lo = xchg32(lsum, hl);
    const float M = fmaxf(mr, mo);
    if (M > -INFINITY) {
      const float tot = (mr > -INFINITY ? lsum * fexp2((mr - M) * c2) : 0.f) +
                        (mo > -INFINITY ? lo * fexp2((mo - M) * c2) : 0.f);
      L2 = M * c2 + flog2(tot);
    } else {
      L2 = INFINITY;  // no visible block: every probability is zero
    }
  }

  // ---- sweep 2: probabilities, value sum, importance
  // Head-sum items of this thread: (row, block within the tile) = (i >> 4, i & 15) for
  // i = tid, tid + nthr; jmax = the row's last block (-1: text row or past the end).
  int64_t jmax[2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const int i = tid + k2 * nthr;
    const int64_t rr = rt0 + (i >> 4);
    jmax[k2] = -1;
    if (i < CQ * 16 && rr < dm.Tq && (!vid || vid[b * dm.Tq + rr])) {
      const int64_t jt = (dm.q0 + rr) / dm.ls;
      jmax[k2] = jt < dm.Ns ? jt : dm.Ns - 1;
    }
  }
  f32x16 oacc[4] = {};
  float carry = 0.f;  // half share of the previous run's last compressed block (hl == 0 lanes)
  const int g16 = l >> 4, i16 = l & 15;
  auto pv_block = [&](const f32x16& s, int bufi, int tile, int kb, float* ipb, bool mask) {
    float p[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) p[j] = fexp2(fmaf(s[j], c2, -L2));
    if (mask) {  // uniform: only tiles with keys past some row's last visible one
      const int lm = lim(tile, kb);
#pragma unroll
      for (int j = 0; j < 16; ++j) p[j] = koff(j) < lm ? p[j] : 0.f;
    }
    // importance of the four selection blocks this lane covers in this 32-key run
    float a[4], oth[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const float half = 0.5f * p[4 * qq + 3];
      a[qq] = p[4 * qq] + p[4 * qq + 1] + p[4 * qq + 2] + half;
      oth[qq] = xchg32(half, hl);
    }
    if (hl == 0) {
      a[0] += carry;
      a[1] += oth[0];
      a[2] += oth[1];
      a[3] += oth[2];
      carry = oth[3];
    } else {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) a[qq] += oth[qq];
    }
    float* ip = ipb + (w * CQ + n) * IPS + kb * 8 + hl;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) ip[2 * qq] = a[qq];
    // O^T += Vc^T P^T in two 16-key steps
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (bf16)p[8 * st + e];
      const int vr = kb * 32 + 16 * st + 4 * (g16 >> 1) + (i16 >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int col = 32 * db + (g16 & 1) * 16 + 4 * (i16 & 3);
        const int o0 = swz128(vr, col >> 3) + (col & 7);
        const int o1 = swz128(vr + 8, col >> 3) + (col & 7);
        const bf16* vhs = vhs_of(bufi);
        oacc[db] = mfma32(cat(lds_read_tr(vhs + o0), lds_read_tr(vhs + o1)), pb, oacc[db]);
        if constexpr (VLO) {
          const bf16* vls = vls_of(bufi);
          oacc[db] = mfma32(cat(lds_read_tr(vls + o0), lds_read_tr(vls + o1)), pb, oacc[db]);
        }
      }
    }
  };
  // Each iteration: probabilities and value sums of tile i (its scores formed before), barrier,
  // the scores of tile i + 1 (MFMA) while the group's heads are summed for tile i.
  const int nt2 = nvmax > 0 ? nvmax / CK + 1 : 0;
  f32x16 s0, s1;
  if (nt2 > 0) {
    stage_k(0, 0, lo2);
    stage_v(0, 0);
    wait_loads();
  }
  __syncthreads();
  if (nt2 > 0) scores2(0, s0, s1, lo2);
  for (int tile = 0; tile < nt2; ++tile) {
    const int bufi = tile & 1;
    if (tile + 1 < nt2) {
      stage_k(tile + 1, bufi ^ 1, lo2);
      stage_v(tile + 1, bufi ^ 1);
    }
    float* ipb = ipart0 + (ipart_bufs == 2 ? bufi : 0) * G * CQ * IPS;
    const bool m = !full(tile);
    pv_block(s0, bufi, tile, 0, ipb, m);
    pv_block(s1, bufi, tile, 1, ipb, m);
    wait_loads();
    __syncthreads();
    if (tile + 1 < nt2) scores2(bufi ^ 1, s0, s1, lo2);
    // sum the group's heads in a fixed order; write the tile's 16 selection blocks
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int i = tid + k2 * nthr;
      const int64_t J = (int64_t)tile * 16 + (i & 15);
      if (J > jmax[k2]) continue;
      const int nn = i >> 4;
      float sum = 0.f;
      for (int ww = 0; ww < G; ++ww) sum += ipb[(ww * CQ + nn) * IPS + (i & 15)];
      if (imp) imp[((b * dm.Tq + rt0 + nn) * dm.Hkv + g) * dm.Ns + J] = sum;
    }
    if (ipart_bufs == 1) __syncthreads();  // the partials are rewritten by the next tile
  }
  // blocks up to the row's own block that no compressed block reaches
  for (int idx = tid; idx < CQ * 16; idx += nthr) {
    const int nn = idx >> 4, jj = idx & 15;
    const int64_t rr = rt0 + nn;
    if (rr >= dm.Tq || (vid && !vid[b * dm.Tq + rr])) continue;
    const int64_t J = (int64_t)nt2 * 16 + jj;
    if (imp && J <= (dm.q0 + rr) / dm.ls && J < dm.Ns) imp[((b * dm.Tq + rr) * dm.Hkv + g) * dm.Ns + J] = 0.f;
  }

  if (!isv) return;
  const int64_t orow = ((b * dm.Tq + r) * dm.Hq + h) * (int64_t)HD;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = 32 * db + 8 * j4 + 4 * hl;
      if (o_f32)
        *(float4*)(o_f32 + orow + d0) =
            make_float4(oacc[db][4 * j4], oacc[db][4 * j4 + 1], oacc[db][4 * j4 + 2], oacc[db][4 * j4 + 3]);
      if (o_bf) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)oacc[db][4 * j4 + e];
        *(bf16x4*)(o_bf + orow + d0) = v4;
      }
    }
  }
  if (lse && hl == 0) lse[(b * dm.Tq + r) * dm.Hq + h] = nv > 0 ? L2 * LN2_F : -INFINITY;
  };
  if constexpr (SPLIT) {
    if (cmp_visible(dm.q0 + rt0, dm.l, dm.d, dm.Nc) < kVloBelow)
      body(std::true_type{});
    else
      body(std::false_type{});
  } else {
    body(std::false_type{});
  }
}

// Dynamic LDS: the staged K / V buffers, then 1 or 2 buffers of importance partials (2 when
// they fit next to the static LDS of the kernel).
static int cmp_ipart_bufs(const Dims& dm, bool split, size_t* bytes) {
  const size_t stage = (size_t)2 * (split ? CmpLds<true>::BUF : CmpLds<false>::BUF);
  const size_t ip = (size_t)dm.G * CQ * IPS * 4;
  const int bufs = stage + 2 * ip + 64 <= (size_t)160 * 1024 ? 2 : 1;
  *bytes = stage + bufs * ip;
  return bufs;
}

hipError_t launch_cmp_fast(const Dims& dm, const void* q, const void* kh, const void* kl8, const void* ksc,
                           const void* vh, const void* vl, const uint8_t* vid, void* o, float* o32, float* lse,
                           float* imp, hipStream_t s) {
  if (dm.Tq <= 0 || dm.B <= 0) return hipSuccess;
  const int ntq = (int)((dm.Tq + CQ - 1) / CQ);
  const int units = (int)(dm.B * dm.Hkv);
  const bool split = kl8 != nullptr;
  if (split && (!ksc || !vl)) return hipErrorInvalidValue;
  auto launch = [&](bool sp, auto kernel) -> hipError_t {
    size_t shm;
    const int bufs = cmp_ipart_bufs(dm, sp, &shm);
    hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    kernel<<<dim3(xcd_grid(units, ntq)), dim3(dm.G * 64), shm, s>>>(
        (const bf16*)q, (const bf16*)kh, (const uint8_t*)kl8, (const uint8_t*)ksc, (const bf16*)vh,
        (const bf16*)vl, vid, (bf16*)o, o32, lse, imp, dm, 0, ntq, bufs);
    return hipGetLastError();
  };
  return split ? launch(true, cmp_fast_kernel<true>) : launch(false, cmp_fast_kernel<false>);
}

// Split keys for the compression branch: the fp32 sum x of each compressed key is stored as
// its bf16 high part hi (row-major [B, Nc, Hkv, 128]) and the remainder x - hi in fp8 e4m3 in
// channel order, with one scale per group of 32 consecutive channels.  Every |x| of a group lies
// below 2^E, so |x - hi| <= 2^(E - 9); the remainder is stored times 2^(17 - E) (at most 256,
// inside e4m3's range) and scale byte 110 + E (E8M0) undoes it.  Groups whose magnitudes are all
// below 2^-100 store zeros.  One thread per 8 channels of a compressed key; the 16 threads of a
// key row are 16 consecutive lanes, and the four of one group reduce their maximum with two lane
// exchanges.
__global__ void __launch_bounds__(256) compress_k8_kernel(const bf16* __restrict__ x, const float* __restrict__ w,
                                                          bf16* __restrict__ hi, uint8_t* __restrict__ lo8,
                                                          uint8_t* __restrict__ sc, int64_t T_len, int H, int l,
                                                          int d, int64_t Nc, int64_t total) {
  __shared__ float ws[64];
  for (int m = threadIdx.x; m < l; m += blockDim.x) ws[m] = w[m];
  __syncthreads();
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool valid = gid < total;  // total is a multiple of 16: whole key rows
  const int c8 = (int)(gid & 15);
  const int64_t row = valid ? gid >> 4 : 0;  // (b, i, h)
  const int h = (int)(row % H);
  const int64_t i = (row / H) % Nc;
  const int64_t b = row / H / Nc;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const bf16* src = x + ((b * T_len + i * d) * H + h) * (int64_t)HD + c8 * 8;
  for (int m = 0; m < l; ++m) {
    const bf16x8 u = *(const bf16x8*)(src + (int64_t)m * H * HD);
    const float wm = ws[m];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(wm, (float)u[e], acc[e]);
  }
  float mx = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(acc[e]));
  mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
  int E = 0;
  (void)frexpf(mx, &E);
  const bool keep = mx > 0.f && E >= -100;
  bf16x8 vh;
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    vh[e] = (bf16)acc[e];
    r[e] = keep ? ldexpf(acc[e] - (float)vh[e], 17 - E) : 0.f;
  }
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(r[4], r[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(r[6], r[7], w1, true);
  if (!valid) return;
  *(bf16x8*)(hi + row * HD + c8 * 8) = vh;
  *(int2*)(lo8 + row * HD + c8 * 8) = make_int2(w0, w1);
  // the first thread of each group of 32 channels writes its scale byte
  if ((c8 & 3) == 0) sc[row * 4 + (c8 >> 2)] = (uint8_t)(keep ? 110 + E : 127);
}

size_t k8_lo_bytes(const Dims& dm) { return (size_t)dm.B * dm.Nc * dm.Hkv * HD; }
size_t k8_sc_bytes(const Dims& dm) { return (size_t)dm.B * dm.Nc * dm.Hkv * 4; }

hipError_t launch_compress_k8(const Dims& dm, const void* k, const float* w_k, void* hi, void* lo8, void* sc,
                              hipStream_t s) {
  if (dm.Nc <= 0 || dm.B <= 0) return hipSuccess;
  if (dm.D != HD || dm.l > 64) return hipErrorInvalidValue;
  const int64_t total = dm.B * dm.Nc * dm.Hkv * 16;
  compress_k8_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>((const bf16*)k, w_k, (bf16*)hi, (uint8_t*)lo8,
                                                                     (uint8_t*)sc, dm.T, dm.Hkv, dm.l, dm.d, dm.Nc,
                                                                     total);
  return hipGetLastError();
}
