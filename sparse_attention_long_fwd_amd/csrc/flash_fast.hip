// Sliding-window rows and dense causal text rows, bf16 MFMA flash tiles on gfx950.
//
// Sliding window (top168.com digest of VideoNSA, section 一): a video row t
// attends to keys [max(0, t - w + 1), t].  Text rows keep dense causal
// attention over every key u <= t (shd-paper.top page, English abstract).
//
// One workgroup = 32 consecutive query rows x up to four heads of one KV group
// (one wave per head; a group of G heads takes ceil(G / 4) workgroups, which
// stage the same K/V tiles: two four-wave workgroups fit a compute unit at
// this register count, so one's loads and barriers overlap the other's
// products), the same tile as the compression branch: S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16, one (row, head) column per lane, online softmax in
// the log2 domain with the running maximum shared by the two lane halves of a
// column (one xor-32 exchange per 64-key tile), O^T += V^T P^T with V^T read
// through ds_read_b64_tr_b16.  K/V tiles of 64 tokens stream global -> LDS
// (double-buffered, XOR-swizzled rows), shared by the G waves.  The running
// maximum is moved only when a tile's maximum exceeds it by more than 8 (log2
// units), so the accumulator is rescaled rarely; values stay below 2^8.
//
// A tile holding both video and text rows runs the window pass for its video
// rows and the dense pass for its text rows.  The grid is ordered last tile
// first, so the long dense rows at the end of a sequence start first.
// Text rows of the first `max_split` tiles may be split over key chunks; the
// chunks' partial (max, sum, output) go to a workspace and a merge kernel
// combines them.
#include "fast_common.hpp"

namespace {
constexpr int FQ = 32;
constexpr int FK = 64;
constexpr int FW = 4;  // waves (heads) per workgroup
constexpr int HD = 128;
constexpr int TILE = FK * HD;
constexpr float RESCALE_SLACK = 8.f;
}  // namespace

__device__ __forceinline__ void fwait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

struct FlashOut {
  float2* lml;    // selection partials (max, sum) per (row, group, slot, head), or NULL (no local pass)
  unsigned char* lo;  // their value records (12-bit, SLC_REC_BYTES each)
  bf16* swa_bf;   // bf16 window output (may be NULL)
  bf16* text;     // dense output of text rows (the layer's out)
  float* part;    // split partials: [slot][chunk][G*32 columns][D + 2] (may be NULL)
  int nsplit;     // key chunks of a split tile (1 = no split)
  int max_split;  // tiles with rank < max_split are split
};

// One pass of online-softmax attention over key tiles [a0, a1) and then [b0, b1)
// (one double-buffered stream: the first tile of the second range is staged
// during the last of the first) for the lanes whose column is active; the key
// of each column is limited to [klo, khi] (inclusive).  Returns (in the
// references) the running maximum, the lane's partial sum and the accumulator
// (unnormalised).  on_split() runs in every wave right after the last tile of
// the first range, with the state over that range in the references.
// compute = false: a wave without a head, which only stages tiles and keeps
// the barriers.
template <typename OnSplit>
__device__ __forceinline__ void flash_pass2(const bf16* __restrict__ kbase, const bf16* __restrict__ vbase,
                                            int64_t stride, int64_t T, int a0, int a1, int b0, int b1,
                                            const bf16x8 (&qf)[8], int64_t klo, int64_t khi, bool active, float c2,
                                            bf16* buf0, int w, int nw, int l, bool compute, float& m_run,
                                            float& l_run, f32x16 (&oacc)[4], OnSplit on_split) {
  const int hl = l >> 5, n = l & 31, g16 = l >> 4, i16 = l & 15;
  m_run = -INFINITY;
  l_run = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  const int na = a1 > a0 ? a1 - a0 : 0, nt = na + (b1 > b0 ? b1 - b0 : 0);
  if (na == 0) on_split();
  if (nt == 0) return;
  auto tile_of = [&](int i) { return i < na ? a0 + i : b0 + (i - na); };
  // keys every active column admits: [lo_all, hi_all] (the largest klo, the smallest khi); tiles
  // inside it need no key mask (inactive columns then take unmasked scores, which only their own
  // output columns see)
  int64_t lo_all = active ? klo : INT64_MIN, hi_all = active ? khi : INT64_MAX;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const int64_t a = __shfl_xor(lo_all, o, 64), b = __shfl_xor(hi_all, o, 64);
    lo_all = a > lo_all ? a : lo_all;
    hi_all = b < hi_all ? b : hi_all;
  }
  auto uniform64 = [](int64_t x) {  // the same in every lane: keep it in scalar registers
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };
  lo_all = uniform64(lo_all);
  hi_all = uniform64(hi_all);
  auto arr = [&](int bufi, int a) { return buf0 + (bufi * 2 + a) * TILE; };
  auto stage = [&](int kt, int bufi) {
    stage_tile64(arr(bufi, 0), kbase, stride, (int64_t)kt * FK, T, w, nw, l);
    stage_tile64(arr(bufi, 1), vbase, stride, (int64_t)kt * FK, T, w, nw, l);
  };
  __syncthreads();  // previous users of the buffers are done
  stage(tile_of(0), 0);
  fwait_loads();
  __syncthreads();
  for (int i = 0; i < nt; ++i) {
    const int kt = tile_of(i);
    const int bufi = i & 1;
    if (i + 1 < nt) stage(tile_of(i + 1), bufi ^ 1);
    if (compute) {
      const bf16* ks_ = arr(bufi, 0);
      const bool full = (int64_t)kt * FK >= lo_all && (int64_t)kt * FK + FK - 1 <= hi_all;  // uniform
      float x[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 s = {};
        const int row = kb * 32 + n;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) s = mfma32(lds_read8(ks_ + swz128(row, 2 * ks + hl)), qf[ks], s);
        if (full) {
#pragma unroll
          for (int j = 0; j < 16; ++j) x[kb * 16 + j] = s[j] * c2;
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int64_t key = (int64_t)kt * FK + kb * 32 + 8 * (j >> 2) + 4 * hl + (j & 3);
            x[kb * 16 + j] = (active && key >= klo && key <= khi) ? s[j] * c2 : -INFINITY;
          }
        }
      }
      float mx = x[0];
#pragma unroll
      for (int j = 1; j < 32; ++j) mx = fmaxf(mx, x[j]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (mx > m_run + RESCALE_SLACK) {
        const float corr = fexp2(m_run - mx);  // 0 on the first raise from -inf
        l_run *= corr;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) oacc[db][j] *= corr;
        m_run = mx;
      }
      float p[32];
      if (m_run > -INFINITY) {
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          p[j] = fexp2(x[j] - m_run);
          l_run += p[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) p[j] = 0.f;
      }
      const bf16* vs_ = arr(bufi, 1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[e] = (bf16)p[kb * 16 + 8 * st + e];
          const int vr = kb * 32 + 16 * st + 4 * (g16 >> 1) + (i16 >> 2);
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const int col = 32 * db + (g16 & 1) * 16 + 4 * (i16 & 3);
            const int o0 = swz128(vr, col >> 3) + (col & 7);
            const int o1 = swz128(vr + 8, col >> 3) + (col & 7);
            oacc[db] = mfma32(cat(lds_read_tr(vs_ + o0), lds_read_tr(vs_ + o1)), pb, oacc[db]);
          }
        }
      }
    }
    if (i + 1 == na) on_split();
    fwait_loads();
    __syncthreads();
  }
}

// The same over one range [kt0, kt1).
__device__ __forceinline__ void flash_pass(const bf16* __restrict__ kbase, const bf16* __restrict__ vbase,
                                           int64_t stride, int64_t T, int kt0, int kt1, const bf16x8 (&qf)[8],
                                           int64_t klo, int64_t khi, bool active, float c2, bf16* buf0, int w,
                                           int nw, int l, bool compute, float& m_run, float& l_run,
                                           f32x16 (&oacc)[4]) {
  flash_pass2(kbase, vbase, stride, T, kt0, kt1, 0, 0, qf, klo, khi, active, c2, buf0, w, nw, l, compute, m_run,
              l_run, oacc, [] {});
}

__global__ void __launch_bounds__(FW * 64) __attribute__((amdgpu_waves_per_eu(2)))
flash_fast_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                         const bf16* __restrict__ v, const uint8_t* __restrict__ vid,
                                                         FlashOut fo, Dims dm, int ntq, int do_swa, int do_text) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* buf0 = (bf16*)smem;
  __shared__ int s_kind;  // bit 0: some video row, bit 1: some text row

  const int G = dm.G;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, hl = l >> 5, n = l & 31;
  const int nsplit = fo.nsplit;
  // ranks [0, max_split * nsplit): (tile, chunk) of the split tiles; then one rank per remaining tile;
  // each rank in nhs workgroups of up to FW heads (adjacent workgroup ranks)
  const int nsr = fo.max_split * nsplit;
  const int nhs = (G + FW - 1) / FW;
  int unit, wrank;
  if (!xcd_remap(blockIdx.x, (int)(dm.B * dm.Hkv), (nsr + ntq - fo.max_split) * nhs, &unit, &wrank)) return;
  const int rank = wrank / nhs;
  const int hw = (wrank % nhs) * FW + w;  // this wave's head within the group
  const bool hact = hw < G;               // a wave without a head stages tiles and keeps the barriers
  const bool split = rank < nsr;
  const int chunk = split ? rank % nsplit : 0;
  const int trank = split ? rank / nsplit : fo.max_split + (rank - nsr);  // tile rank, last tile first
  const int64_t b = unit / dm.Hkv;
  const int g = unit % dm.Hkv;
  const int64_t rt0 = (int64_t)(ntq - 1 - trank) * FQ;

  if (tid == 0) s_kind = 0;
  __syncthreads();
  if (tid < FQ) {
    const int64_t r = rt0 + tid;
    if (r < dm.Tq) {
      const bool v_ = !vid || vid[b * dm.Tq + r];
      atomicOr(&s_kind, v_ ? 1 : 2);
    }
  }
  __syncthreads();
  const int kind = s_kind;

  const int64_t r = rt0 + n;
  const bool rvalid = r < dm.Tq;
  const bool isv = rvalid && (!vid || vid[b * dm.Tq + r]);
  const int64_t t = dm.q0 + r;
  const int h = g * G + (hact ? hw : 0);
  const float c2 = dm.scale * LOG2E_F;
  const int64_t rlast = (rt0 + FQ < dm.Tq ? rt0 + FQ : dm.Tq) - 1;
  const int64_t tfirst = dm.q0 + rt0, tlast = dm.q0 + rlast;

  bf16x8 qf[8];
  {
    const bf16* qrow = q + ((b * dm.Tq + (rvalid ? r : 0)) * dm.Hq + h) * (int64_t)HD + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = (rvalid && hact) ? *(const bf16x8*)(qrow + 16 * ks) : zero8();
  }
  const int64_t stride = (int64_t)dm.Hkv * HD;
  const bf16* kbase = k + (b * dm.T * dm.Hkv + g) * (int64_t)HD;
  const bf16* vbase = v + (b * dm.T * dm.Hkv + g) * (int64_t)HD;
  const int64_t orow = ((b * dm.Tq + r) * dm.Hq + h) * (int64_t)HD;
  float m_run, l_run;
  f32x16 oacc[4];

  // ---- window pass (video rows), only by chunk 0
  if (do_swa && (kind & 1) && chunk == 0) {
    int64_t lo0 = tfirst - dm.w + 1;
    if (lo0 < 0) lo0 = 0;
    const int kt0 = (int)(lo0 / FK), kt1 = (int)(tlast / FK) + 1;
    int64_t klo = t - dm.w + 1;
    if (klo < 0) klo = 0;
    if (fo.lml) {
      // The row tile's forced local selection blocks (jt - n_local + 1 .. jt, inside every row's
      // window) go first; the state after them is the selection partial of those blocks (the
      // window and selection masks agree there), stored in the row's first local slot.
      const int jt = kt1 - 1;
      const int nle = dm.n_local < jt + 1 ? dm.n_local : jt + 1;
      const int ktl = jt - nle + 1 > kt0 ? jt - nle + 1 : kt0;
      flash_pass2(kbase, vbase, stride, dm.T, ktl, kt1, kt0, ktl, qf, klo, t, isv, c2, buf0, w, FW, l, hact, m_run,
                  l_run, oacc, [&] {
        const float lt = l_run + __shfl_xor(l_run, 32, 64);
        // normalised to sum 1 (the maximum is kept lazily), as a 12-bit record whose exponent comes
        // from both lane halves' largest value
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        float amax = 0.f;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) amax = fmaxf(amax, fabsf(oacc[db][jj]));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64)) * inv;
        const int ex = rec12_exp(amax);
        if (isv && hact) {
          const int nvalid = dm.n < jt + 1 ? dm.n : jt + 1;
          const int64_t rec0 = (((b * dm.Tq + r) * dm.Hkv + g) * dm.n + (nvalid - nle)) * G + hw;
          rec12_store_half(fo.lo + rec0 * SLC_REC_BYTES, hl, oacc, inv, ex);
          if (hl == 0) {
            fo.lml[rec0] = lt > 0.f ? rec12_ml(m_run + flog2(lt), 1.f, ex) : make_float2(-INFINITY, 0.f);
            for (int e = 1; e < nle; ++e) fo.lml[rec0 + (int64_t)e * G] = make_float2(-INFINITY, 0.f);
          }
        }
      });
    } else {
      flash_pass(kbase, vbase, stride, dm.T, kt0, kt1, qf, klo, t, isv, c2, buf0, w, FW, l, hact, m_run, l_run,
                 oacc);
    }
    const float lt = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (isv && hact) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int d0 = 32 * db + 8 * j4 + 4 * hl;
          if (fo.swa_bf) {
            bf16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = (bf16)(oacc[db][4 * j4 + e] * inv);
            *(bf16x4*)(fo.swa_bf + orow + d0) = v4;
          }
        }
    }
  }

  // ---- dense pass (text rows), whole range or one key chunk
  if (do_text && (kind & 2)) {
    const bool ist = rvalid && !isv;
    const int ktall = (int)(tlast / FK) + 1;
    int kt0 = 0, kt1 = ktall;
    if (split) {
      const int per = (ktall + nsplit - 1) / nsplit;
      kt0 = chunk * per;
      kt1 = kt0 + per < ktall ? kt0 + per : ktall;
    }
    flash_pass(kbase, vbase, stride, dm.T, kt0, kt1, qf, 0, t, ist, c2, buf0, w, FW, l, hact, m_run, l_run, oacc);
    const float lt = l_run + __shfl_xor(l_run, 32, 64);
    if (!hact) {
      // no head: nothing to store
    } else if (split) {
      // partial for (tile slot, chunk, column hw*32+n): [D] normalised output, then max and sum
      float* pp = fo.part + (((int64_t)(unit * fo.max_split + trank) * nsplit + chunk) * (G * FQ) + hw * FQ + n) *
                                (HD + 2);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int d0 = 32 * db + 8 * j4 + 4 * hl;
          *(float4*)(pp + d0) = make_float4(oacc[db][4 * j4] * inv, oacc[db][4 * j4 + 1] * inv,
                                            oacc[db][4 * j4 + 2] * inv, oacc[db][4 * j4 + 3] * inv);
        }
      if (hl == 0) {
        pp[HD] = m_run;
        pp[HD + 1] = lt;
      }
    } else if (ist) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int d0 = 32 * db + 8 * j4 + 4 * hl;
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (bf16)(oacc[db][4 * j4 + e] * inv);
          *(bf16x4*)(fo.text + orow + d0) = v4;
        }
    }
  }
}

// Combines the key chunks of split text tiles: one thread per (row, head, 4 channels).
__global__ void __launch_bounds__(256) flash_merge_kernel(const uint8_t* __restrict__ vid, FlashOut fo, Dims dm,
                                                          int ntq) {
  const int G = dm.G;
  const int64_t per_unit = (int64_t)fo.max_split * G * FQ * (HD / 4);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= per_unit * dm.B * dm.Hkv) return;
  const int unit = (int)(gid / per_unit);
  int64_t rem = gid % per_unit;
  const int c4 = (int)(rem % (HD / 4));
  rem /= (HD / 4);
  const int col = (int)(rem % (G * FQ));
  const int trank = (int)(rem / (G * FQ));
  if (trank >= ntq) return;
  const int64_t b = unit / dm.Hkv;
  const int g = unit % dm.Hkv;
  const int w = col / FQ, n = col % FQ;
  const int64_t r = (int64_t)(ntq - 1 - trank) * FQ + n;
  if (r >= dm.Tq || !vid || vid[b * dm.Tq + r]) return;  // text rows only
  const int nsplit = fo.nsplit;
  const float* base = fo.part + (((int64_t)(unit * fo.max_split + trank) * nsplit) * (G * FQ) + col) * (HD + 2);
  const int64_t cstride = (int64_t)(G * FQ) * (HD + 2);
  float M = -INFINITY;
  for (int c = 0; c < nsplit; ++c) {
    const float* pc = base + c * cstride;
    if (pc[HD + 1] > 0.f) M = fmaxf(M, pc[HD]);
  }
  float4 acc = make_float4(0, 0, 0, 0);
  float wsum = 0.f;
  for (int c = 0; c < nsplit; ++c) {
    const float* pc = base + c * cstride;
    const float lc = pc[HD + 1];
    if (!(lc > 0.f)) continue;
    const float wc = lc * fexp2(pc[HD] - M);
    const float4 o = *(const float4*)(pc + 4 * c4);
    acc.x += wc * o.x;
    acc.y += wc * o.y;
    acc.z += wc * o.z;
    acc.w += wc * o.w;
    wsum += wc;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int h = g * G + w;
  bf16x4 v4;
  v4[0] = (bf16)(acc.x * inv);
  v4[1] = (bf16)(acc.y * inv);
  v4[2] = (bf16)(acc.z * inv);
  v4[3] = (bf16)(acc.w * inv);
  *(bf16x4*)(fo.text + ((b * dm.Tq + r) * dm.Hq + h) * (int64_t)HD + 4 * c4) = v4;
}

namespace {
constexpr int MAX_SPLIT_TILES = 64;  // text tiles (last first) that may be split over key chunks
constexpr int TEXT_CHUNK_TILES = 128;  // 64-token key tiles per chunk of a split text tile
}  // namespace

int flash_nsplit(const Dims& dm) {
  const int64_t ktiles = (dm.q0 + dm.Tq + FK - 1) / FK;
  int ns = (int)((ktiles + TEXT_CHUNK_TILES - 1) / TEXT_CHUNK_TILES);
  return ns < 1 ? 1 : (ns > 16 ? 16 : ns);
}

size_t flash_workspace(const Dims& dm) {
  const int ns = flash_nsplit(dm);
  if (ns <= 1) return 0;
  return (size_t)dm.B * dm.Hkv * MAX_SPLIT_TILES * ns * dm.G * FQ * (HD + 2) * sizeof(float);
}

// swa_bf: window output (may be NULL); text: output of text rows (NULL: skip them).
bool local_fusable(const Dims& dm) {
  return dm.ls == FK && dm.n_local >= 1 && dm.w >= FK * dm.n_local && dm.q0 % FQ == 0;
}

hipError_t launch_flash_fast(const Dims& dm, const void* q, const void* k, const void* v, const uint8_t* vid,
                             void* swa_bf, void* text, void* ws, hipStream_t s, void* local_ml,
                             void* local_o) {
  if (dm.Tq <= 0 || dm.B <= 0) return hipSuccess;
  const int ntq = (int)((dm.Tq + FQ - 1) / FQ);
  const int units = (int)(dm.B * dm.Hkv);
  FlashOut fo;
  if ((local_ml != nullptr) != (local_o != nullptr) || (local_ml && !local_fusable(dm))) return hipErrorInvalidValue;
  fo.lml = (float2*)local_ml;
  fo.lo = (unsigned char*)local_o;
  fo.swa_bf = (bf16*)swa_bf;
  fo.text = (bf16*)text;
  fo.nsplit = (text && vid) ? flash_nsplit(dm) : 1;
  fo.max_split = fo.nsplit > 1 ? (ntq < MAX_SPLIT_TILES ? ntq : MAX_SPLIT_TILES) : 0;
  fo.part = (float*)ws;
  if (fo.nsplit > 1 && !ws) fo.nsplit = 1, fo.max_split = 0;
  const int do_swa = (swa_bf || local_ml) ? 1 : 0;
  const int do_text = text ? 1 : 0;
  if (!do_swa && !do_text) return hipSuccess;
  const int nhs = (dm.G + FW - 1) / FW;
  dim3 grid(xcd_grid(units, (fo.max_split * fo.nsplit + ntq - fo.max_split) * nhs)), block(FW * 64);
  const size_t shm = (size_t)2 * 2 * TILE * 2;
  hipError_t e = hipFuncSetAttribute((const void*)flash_fast_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)shm);
  if (e != hipSuccess) return e;
  flash_fast_kernel<<<grid, block, shm, s>>>((const bf16*)q, (const bf16*)k, (const bf16*)v, vid, fo, dm, ntq,
                                             do_swa, do_text);
  e = hipGetLastError();
  if (e != hipSuccess || fo.nsplit <= 1) return e;
  const int64_t total = (int64_t)units * fo.max_split * dm.G * FQ * (HD / 4);
  flash_merge_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s>>>(vid, fo, dm, ntq);
  return hipGetLastError();
}
