// One wave selects the blocks of one (row, KV group): the forced blocks and the kk best free
// candidates by (importance descending, block index ascending), written ascending and -1 padded
// (top168.com digest of VideoNSA, section 一: the selection branch keeps the most important
// segments).
//
// Threshold method: each lane takes up to TK candidates (strided by 64; TK = 4, 8, 16 or 32, the
// smallest that holds the row's candidates, so short rows load and scan fewer slots).  The kk-th largest
// of the 64 lane maxima, th, is a lower bound of the kk-th largest candidate (the kk lanes with
// the largest maxima each hold a value >= th), so the candidates >= th contain the answer.  They
// are compacted into LDS, one per lane (a wave prefix sum gives each lane its slots), and the
// exact kk-th largest value among them is found by a bitwise search on order-preserving integer
// keys with wave ballots; ties at that value go to the lower block indices.  Rows with more
// candidates than the registers hold take the same steps over two streamed passes; rows with more
// than 64 values >= th (heavy ties) take kk rounds of a wave-wide arg-max instead, each strictly
// after the previous pick.
#pragma once
#include "common.hpp"

constexpr int TK_REG = 32;  // most candidates a lane holds in registers

// (a, ja) ranks before (b, jb)
__device__ __forceinline__ bool tk_before(float a, int ja, float b, int jb) { return a > b || (a == b && ja < jb); }

// LDS scratch of one wave
struct TopkScratch {
  float v[64];
  int j[64];
  int sel[32];
};

__device__ __forceinline__ void tk_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Integer key with the order of the float (larger float <-> larger unsigned key).
__device__ __forceinline__ uint32_t tk_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Largest key K with #{lanes: key >= K} >= kk (the kk-th largest key); lanes that take no part
// pass key 0 (every real key has its top bit set).  Two bits a step, three independent ballots.
// Uniform result.
__device__ __forceinline__ uint32_t tk_kth_key(uint32_t key, int kk) {
  uint32_t res = 0;
#pragma unroll
  for (int bit = 30; bit >= 0; bit -= 2) {
    const uint32_t c1 = res | (1u << bit), c2 = res | (2u << bit), c3 = res | (3u << bit);
    const int n1 = (int)__popcll(__ballot(key >= c1));
    const int n2 = (int)__popcll(__ballot(key >= c2));
    const int n3 = (int)__popcll(__ballot(key >= c3));
    res = n3 >= kk ? c3 : n2 >= kk ? c2 : n1 >= kk ? c1 : res;
  }
  return res;
}

// x: importance indexed by block (global or LDS).  Free candidates [lo, hi); forced blocks
// [0, lo) and [hi, nj); kk = places for free candidates (n minus the forced count); out: n
// entries.  Whole wave, uniform arguments.  TK: register slots a lane takes (see wave_select);
// 0: the candidates are streamed twice instead of held.
template <int TK>
__device__ inline void wave_select_tk(const float* __restrict__ x, int lo, int hi, int nj, int kk, int n,
                                      TopkScratch* sc, int32_t* __restrict__ out, int lane) {
  uint64_t chosen = 0;  // lanes whose (sc_v, sc_j) entry is chosen (threshold path)
  int cj = 0;           // this lane's entry index (threshold path)
  int nsel = 0;         // chosen free blocks
  bool in_sel = false;  // chosen blocks are in sc->sel (round / all paths) rather than lanes
  const int nc = hi - lo;
  if (kk > 0 && nc > 0) {
    if (nc <= kk) {
      if (lane < nc) sc->sel[lane] = lo + lane;
      nsel = nc;
      in_sel = true;
    } else {
      bool done = false;
      if (TK == 0 || nc <= 64 * TK) {
        // compact the candidates >= th into LDS, one ballot per slot that has any
        int total = 0;
        auto compact = [&](float v, int j, uint32_t thk) {
          const bool take = j < hi && tk_key(v) >= thk;
          const uint64_t bal = __ballot(take);
          if (bal == 0) return;  // uniform
          const int pos = total + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          if (take && pos < 64) {
            sc->v[pos] = v;
            sc->j[pos] = j;
          }
          total += (int)__popcll(bal);
        };
        if constexpr (TK > 0) {
          float cv[TK > 0 ? TK : 1];
          float lm = -INFINITY;
#pragma unroll
          for (int c = 0; c < TK; ++c) {  // unconditional (clamped) loads, all in flight at once
            const int j = lo + lane + 64 * c;
            cv[c] = x[j < hi ? j : hi - 1];
          }
#pragma unroll
          for (int c = 0; c < TK; ++c) {
            if (lo + lane + 64 * c >= hi) cv[c] = -INFINITY;
            else lm = fmaxf(lm, cv[c]);
          }
          // th: the kk-th largest lane maximum (lanes without a candidate take no part)
          const uint32_t thk = tk_kth_key(lane < nc ? tk_key(lm) : 0u, kk);
#pragma unroll
          for (int c = 0; c < TK; ++c) compact(cv[c], lo + lane + 64 * c, thk);
        } else {
          // more candidates than the registers hold: the same steps over two streamed passes
          // (the second reads what the first brought into the caches), SB loads in flight a lane
          constexpr int SB = 8;
          float lm = -INFINITY;
          for (int j0 = lo; j0 < hi; j0 += 64 * SB) {
            float cv[SB];
#pragma unroll
            for (int c = 0; c < SB; ++c) {
              const int j = j0 + lane + 64 * c;
              cv[c] = x[j < hi ? j : hi - 1];
            }
#pragma unroll
            for (int c = 0; c < SB; ++c)
              if (j0 + lane + 64 * c < hi) lm = fmaxf(lm, cv[c]);
          }
          const uint32_t thk = tk_kth_key(lane < nc ? tk_key(lm) : 0u, kk);
          for (int j0 = lo; j0 < hi; j0 += 64 * SB) {
            float cv[SB];
#pragma unroll
            for (int c = 0; c < SB; ++c) {
              const int j = j0 + lane + 64 * c;
              cv[c] = x[j < hi ? j : hi - 1];
            }
#pragma unroll
            for (int c = 0; c < SB; ++c) compact(cv[c], j0 + lane + 64 * c, thk);
          }
        }
        if (total <= 64) {
          tk_wave_sync();
          // exact rank of each entry among the total (>= kk) ones: importance, then index
          const bool act = lane < total;
          const float v = act ? sc->v[lane] : -INFINITY;
          cj = act ? sc->j[lane] : 0x7fffffff;
          int rk = 0;
          for (int f = 0; f < total; ++f) {
            const float vf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), f));
            const int jf = __builtin_amdgcn_readlane(cj, f);
            rk += tk_before(vf, jf, v, cj) ? 1 : 0;
          }
          chosen = __ballot(act && rk < kk);
          nsel = kk;
          done = true;
        }
      }
      if (!done) {
        float pv = INFINITY;
        int pj = -1;
        for (int round = 0; round < kk; ++round) {
          float bv = -INFINITY;
          int bj = 0x7fffffff;
          for (int j = lo + lane; j < hi; j += 64) {
            const float xv = x[j];
            if (tk_before(pv, pj, xv, j) && tk_before(xv, j, bv, bj)) {
              bv = xv;
              bj = j;
            }
          }
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oj = __shfl_xor(bj, o, 64);
            if (tk_before(ov, oj, bv, bj)) {
              bv = ov;
              bj = oj;
            }
          }
          if (lane == 0) sc->sel[round] = bj;
          pv = bv;
          pj = bj;
        }
        nsel = kk;
        in_sel = true;
      }
    }
  }
  tk_wave_sync();
  // ascending: forced [0, lo), chosen (all inside [lo, hi)), forced [hi, nj), then -1
  if (in_sel) {
    if (lane < nsel) {
      const int J = sc->sel[lane];
      int pos = lo;
      for (int c = 0; c < nsel; ++c) pos += sc->sel[c] < J ? 1 : 0;
      out[pos] = J;
    }
  } else if (chosen) {
    int pos = lo;
    for (uint64_t m = chosen; m; m &= m - 1) pos += __builtin_amdgcn_readlane(cj, (int)__builtin_ctzll(m)) < cj ? 1 : 0;
    if ((chosen >> lane) & 1) out[pos] = cj;
  }
  if (lane < lo) out[lane] = lane;
  const int a = lo + nsel;
  if (lane >= a && lane < n) out[lane] = lane - a < nj - hi ? hi + (lane - a) : -1;
  tk_wave_sync();  // the scratch may be reused by the next call
}

// The selection with the fewest register slots that hold the row's free candidates (the result
// does not depend on the slot count: lane l always takes candidates lo + l + 64 c).
__device__ inline void wave_select(const float* __restrict__ x, int lo, int hi, int nj, int kk, int n,
                                   TopkScratch* sc, int32_t* __restrict__ out, int lane) {
  const int nc = hi - lo;
  if (nc <= 64 * 4) wave_select_tk<4>(x, lo, hi, nj, kk, n, sc, out, lane);
  else if (nc <= 64 * 8) wave_select_tk<8>(x, lo, hi, nj, kk, n, sc, out, lane);
  else if (nc <= 64 * 16) wave_select_tk<16>(x, lo, hi, nj, kk, n, sc, out, lane);
  else if (nc <= 64 * TK_REG) wave_select_tk<TK_REG>(x, lo, hi, nj, kk, n, sc, out, lane);
  else wave_select_tk<0>(x, lo, hi, nj, kk, n, sc, out, lane);
}

// Forced-block bounds of the row at absolute position t: free candidates [*lo, *hi), forced
// [0, *lo) and [*hi, *nj); returns kk.
__device__ __forceinline__ int tk_bounds(int64_t t, int ls, int64_t Ns, int n, int n_init, int n_local, int* lo,
                                         int* hi, int* nj) {
  const int64_t jt = t / ls;
  *nj = (int)(jt + 1 < Ns ? jt + 1 : Ns);
  *lo = n_init < *nj ? n_init : *nj;
  const int h0 = (int)jt - n_local + 1;
  *hi = h0 < *lo ? *lo : h0;
  return n - (*lo + (*nj > *hi ? *nj - *hi : 0));
}
