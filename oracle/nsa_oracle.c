/*
 * nsa_oracle.c -- plain fp64 CPU reference of the forward pass of VideoNSA's
 * hybrid attention layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the test-suite, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or table with the HIP library.
 *
 * What it follows (pages are cited by title and section):
 *  - "VideoNSA: Native Sparse Attention Scales Video Understanding"
 *    (shd-paper.top digest), English abstract: text keeps dense attention,
 *    video goes through Native Sparse Attention (hybrid routing).
 *  - top168.com digest of the same paper, section 一 (the three-branch
 *    mechanism): a compression branch that merges neighbouring content, a
 *    selection branch that scores segments by importance and attends to the
 *    chosen ones in detail, a sliding-window branch over the most recent
 *    tokens, and a learned per-head weighting of the three.
 *  - "VideoNSA：重新定义视频理解的稀疏注意力机制" (vcloud.csdn.net), section 2.2
 *    (CMP / SLC / SWA) and section 3.1 (three gate values per head).
 *  - mind-verse.de, "VideoNSA: Ein innovativer Ansatz": dense attention for
 *    text, NSA for video.
 * The pages give the roles of the branches but no formulas.  The exact
 * definitions below (block compression as a positional weighted sum, block
 * importance from the compression probabilities, top-n per GQA group with
 * forced blocks and lower-index tie-break, window semantics, ungated dense text
 * rows) are the plain readings listed with their reasons in the design notes.
 *
 * Conventions: all tensors are row-major, token-major:
 *   q   [R, Hq, D]      (only the R query rows asked for)
 *   k,v [T, Hkv, D]     (one batch element)
 *   kc,vc [Nc, Hkv, D]  compressed keys / values, fp64
 * Inputs arrive as float (bf16 and fp32 inputs are exact in float) and every
 * operation is carried out in double.  Head h uses KV head h / G, G = Hq / Hkv.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of compressed blocks: block i covers tokens [i*d, i*d + l - 1]. */
int64_t oracle_num_cmp_blocks(int64_t T, int64_t l, int64_t d) {
  if (T < l) return 0;
  return (T - l) / d + 1;
}

/* Number of selection blocks of size ls: block j covers [j*ls, j*ls + ls - 1]. */
int64_t oracle_num_sel_blocks(int64_t T, int64_t ls) { return (T + ls - 1) / ls; }

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Compression branch input: each compressed key/value is the positional
 * weighted sum of the l consecutive tokens of its block,
 *   kc[i, h, :] = sum_{m < l} w[m] * x[i*d + m, h, :].
 * (top168.com digest section 一 and the csdn page section 2.2: the compression
 * branch merges neighbouring tokens into one representative token.)
 */
void oracle_compress(const float* x, int64_t T, int64_t H, int64_t D, const float* w, int64_t l,
                     int64_t d, double* out) {
  int64_t Nc = oracle_num_cmp_blocks(T, l, d);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < Nc; ++i) {
    for (int64_t h = 0; h < H; ++h) {
      for (int64_t e = 0; e < D; ++e) {
        double s = 0.0;
        for (int64_t m = 0; m < l; ++m) s += (double)w[m] * (double)x[((i * d + m) * H + h) * D + e];
        out[(i * H + h) * D + e] = s;
      }
    }
  }
}

/* Tokens shared by compressed block i and selection block j, over l. */
static double overlap_fraction(int64_t i, int64_t j, int64_t l, int64_t d, int64_t ls) {
  int64_t a0 = i * d, a1 = i * d + l - 1;
  int64_t b0 = j * ls, b1 = j * ls + ls - 1;
  int64_t lo = a0 > b0 ? a0 : b0, hi = a1 < b1 ? a1 : b1;
  return hi >= lo ? (double)(hi - lo + 1) / (double)l : 0.0;
}

static double dot(const float* a, const double* b, int64_t n) {
  double s = 0.0;
  for (int64_t e = 0; e < n; ++e) s += (double)a[e] * b[e];
  return s;
}

static double dotf(const float* a, const float* b, int64_t n) {
  double s = 0.0;
  for (int64_t e = 0; e < n; ++e) s += (double)a[e] * (double)b[e];
  return s;
}

/*
 * Compression-branch attention and block importance for R query rows.
 * For row r at absolute position t = pos[r] and head h:
 *   visible compressed blocks C(t) = { i : i*d + l - 1 <= t }
 *   p_i = softmax_i( scale * <q, kc_i> ) over C(t);  o_cmp = sum_i p_i vc_i
 *   lse = log sum_i exp(scale * <q, kc_i>)   (-inf when C(t) is empty; o = 0)
 * Block importance of selection block j for KV head g sums the probabilities of
 * the group's heads, each compressed block weighted by the fraction of its
 * tokens that fall in j:
 *   imp[r, g, j] = sum_{h in group g} sum_{i in C(t)} frac(i, j) * p_{h,i}.
 * (top168.com digest section 一: the selection branch scores every segment by
 * importance; the score is read from the compression branch's probabilities.)
 * imp is written for all j < Ns (zero where nothing contributes).
 */
void oracle_cmp_rows(const float* q, const int64_t* pos, int64_t R, const double* kc,
                     const double* vc, int64_t Nc, int64_t Hq, int64_t Hkv, int64_t D, int64_t l,
                     int64_t d, int64_t ls, int64_t Ns, double scale, double* o, double* lse,
                     double* imp) {
  int64_t G = Hq / Hkv;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)(Nc > 0 ? Nc : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
      int64_t t = pos[r];
      int64_t nvis = (t + 1 >= l) ? (t + 1 - l) / d + 1 : 0;
      if (nvis > Nc) nvis = Nc;
      for (int64_t g = 0; g < Hkv; ++g)
        for (int64_t j = 0; j < Ns; ++j) imp[(r * Hkv + g) * Ns + j] = 0.0;
      for (int64_t h = 0; h < Hq; ++h) {
        int64_t g = h / G;
        const float* qh = q + (r * Hq + h) * D;
        double* oh = o + (r * Hq + h) * D;
        for (int64_t e = 0; e < D; ++e) oh[e] = 0.0;
        if (nvis == 0) {
          lse[r * Hq + h] = -INFINITY;
          continue;
        }
        double m = -INFINITY;
        for (int64_t i = 0; i < nvis; ++i) {
          z[i] = scale * dot(qh, kc + (i * Hkv + g) * D, D);
          if (z[i] > m) m = z[i];
        }
        double s = 0.0;
        for (int64_t i = 0; i < nvis; ++i) s += exp(z[i] - m);
        double L = m + log(s);
        lse[r * Hq + h] = L;
        for (int64_t i = 0; i < nvis; ++i) {
          double p = exp(z[i] - L);
          const double* vi = vc + (i * Hkv + g) * D;
          for (int64_t e = 0; e < D; ++e) oh[e] += p * vi[e];
          int64_t j0 = (i * d) / ls, j1 = (i * d + l - 1) / ls;
          for (int64_t j = j0; j <= j1 && j < Ns; ++j)
            imp[(r * Hkv + g) * Ns + j] += overlap_fraction(i, j, l, d, ls) * p;
        }
      }
    }
    free(z);
  }
}

/* Ranking order of free candidates: larger importance first, then lower index. */
typedef struct {
  double v;
  int64_t j;
} cand_t;

static int cand_cmp(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/*
 * Top-n block selection per (row, KV head).  Candidates are the selection
 * blocks up to the one holding t: J(t) = {0 .. t / ls}.  Forced blocks
 *   F(t) = ({0 .. n_init-1} U {jt-n_local+1 .. jt}) intersected with J(t)
 * are always taken and count inside n; the remaining n - |F| places go to the
 * free candidates in order of (importance descending, index ascending).  The
 * chosen set is written ascending and padded with -1.
 * gap[r, g] (optional) is the importance difference between the last free
 * candidate taken and the first one left out (+inf when the choice is forced:
 * no free place, or every free candidate fits).
 */
void oracle_topk_rows(const double* imp, const int64_t* pos, int64_t R, int64_t Hkv, int64_t Ns,
                      int64_t ls, int64_t n, int64_t n_init, int64_t n_local, int32_t* idx,
                      double* gap) {
#pragma omp parallel
  {
    cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)(Ns > 0 ? Ns : 1));
    char* forced = (char*)malloc((size_t)(Ns > 0 ? Ns : 1));
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < R; ++r) {
      int64_t jt = pos[r] / ls;
      for (int64_t g = 0; g < Hkv; ++g) {
        const double* row = imp + (r * Hkv + g) * Ns;
        int32_t* out = idx + (r * Hkv + g) * n;
        int64_t nf = 0, nc = 0, cnt = 0;
        for (int64_t j = 0; j <= jt && j < Ns; ++j) {
          forced[j] = (char)(j < n_init || j > jt - n_local);
          if (forced[j]) ++nf;
        }
        for (int64_t j = 0; j <= jt && j < Ns; ++j)
          if (!forced[j]) {
            cand[nc].v = row[j];
            cand[nc].j = j;
            ++nc;
          }
        qsort(cand, (size_t)nc, sizeof(cand_t), cand_cmp);
        int64_t k = n - nf;
        if (k < 0) k = 0;
        int64_t take = k < nc ? k : nc;
        for (int64_t j = 0; j <= jt && j < Ns; ++j)
          if (forced[j]) out[cnt++] = (int32_t)j;
        for (int64_t c = 0; c < take; ++c) out[cnt++] = (int32_t)cand[c].j;
        qsort(out, (size_t)cnt, sizeof(int32_t), cmp_i32);
        for (int64_t c = cnt; c < n; ++c) out[c] = -1;
        if (gap) gap[r * Hkv + g] = (k == 0 || k >= nc) ? INFINITY : cand[k - 1].v - cand[k].v;
      }
    }
    free(cand);
    free(forced);
  }
}

/*
 * Softmax attention of one query over an explicit key list (absolute token
 * positions), in fp64.  Writes the output and returns the log-sum-exp
 * (-inf and a zero output for an empty list).
 */
static double attend_list(const float* qh, const float* k, const float* v, int64_t Hkv, int64_t g,
                          int64_t D, const int64_t* keys, int64_t nk, double scale, double* z,
                          double* out) {
  for (int64_t e = 0; e < D; ++e) out[e] = 0.0;
  if (nk == 0) return -INFINITY;
  double m = -INFINITY;
  for (int64_t a = 0; a < nk; ++a) {
    z[a] = scale * dotf(qh, k + (keys[a] * Hkv + g) * D, D);
    if (z[a] > m) m = z[a];
  }
  double s = 0.0;
  for (int64_t a = 0; a < nk; ++a) s += exp(z[a] - m);
  double L = m + log(s);
  for (int64_t a = 0; a < nk; ++a) {
    double p = exp(z[a] - L);
    const float* va = v + (keys[a] * Hkv + g) * D;
    for (int64_t e = 0; e < D; ++e) out[e] += p * (double)va[e];
  }
  return L;
}

/*
 * Selection and sliding-window branches for R query rows.
 *  SLC: keys are the tokens u <= t whose selection block (u / ls) is in the
 *       row's chosen set for the head's KV group (top168.com digest section 一;
 *       csdn page section 2.2: attend at full resolution to the chosen blocks).
 *  SWA: keys are u in [max(0, t - w + 1), t], the w most recent tokens
 *       including t (top168.com digest section 一: the window keeps the latest
 *       events in detail).
 * idx is [R, Hkv, n] (ascending, -1 padded).  Either output may be NULL.
 */
void oracle_sparse_rows(const float* q, const int64_t* pos, int64_t R, const float* k,
                        const float* v, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, int64_t ls,
                        const int32_t* idx, int64_t n, int64_t w, double scale, double* o_slc,
                        double* o_swa) {
  int64_t G = Hq / Hkv;
#pragma omp parallel
  {
    int64_t cap = n * ls + w + 1;
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    double* z = (double*)malloc(sizeof(double) * (size_t)cap);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
      int64_t t = pos[r];
      for (int64_t h = 0; h < Hq; ++h) {
        int64_t g = h / G;
        const float* qh = q + (r * Hq + h) * D;
        if (o_slc) {
          int64_t nk = 0;
          const int32_t* sel = idx + (r * Hkv + g) * n;
          for (int64_t c = 0; c < n; ++c) {
            if (sel[c] < 0) continue;
            for (int64_t u = (int64_t)sel[c] * ls; u < ((int64_t)sel[c] + 1) * ls && u <= t && u < T; ++u)
              keys[nk++] = u;
          }
          attend_list(qh, k, v, Hkv, g, D, keys, nk, scale, z, o_slc + (r * Hq + h) * D);
        }
        if (o_swa) {
          int64_t nk = 0, lo = t - w + 1 > 0 ? t - w + 1 : 0;
          for (int64_t u = lo; u <= t && u < T; ++u) keys[nk++] = u;
          attend_list(qh, k, v, Hkv, g, D, keys, nk, scale, z, o_swa + (r * Hq + h) * D);
        }
      }
    }
    free(keys);
    free(z);
  }
}

/*
 * Dense causal attention for R query rows: keys are every token u <= t, text
 * and video alike.  This is the path of text rows (English abstract on the
 * shd-paper.top page; mind-verse.de, "VideoNSA: Ein innovativer Ansatz").
 * lse (optional) receives the log-sum-exp per (row, head).
 */
void oracle_dense_rows(const float* q, const int64_t* pos, int64_t R, const float* k,
                       const float* v, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, double scale,
                       double* o, double* lse) {
  int64_t G = Hq / Hkv;
#pragma omp parallel
  {
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
    double* z = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
      int64_t t = pos[r];
      int64_t nk = 0;
      for (int64_t u = 0; u <= t && u < T; ++u) keys[nk++] = u;
      for (int64_t h = 0; h < Hq; ++h) {
        double L = attend_list(q + (r * Hq + h) * D, k, v, Hkv, h / G, D, keys, nk, scale, z,
                               o + (r * Hq + h) * D);
        if (lse) lse[r * Hq + h] = L;
      }
    }
    free(keys);
    free(z);
  }
}

/*
 * Gate values of the three branches from a token's hidden state (top168.com
 * digest, section 一: a learned weighting mixes the branches per head;
 * "VideoNSA：重新定义视频理解的稀疏注意力机制", section 3.1: three gate values
 * per head come from the token's features).  Plain per-token reading: a
 * linear map of the hidden state followed by the logistic function,
 *   z[t][f] = b[f] + sum_k x[t][k] * w[f][k],   g[t][f] = 1 / (1 + exp(-z)),
 * for f = 3 h + c (head h, branch c in cmp, slc, swa order).  The pages'
 * pooled, softmax-normalised gate network is not followed.
 *   x [R, K], w [N, K], b [N] or NULL, g [R, N] (fp64).
 */
void oracle_gate_proj(const float* x, int64_t R, int64_t K, const float* w, int64_t N, const float* b,
                      double* g) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t f = 0; f < N; ++f) {
      double z = b ? (double)b[f] : 0.0;
      for (int64_t k = 0; k < K; ++k) z += (double)x[r * K + k] * (double)w[f * K + k];
      g[r * N + f] = 1.0 / (1.0 + exp(-z));
    }
  }
}

/*
 * Backward pass of one attention branch for one (row, head): softmax attention
 * of query qh over the listed keys of K / V (fp64, [N, Hkv, D], KV head g),
 * whose output enters the loss scaled by `gate` against the upstream gradient
 * dout.  With P the probabilities and E = sum_a P_a <dout, v_a>:
 *   d gate = E,   ds_a = gate * P_a * (<dout, v_a> - E),
 *   dq += scale * sum_a ds_a k_a,  dK[a] += scale * ds_a q,  dV[a] += gate * P_a dout.
 * Returns E (0 for an empty list: the branch output is 0).
 */
static double branch_bwd(const double* qh, const double* K, const double* V, int64_t Hkv, int64_t g, int64_t D,
                         const int64_t* keys, int64_t nk, double scale, double gate, const double* dout,
                         double* z, double* dpv, double* dq, double* dK, double* dV) {
  if (nk == 0) return 0.0;
  double m = -INFINITY;
  for (int64_t a = 0; a < nk; ++a) {
    const double* ka = K + (keys[a] * Hkv + g) * D;
    double s = 0.0;
    for (int64_t e = 0; e < D; ++e) s += qh[e] * ka[e];
    z[a] = scale * s;
    if (z[a] > m) m = z[a];
  }
  double sum = 0.0;
  for (int64_t a = 0; a < nk; ++a) sum += exp(z[a] - m);
  const double L = m + log(sum);
  double E = 0.0;
  for (int64_t a = 0; a < nk; ++a) {
    const double* va = V + (keys[a] * Hkv + g) * D;
    double s = 0.0;
    for (int64_t e = 0; e < D; ++e) s += dout[e] * va[e];
    dpv[a] = s;
    z[a] = exp(z[a] - L);  /* now the probability */
    E += z[a] * s;
  }
  for (int64_t a = 0; a < nk; ++a) {
    const double p = z[a], ds = gate * p * (dpv[a] - E);
    const double* ka = K + (keys[a] * Hkv + g) * D;
    double* dka = dK + (keys[a] * Hkv + g) * D;
    double* dva = dV + (keys[a] * Hkv + g) * D;
    for (int64_t e = 0; e < D; ++e) {
      dq[e] += scale * ds * ka[e];
      dka[e] += scale * ds * qh[e];
      dva[e] += gate * p * dout[e];
    }
  }
  return E;
}

/*
 * Backward pass of the hybrid layer for one batch element, the loss being
 * sum(dout * out) for the layer output out of R query rows (row r at position
 * pos[r]).  The forward is the one above: for video rows out = g_cmp o_cmp +
 * g_slc o_slc + g_swa o_swa over the branches' key sets, for text rows dense
 * causal attention (ungated).  The chosen blocks idx [R, Hkv, n] are held
 * fixed: top-n selection passes no gradient (the importance only picks
 * indices).  Compressed keys and values kc, vc [Nc, Hkv, D] are the forward's
 * positional weighted sums, so their gradients flow back to k, v and to the
 * weights w_k, w_v [l]:
 *   dk[i d + m] += w_k[m] dkc[i],   dw_k[m] = sum_i <dkc[i], k[i d + m]>   (likewise v).
 * Outputs (fp64): dq [R, Hq, D], dk, dv [T, Hkv, D], dgates [R, Hq, 3]
 * (zero for text rows), dw_k, dw_v [l].  Serial: test sizes only.
 */
void oracle_layer_bwd(const float* q, const int64_t* pos, int64_t R, const float* k, const float* v, int64_t T,
                      int64_t Hq, int64_t Hkv, int64_t D, const double* kc, const double* vc, int64_t Nc,
                      const float* w_k, const float* w_v, int64_t l, int64_t d, int64_t ls, const int32_t* idx,
                      int64_t n, int64_t w, double scale, const float* gates, const unsigned char* is_video,
                      const float* dout, double* dq, double* dk, double* dv, double* dgates, double* dw_k,
                      double* dw_v) {
  const int64_t G = Hq / Hkv;
  double* kd = (double*)malloc(sizeof(double) * (size_t)(T * Hkv * D + 1));
  double* vd = (double*)malloc(sizeof(double) * (size_t)(T * Hkv * D + 1));
  double* dkc = (double*)calloc((size_t)(Nc * Hkv * D + 1), sizeof(double));
  double* dvc = (double*)calloc((size_t)(Nc * Hkv * D + 1), sizeof(double));
  const int64_t cap = (T > Nc ? T : Nc) + 1;
  int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
  double* z = (double*)malloc(sizeof(double) * (size_t)cap);
  double* dpv = (double*)malloc(sizeof(double) * (size_t)cap);
  double qh[1024], dh[1024];
  for (int64_t x = 0; x < T * Hkv * D; ++x) {
    kd[x] = k[x];
    vd[x] = v[x];
    dk[x] = 0.0;
    dv[x] = 0.0;
  }
  for (int64_t m = 0; m < l; ++m) dw_k[m] = dw_v[m] = 0.0;
  for (int64_t r = 0; r < R; ++r) {
    const int64_t t = pos[r];
    for (int64_t h = 0; h < Hq; ++h) {
      const int64_t g = h / G, row = r * Hq + h;
      for (int64_t e = 0; e < D; ++e) {
        qh[e] = q[row * D + e];
        dh[e] = dout[row * D + e];
        dq[row * D + e] = 0.0;
      }
      double* dqh = dq + row * D;
      double* dg = dgates + row * 3;
      dg[0] = dg[1] = dg[2] = 0.0;
      if (!is_video[r]) {
        int64_t nk = 0;
        for (int64_t u = 0; u <= t && u < T; ++u) keys[nk++] = u;
        branch_bwd(qh, kd, vd, Hkv, g, D, keys, nk, scale, 1.0, dh, z, dpv, dqh, dk, dv);
        continue;
      }
      const float* gg = gates + row * 3;
      /* compression branch: the visible compressed blocks */
      int64_t nvis = (t + 1 >= l) ? (t + 1 - l) / d + 1 : 0;
      if (nvis > Nc) nvis = Nc;
      for (int64_t i = 0; i < nvis; ++i) keys[i] = i;
      dg[0] = branch_bwd(qh, kc, vc, Hkv, g, D, keys, nvis, scale, gg[0], dh, z, dpv, dqh, dkc, dvc);
      /* selection branch: tokens u <= t of the chosen blocks */
      int64_t nk = 0;
      const int32_t* sel = idx + (r * Hkv + g) * n;
      for (int64_t c = 0; c < n; ++c) {
        if (sel[c] < 0) continue;
        for (int64_t u = (int64_t)sel[c] * ls; u < ((int64_t)sel[c] + 1) * ls && u <= t && u < T; ++u)
          keys[nk++] = u;
      }
      dg[1] = branch_bwd(qh, kd, vd, Hkv, g, D, keys, nk, scale, gg[1], dh, z, dpv, dqh, dk, dv);
      /* sliding window: the w most recent tokens including t */
      nk = 0;
      for (int64_t u = (t - w + 1 > 0 ? t - w + 1 : 0); u <= t && u < T; ++u) keys[nk++] = u;
      dg[2] = branch_bwd(qh, kd, vd, Hkv, g, D, keys, nk, scale, gg[2], dh, z, dpv, dqh, dk, dv);
    }
  }
  /* back through the compression */
  for (int64_t i = 0; i < Nc; ++i)
    for (int64_t m = 0; m < l; ++m) {
      const int64_t u = i * d + m;
      for (int64_t x = 0; x < Hkv * D; ++x) {
        const double gk = dkc[i * Hkv * D + x], gv = dvc[i * Hkv * D + x];
        dk[u * Hkv * D + x] += (double)w_k[m] * gk;
        dv[u * Hkv * D + x] += (double)w_v[m] * gv;
        dw_k[m] += gk * kd[u * Hkv * D + x];
        dw_v[m] += gv * vd[u * Hkv * D + x];
      }
    }
  free(kd);
  free(vd);
  free(dkc);
  free(dvc);
  free(keys);
  free(z);
  free(dpv);
}
