// C ABI of the NSA library: argument validation, workspace layout and kernel
// dispatch.  Every entry point validates all arguments before the first launch
// and reports failures through a status code plus a thread-local message.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <cmath>

#include "../../include/nsa.h"
#include "backward.hpp"
#include "common.hpp"
#include "fast.hpp"

namespace {

thread_local char g_err[512] = "";
std::atomic<int> g_force_generic{0};

// Phase timing of nsa_hybrid_layer_fwd (measurement aid): when enabled, the
// call records a HIP event on its stream at each phase boundary.
constexpr int kMaxMarks = 8;
hipEvent_t g_marks[kMaxMarks];
int g_nmarks = 0;        // events recorded by the current pass of a profiled call
bool g_profiling = false;
// A layer call that runs in row chunks adds each pass's phase times here (g_nacc phases; 0 when the
// last call ran in one pass).
float g_acc[kMaxMarks];
int g_nacc = 0;
void prof_mark(hipStream_t s) {
  if (g_profiling && g_nmarks < kMaxMarks) (void)hipEventRecord(g_marks[g_nmarks++], s);
}


int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(NSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// Adds the phase times of the pass just recorded to g_acc (waits for its last event).
int32_t prof_accumulate() {
  if (g_nmarks < 2) return NSA_OK;
  hipError_t e = hipEventSynchronize(g_marks[g_nmarks - 1]);
  if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  if (g_nacc == 0)
    for (int i = 0; i < kMaxMarks; ++i) g_acc[i] = 0.f;
  for (int i = 0; i + 1 < g_nmarks; ++i) {
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_marks[i], g_marks[i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    g_acc[i] += ms;
  }
  g_nacc = g_nmarks - 1;
  g_nmarks = 0;
  return NSA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int64_t ncmp(int64_t T, int l, int d) { return T < l ? 0 : (T - l) / d + 1; }
int64_t nsel(int64_t T, int ls) { return (T + ls - 1) / ls; }

size_t esize(int dtype) { return dtype == NSA_BF16 ? 2 : 4; }

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Shape/parameter validation shared by the attention entry points.
int check_dims(const nsa_shape* sh, const nsa_params* pr, int32_t dtype, Dims* dm, bool need_params_topk) {
  if (!sh || !pr) return fail(NSA_ERR_INVALID_ARG, "shape and params must not be NULL");
  if (dtype != NSA_F32 && dtype != NSA_BF16) return fail(NSA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (sh->batch < 0 || sh->q_len < 0 || sh->kv_len < 0 || sh->q_start < 0)
    return fail(NSA_ERR_INVALID_ARG, "negative size in shape");
  if (sh->q_start + sh->q_len > sh->kv_len)
    return fail(NSA_ERR_INVALID_ARG, "q_start + q_len (%lld) exceeds kv_len (%lld)",
                (long long)(sh->q_start + sh->q_len), (long long)sh->kv_len);
  if (sh->num_q_heads <= 0 || sh->num_kv_heads <= 0 || sh->num_q_heads % sh->num_kv_heads != 0)
    return fail(NSA_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                sh->num_q_heads, sh->num_kv_heads);
  if (sh->head_dim <= 0) return fail(NSA_ERR_INVALID_ARG, "head_dim must be positive");
  if (sh->head_dim % 8 != 0 || sh->head_dim > 256)
    return fail(NSA_ERR_UNSUPPORTED, "head_dim %d: kernels cover multiples of 8 up to 256", sh->head_dim);
  if (pr->cmp_block <= 0 || pr->cmp_stride <= 0 || pr->sel_block <= 0)
    return fail(NSA_ERR_INVALID_ARG, "block sizes must be positive");
  if (pr->window <= 0) return fail(NSA_ERR_INVALID_ARG, "window must be positive");
  if (pr->n_init < 0 || pr->n_local < 1) return fail(NSA_ERR_INVALID_ARG, "n_init must be >= 0 and n_local >= 1");
  if (need_params_topk) {
    if (pr->top_n < pr->n_init + pr->n_local)
      return fail(NSA_ERR_INVALID_ARG, "top_n (%d) < n_init + n_local (%d)", pr->top_n, pr->n_init + pr->n_local);
    if (pr->top_n > 32) return fail(NSA_ERR_UNSUPPORTED, "top_n %d > 32", pr->top_n);
  }
  if (!(pr->scale >= 0.f) || std::isinf(pr->scale)) return fail(NSA_ERR_INVALID_ARG, "scale must be finite, >= 0");
  if (sh->kv_len > ((int64_t)1 << 31)) return fail(NSA_ERR_UNSUPPORTED, "kv_len above 2^31");
  dm->B = sh->batch;
  dm->Tq = sh->q_len;
  dm->T = sh->kv_len;
  dm->q0 = sh->q_start;
  dm->Hq = sh->num_q_heads;
  dm->Hkv = sh->num_kv_heads;
  dm->D = sh->head_dim;
  dm->G = sh->num_q_heads / sh->num_kv_heads;
  dm->l = pr->cmp_block;
  dm->d = pr->cmp_stride;
  dm->ls = pr->sel_block;
  dm->n = pr->top_n;
  dm->n_init = pr->n_init;
  dm->n_local = pr->n_local;
  dm->w = pr->window;
  dm->scale = pr->scale > 0.f ? pr->scale : 1.0f / sqrtf((float)sh->head_dim);
  dm->Nc = ncmp(sh->kv_len, pr->cmp_block, pr->cmp_stride);
  dm->Ns = nsel(sh->kv_len, pr->sel_block);
  return NSA_OK;
}

bool use_fast(int32_t dtype, const Dims& dm) { return !g_force_generic.load() && fast_supported(dtype, dm); }

// Workspace layout of nsa_sparse_attn_fwd.
struct SparseWs {
  size_t fast_bytes;
  size_t total;
};
SparseWs sparse_ws(const Dims& dm, int32_t dtype) {
  SparseWs w{};
  w.fast_bytes = fast_supported(dtype, dm) ? round_up(fast_sparse_workspace(dm)) : 0;
  w.total = w.fast_bytes;
  return w;
}

struct LayerWs {
  size_t kc, vc, kv16, o_cmp, lse, imp, idx, o_swa, sparse, dec, total;
};
// One query row per sequence on the MFMA path: the split decode kernels.
bool use_decode(int32_t dtype, const Dims& dm) { return use_fast(dtype, dm) && decode_supported(dm); }

// Sized for the kernels the call will dispatch to (nsa_set_force_generic included).
LayerWs layer_ws(const Dims& dm, int32_t dtype) {
  LayerWs w{};
  const size_t es = esize(dtype);
  const bool fast = use_fast(dtype, dm);
  // compressed keys / values computed inside the layer keep fp32 precision: bf16 high + low
  // parts on the MFMA path, fp32 on the generic path (4 bytes per element either way)
  w.kc = round_up((size_t)dm.B * dm.Nc * dm.Hkv * dm.D * 2) * 2;
  w.vc = w.kc;
  // prefill split keys: bf16 high parts, then fp8 low parts and their scales
  if (fast) w.kc += 512;
  w.lse = round_up((size_t)dm.B * dm.Tq * dm.Hq * 4);
  w.idx = round_up((size_t)dm.B * dm.Tq * dm.Hkv * dm.n * 4);
  if (fast && decode_supported(dm)) {
    w.dec = round_up(decode_workspace(dm));
  } else if (fast) {
    if (cmp_group_supported(dm)) {
      // the group kernel's fp16 key / value tiles replace the row-major compressed keys / values
      w.kc = w.vc = 0;
      w.kv16 = round_up(kv16_tiles_bytes(dm));
    }
    // fp32 branch output of the compression path (read by the combine)
    w.o_cmp = round_up((size_t)dm.B * dm.Tq * dm.Hq * dm.D * 4);
    w.imp = round_up((size_t)dm.B * dm.Tq * dm.Hkv * dm.Ns * 4);
    w.sparse = sparse_ws(dm, dtype).total;
  } else {
    w.o_cmp = round_up((size_t)dm.B * dm.Tq * dm.Hq * dm.D * es);
    w.imp = round_up((size_t)dm.B * dm.Tq * dm.Hkv * dm.Ns * 4);
    w.o_swa = round_up((size_t)dm.B * dm.Tq * dm.Hq * dm.D * es);
  }
  w.total = w.kc + w.vc + w.kv16 + w.o_cmp + w.lse + w.imp + w.idx + w.o_swa + w.sparse + w.dec;
  return w;
}

// Row chunking of the layer.  Every stage is independent across query rows except the compression
// of K / V, so a prefill on the MFMA path may run as passes over chunks of rows: per batch element,
// the compression once, then each chunk's rows with q_start moved to the chunk (bit-identical
// results).  The per-row scratch (fp32 branch outputs, importance, selection partials) then covers
// one chunk only.  Chunks are multiples of 64 rows; decode (one row) never splits.
constexpr int64_t kChunkAlign = 64;
constexpr size_t kDefaultWsCap = (size_t)7 << 30;  // default workspace bound of the layer

bool can_chunk(int32_t dtype, const Dims& dm) { return use_fast(dtype, dm) && !decode_supported(dm); }

// Rows of the chunk a pass covers when at most `rows` rows run together (0: all).
int64_t chunk_rows(const Dims& dm, int32_t dtype, int64_t rows) {
  if (rows <= 0 || rows >= dm.Tq || !can_chunk(dtype, dm)) return dm.Tq;
  return rows < kChunkAlign ? kChunkAlign : rows / kChunkAlign * kChunkAlign;
}

// The shape a chunk pass is sized for: one batch element, r rows, placed last in the sequence.
// Some scratch grows with how far the rows reach (the key splits of long text rows in the window
// pass follow q_start + rows), so the last chunk is the largest.
Dims chunk_dims(const Dims& dm, int64_t r) {
  Dims c = dm;
  c.B = 1;
  c.Tq = r;
  c.q0 = dm.q0 + dm.Tq - r;
  return c;
}

// Workspace of the layer when at most `rows` query rows run in one pass.
size_t layer_ws_rows(const Dims& dm, int32_t dtype, int64_t rows) {
  const int64_t r = chunk_rows(dm, dtype, rows);
  if (r >= dm.Tq) return layer_ws(dm, dtype).total;
  return layer_ws(chunk_dims(dm, r), dtype).total;
}

// True when every region of `need` fits the corresponding region of the carve `w`.
bool ws_fits(const LayerWs& need, const LayerWs& w) {
  return need.kc <= w.kc && need.vc <= w.vc && need.kv16 <= w.kv16 && need.o_cmp <= w.o_cmp &&
         need.lse <= w.lse && need.imp <= w.imp && need.idx <= w.idx && need.o_swa <= w.o_swa &&
         need.sparse <= w.sparse && need.dec <= w.dec;
}

// The largest chunk (all rows, else a multiple of 64) whose workspace fits `bytes`; 0 if none does.
int64_t fit_chunk_rows(const Dims& dm, int32_t dtype, size_t bytes) {
  if (layer_ws_rows(dm, dtype, 0) <= bytes) return dm.Tq;
  if (!can_chunk(dtype, dm) || layer_ws_rows(dm, dtype, kChunkAlign) > bytes) return 0;
  int64_t lo = 1, hi = (dm.Tq - 1) / kChunkAlign;  // in units of 64 rows; lo fits
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (layer_ws_rows(dm, dtype, mid * kChunkAlign) <= bytes)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo * kChunkAlign;
}

// Default: every row in one pass when that needs at most kDefaultWsCap bytes, else the largest
// chunk that stays within it, rounded down to whole kChunkRound rows when it holds any (at 128K
// the compression kernels ran ~3 % slower in passes of 43,712 rows than of 32,768 or 65,536).
constexpr int64_t kChunkRound = 16384;

int64_t default_chunk_rows(const Dims& dm, int32_t dtype) {
  const int64_t r = fit_chunk_rows(dm, dtype, kDefaultWsCap);
  if (r <= 0) return chunk_rows(dm, dtype, kChunkAlign);
  return (r < dm.Tq && r >= kChunkRound) ? r / kChunkRound * kChunkRound : r;
}

// kc/vc: compressed keys/values (bf16 high parts on the MFMA path, or cdtype on the generic path);
// kl8 / ksc / vl: on the MFMA path when the layer compressed them itself, the keys' fp8 low parts
// and their scales and the values' bf16 low parts; kv16: instead of all these, the group kernel's
// fp16 key / value tiles.
// The MFMA compression kernels take 64-token selection blocks from row-major compressed keys and
// 32-, 64- or 128-token blocks from the group kernel's tiles; other calls run the generic kernel
// (its output in dtype, no fp32 copy).
bool cmp_on_fast(int32_t dtype, const Dims& dm, bool kv16) { return use_fast(dtype, dm) && (kv16 || dm.ls == 64); }

int run_cmp(int32_t dtype, int32_t cdtype, const Dims& dm, const void* q, const void* kc, const void* kl8,
            const void* ksc, const void* vc, const void* vl, const void* kv16, const uint8_t* vid, void* o, float* o32,
            float* lse, float* imp, hipStream_t s) {
  hipError_t e;
  if (!cmp_on_fast(dtype, dm, kv16 != nullptr)) {
    e = launch_cmp_generic(dtype, cdtype, dm, q, kc, vc, vid, o, lse, imp, s);
  } else if (kv16) {
    e = launch_cmp_group(dm, q, kv16, vid, o, o32, lse, imp, s);
  } else {
    e = launch_cmp_fast(dm, q, kc, kl8, ksc, vc, vl, vid, o, o32, lse, imp, s);
  }
  if (e != hipSuccess) return hip_fail(e, "compression-branch kernel");
  return NSA_OK;
}

// Keys and values of each branch: the compression branch compresses (kc, vc); the selection
// branch reads (ks, vs); the window branch and the text rows read (kw, vw).
struct BranchKV {
  const void *kc, *vc, *ks, *vs, *kw, *vw;
  bool shared() const { return kc == ks && ks == kw && vc == vs && vs == vw; }
};

// forced_local: idx is the layer's own top-n (its forced blocks present), not a caller's set.
int run_sparse(int32_t dtype, const Dims& dm, const void* q, const BranchKV& kv, const int32_t* idx,
               const uint8_t* vid, const void* o_cmp, bool ocmp_f32, const float* gates, void* out, void* o_slc,
               void* o_swa, void* ws, hipStream_t s, bool forced_local = false) {
  hipError_t e = use_fast(dtype, dm)
                     ? launch_sparse_fast(dm, q, kv.ks, kv.vs, kv.kw, kv.vw, idx, vid, o_cmp, ocmp_f32, gates, out,
                                          o_slc, o_swa, ws, s, prof_mark, forced_local, !g_profiling)
                     : launch_sparse_generic(dtype, dm, q, kv.ks, kv.vs, kv.kw, kv.vw, idx, vid, o_cmp, gates, out,
                                             o_slc, o_swa, s);
  if (e != hipSuccess) return hip_fail(e, "selection/window kernel");
  return NSA_OK;
}

}  // namespace

extern "C" {

const char* nsa_status_string(int32_t status) {
  switch (status) {
    case NSA_OK: return "NSA_OK";
    case NSA_ERR_INVALID_ARG: return "NSA_ERR_INVALID_ARG";
    case NSA_ERR_UNSUPPORTED: return "NSA_ERR_UNSUPPORTED";
    case NSA_ERR_HIP: return "NSA_ERR_HIP";
    case NSA_ERR_WORKSPACE_TOO_SMALL: return "NSA_ERR_WORKSPACE_TOO_SMALL";
    default: return "NSA_UNKNOWN_STATUS";
  }
}

const char* nsa_last_error(void) { return g_err; }

int64_t nsa_num_cmp_blocks(int64_t kv_len, int32_t cmp_block, int32_t cmp_stride) {
  if (kv_len < 0 || cmp_block <= 0 || cmp_stride <= 0) return -1;
  return ncmp(kv_len, cmp_block, cmp_stride);
}

int64_t nsa_num_sel_blocks(int64_t kv_len, int32_t sel_block) {
  if (kv_len < 0 || sel_block <= 0) return -1;
  return nsel(kv_len, sel_block);
}

int32_t nsa_set_force_generic(int32_t on) { return g_force_generic.exchange(on ? 1 : 0); }

int32_t nsa_profile_enable(int32_t on) {
  g_err[0] = 0;
  static bool created = false;
  if (on && !created) {
    for (int i = 0; i < kMaxMarks; ++i) {
      hipError_t e = hipEventCreate(&g_marks[i]);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
    created = true;
  }
  g_profiling = on != 0;
  g_nmarks = 0;
  return NSA_OK;
}

int32_t nsa_profile_read(float* ms, int32_t max_phases) {
  g_err[0] = 0;
  if (!g_profiling) return 0;
  if (g_nacc > 0) {
    int n = 0;
    for (; n < g_nacc && n < max_phases; ++n) ms[n] = g_acc[n];
    return n;
  }
  if (g_nmarks < 2) return 0;
  hipError_t e = hipEventSynchronize(g_marks[g_nmarks - 1]);
  if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  int n = 0;
  for (int i = 0; i + 1 < g_nmarks && n < max_phases; ++i, ++n) {
    e = hipEventElapsedTime(&ms[n], g_marks[i], g_marks[i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
  }
  return n;
}

int32_t nsa_compress_kv(const void* k, const void* v, int32_t dtype, int64_t batch, int64_t kv_len,
                        int32_t num_kv_heads, int32_t head_dim, const float* w_k, const float* w_v,
                        int32_t cmp_block, int32_t cmp_stride, void* k_cmp, void* v_cmp, void* stream) {
  g_err[0] = 0;
  if (dtype != NSA_F32 && dtype != NSA_BF16) return fail(NSA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (batch < 0 || kv_len < 0 || num_kv_heads <= 0 || head_dim <= 0 || cmp_block <= 0 || cmp_stride <= 0)
    return fail(NSA_ERR_INVALID_ARG, "sizes must be positive (batch, kv_len >= 0)");
  if (head_dim % 8 != 0 || head_dim > 256)
    return fail(NSA_ERR_UNSUPPORTED, "head_dim %d: multiples of 8 up to 256", head_dim);
  const int64_t Nc = ncmp(kv_len, cmp_block, cmp_stride);
  if (Nc == 0 || batch == 0) return NSA_OK;
  if (!k || !v || !w_k || !w_v || !k_cmp || !v_cmp) return fail(NSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cmp) || !aligned16(v_cmp))
    return fail(NSA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_compress(dtype, 0, k, w_k, k_cmp, nullptr, batch, kv_len, num_kv_heads, head_dim, cmp_block,
                                 cmp_stride, Nc, s);
  if (e == hipSuccess)
    e = launch_compress(dtype, 0, v, w_v, v_cmp, nullptr, batch, kv_len, num_kv_heads, head_dim, cmp_block,
                        cmp_stride, Nc, s);
  if (e != hipSuccess) return hip_fail(e, "compress kernel");
  return NSA_OK;
}

int32_t nsa_cmp_attn_scores(const void* q, const void* k_cmp, const void* v_cmp, int32_t dtype,
                            const nsa_shape* shape, const nsa_params* params, const uint8_t* is_video,
                            void* o_cmp, float* lse, float* importance, void* stream) {
  g_err[0] = 0;
  Dims dm;
  int st = check_dims(shape, params, dtype, &dm, false);
  if (st != NSA_OK) return st;
  if (!o_cmp && !importance) return fail(NSA_ERR_INVALID_ARG, "o_cmp and importance are both NULL");
  if (dm.B == 0 || dm.Tq == 0) return NSA_OK;
  if (!q || (dm.Nc > 0 && (!k_cmp || !v_cmp))) return fail(NSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k_cmp) || !aligned16(v_cmp) || !aligned16(o_cmp))
    return fail(NSA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (!cmp_on_fast(dtype, dm, false) && dm.Ns > 16384)
    return fail(NSA_ERR_UNSUPPORTED, "generic kernel handles at most 16384 selection blocks");
  return run_cmp(dtype, dtype, dm, q, k_cmp, nullptr, nullptr, v_cmp, nullptr, nullptr, is_video, o_cmp, nullptr, lse,
                 importance,
                 (hipStream_t)stream);
}

int32_t nsa_topk_blocks(const float* importance, const nsa_shape* shape, const nsa_params* params,
                        const uint8_t* is_video, int32_t* block_idx, void* stream) {
  g_err[0] = 0;
  Dims dm;
  int st = check_dims(shape, params, NSA_F32, &dm, true);
  if (st != NSA_OK) return st;
  if (dm.B == 0 || dm.Tq == 0) return NSA_OK;
  if (!importance || !block_idx) return fail(NSA_ERR_INVALID_ARG, "NULL tensor pointer");
  hipError_t e = launch_topk(dm, importance, is_video, block_idx, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "top-n kernel");
  return NSA_OK;
}

size_t nsa_sparse_attn_workspace_size(const nsa_shape* shape, const nsa_params* params, int32_t dtype) {
  Dims dm;
  if (check_dims(shape, params, dtype, &dm, true) != NSA_OK) return 0;
  return sparse_ws(dm, dtype).total;
}

int32_t nsa_sparse_attn_fwd(const void* q, const void* k, const void* v, int32_t dtype, const nsa_shape* shape,
                            const nsa_params* params, const int32_t* block_idx, const uint8_t* is_video,
                            const void* o_cmp, const float* gates, void* out, void* o_slc, void* o_swa,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  Dims dm;
  int st = check_dims(shape, params, dtype, &dm, true);
  if (st != NSA_OK) return st;
  if (!out && !o_slc && !o_swa) return fail(NSA_ERR_INVALID_ARG, "no output requested");
  if (out && (!o_cmp || !gates)) return fail(NSA_ERR_INVALID_ARG, "out needs o_cmp and gates");
  if (dm.B == 0 || dm.Tq == 0) return NSA_OK;
  if (!q || !k || !v || !block_idx) return fail(NSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_cmp) || !aligned16(out) ||
      !aligned16(o_slc) || !aligned16(o_swa))
    return fail(NSA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  const SparseWs w = sparse_ws(dm, dtype);
  const bool fast = use_fast(dtype, dm);
  if (fast && workspace_bytes < w.total)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes, w.total);
  if (fast && w.total > 0 && !workspace) return fail(NSA_ERR_INVALID_ARG, "NULL workspace");
  return run_sparse(dtype, dm, q, BranchKV{k, v, k, v, k, v}, block_idx, is_video, o_cmp, false, gates, out, o_slc,
                    o_swa, workspace,
                    (hipStream_t)stream);
}

size_t nsa_hybrid_layer_workspace_size_rows(const nsa_shape* shape, const nsa_params* params, int32_t dtype,
                                            int64_t rows_per_chunk) {
  Dims dm;
  if (check_dims(shape, params, dtype, &dm, true) != NSA_OK) return 0;
  if (rows_per_chunk < 0) return 0;
  return layer_ws_rows(dm, dtype, rows_per_chunk);
}

size_t nsa_hybrid_layer_workspace_size(const nsa_shape* shape, const nsa_params* params, int32_t dtype) {
  Dims dm;
  if (check_dims(shape, params, dtype, &dm, true) != NSA_OK) return 0;
  return layer_ws_rows(dm, dtype, default_chunk_rows(dm, dtype));
}

}  // extern "C"

namespace {

// The tensors of one layer pass.
struct LayerIO {
  const void* q;
  BranchKV kv;
  const void *kc_in, *vc_in;
  const float* gates;
  const uint8_t* vid;
  void *out, *o_cmp, *o_slc, *o_swa;
  int32_t* idx_out;
};

// One pass of the layer over dm's rows with the workspace carved as w.  compress = false: the
// compressed K / V of an earlier pass of the same batch element are still in the workspace.
int32_t layer_pass(const Dims& dm, int32_t dtype, const LayerIO& io, const float* w_k, const float* w_v,
                   const LayerWs& w, void* workspace, bool compress, hipStream_t s) {
  const void* q = io.q;
  const BranchKV& kv = io.kv;
  const void* k_cmp_in = io.kc_in;
  const void* v_cmp_in = io.vc_in;
  const float* gates = io.gates;
  const uint8_t* is_video = io.vid;
  void* out = io.out;
  void* o_cmp = io.o_cmp;
  void* o_slc = io.o_slc;
  void* o_swa = io.o_swa;
  int32_t* block_idx_out = io.idx_out;
  int st;
  char* p = (char*)workspace;
  void* kc = p;
  p += w.kc;
  void* vc = p;
  p += w.vc;
  // the group kernel's key / value tiles, when the layer compresses K / V itself
  void* kv16 = w.kv16 && !k_cmp_in ? p : nullptr;
  p += w.kv16;
  void* ocmp_ws = p;
  p += w.o_cmp;
  float* lse = (float*)p;
  p += w.lse;
  float* imp = (float*)p;
  p += w.imp;
  int32_t* idx_ws = (int32_t*)p;
  p += w.idx;
  void* oswa_ws = p;
  p += w.o_swa;
  void* sparse_ws_ptr = p;

  g_nmarks = 0;
  prof_mark(s);
  const void* kc_use = k_cmp_in;
  const void* vc_use = v_cmp_in;
  const void* kl_use = nullptr;
  const void* ksc_use = nullptr;
  const void* vl_use = nullptr;
  int32_t cdtype = dtype;
  if (!kc_use) {
    // Compressed inside the layer, carried at fp32 precision: the MFMA path as bf16 high + low
    // parts (both enter every product), the generic path as fp32.  Prefill on the MFMA path: with
    // 4..7 query heads per KV head the group kernel's fp16 key / value tiles instead; with 8, the
    // keys' low parts in fp8 with per-group scales (the scaled fp8 product of cmp_fast_kernel).
    const bool fast = use_fast(dtype, dm);
    const bool k8 = fast && !decode_supported(dm) && !kv16;
    void* kl = fast ? (char*)kc + round_up((size_t)dm.B * dm.Nc * dm.Hkv * dm.D * 2) : nullptr;
    void* vl = fast ? (char*)vc + w.vc / 2 : nullptr;
    void* ksc = k8 ? (char*)kl + round_up(k8_lo_bytes(dm)) : nullptr;
    hipError_t e = hipSuccess;
    if (kv16) {
      if (compress) e = launch_compress_kv16(dm, kv.kc, w_k, kv.vc, w_v, kv16, s);
      kl = vl = nullptr;
    } else if (compress) {
      e = k8 ? launch_compress_k8(dm, kv.kc, w_k, kc, kl, ksc, s)
             : launch_compress(dtype, fast ? 2 : 1, kv.kc, w_k, kc, kl, dm.B, dm.T, dm.Hkv, dm.D, dm.l, dm.d, dm.Nc,
                               s);
      if (e == hipSuccess)
        e = launch_compress(dtype, fast ? 2 : 1, kv.vc, w_v, vc, vl, dm.B, dm.T, dm.Hkv, dm.D, dm.l, dm.d, dm.Nc, s);
    }
    if (e != hipSuccess) return hip_fail(e, "compress kernel");
    kc_use = kc;
    vc_use = vc;
    kl_use = kl;
    ksc_use = ksc;
    vl_use = vl;
    cdtype = fast ? dtype : NSA_F32;
  }
  if (use_decode(dtype, dm)) {
    // one row per sequence: phases = compress | compression branch + top-n | selection, window, combine
    int32_t* didx = block_idx_out ? block_idx_out : idx_ws;
    prof_mark(s);
    hipError_t e = launch_decode_fast(dm, DecVar{}, q, kc_use, kl_use, vc_use, vl_use, kv.ks, kv.vs, is_video, gates,
                                      out, o_cmp,
                                      o_slc, o_swa, didx, lse, nullptr, sparse_ws_ptr, s, prof_mark);
    if (e != hipSuccess) return hip_fail(e, "decode kernels");
    prof_mark(s);
    return NSA_OK;
  }
  const bool fast = use_fast(dtype, dm);
  // MFMA path: the combine reads an fp32 copy of the compression output; the caller's bf16 copy is
  // optional.  Compression on the generic kernel (caller's compressed keys with 32- or 128-token
  // selection blocks): its output in dtype, in the fp32 buffer's space when the caller gives none.
  const bool c32 = cmp_on_fast(dtype, dm, kv16 != nullptr);
  prof_mark(s);
  void* ocmp = c32 ? o_cmp : (o_cmp ? o_cmp : ocmp_ws);
  float* ocmp32 = c32 ? (float*)ocmp_ws : nullptr;
  const void* ocmb = c32 ? (const void*)ocmp32 : ocmp;  // what the combine reads
  int32_t* idx = block_idx_out ? block_idx_out : idx_ws;
  st = run_cmp(dtype, cdtype, dm, q, kc_use, kl_use, ksc_use, vc_use, vl_use, kv16, is_video,
               ocmp, ocmp32, lse, imp, s);
  if (st != NSA_OK) return st;
  prof_mark(s);
  // The window pass needs neither the compression branch nor the top-n: outside phase timing it
  // starts here on the side stream, beside the top-n and the selection kernels.
  const SideStream* side = (fast && !g_profiling) ? side_stream(s) : nullptr;
  if (side) {
    hipError_t e = launch_sparse_window(dm, q, kv.ks, kv.vs, kv.kw, kv.vw, is_video, out, o_swa, sparse_ws_ptr, s,
                                        side, true);
    const char* where = "window kernel";
    if (e == hipSuccess) {
      e = launch_topk(dm, imp, is_video, idx, s);
      where = "top-n kernel";
    }
    if (e == hipSuccess) {
      e = launch_sparse_select(dm, q, kv.ks, kv.vs, kv.kw, kv.vw, idx, is_video, ocmb, c32, gates, out, o_slc,
                               o_swa, sparse_ws_ptr, s, side, true);
      where = "selection kernels";
    }
    if (e != hipSuccess) {
      (void)join_side_stream(side, s);  // the caller's stream still waits for the forked window pass
      return hip_fail(e, where);
    }
    return NSA_OK;
  }
  hipError_t e = launch_topk(dm, imp, is_video, idx, s);
  if (e != hipSuccess) return hip_fail(e, "top-n kernel");
  prof_mark(s);
  if (fast) {
    st = run_sparse(dtype, dm, q, kv, idx, is_video, ocmb, c32, gates, out, o_slc, o_swa, sparse_ws_ptr, s,
                    true);
    prof_mark(s);
    return st;
  }
  void* oswa = o_swa ? o_swa : oswa_ws;
  return run_sparse(dtype, dm, q, kv, idx, is_video, ocmp, false, gates, out, o_slc, oswa, sparse_ws_ptr, s);
}

// The whole layer (nsa_hybrid_layer_fwd and its per-branch K/V form).
int32_t layer_fwd(const void* q, const BranchKV& kv, const void* k_cmp_in, const void* v_cmp_in,
                  const float* w_k, const float* w_v, const float* gates, const uint8_t* is_video, int32_t dtype,
                  const nsa_shape* shape, const nsa_params* params, void* out, void* o_cmp, void* o_slc,
                  void* o_swa, int32_t* block_idx_out, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  Dims dm;
  int st = check_dims(shape, params, dtype, &dm, true);
  if (st != NSA_OK) return st;
  if (!out) return fail(NSA_ERR_INVALID_ARG, "out must not be NULL");
  if ((k_cmp_in == nullptr) != (v_cmp_in == nullptr))
    return fail(NSA_ERR_INVALID_ARG, "give both k_cmp_in and v_cmp_in, or neither");
  if (dm.B == 0 || dm.Tq == 0) return NSA_OK;
  // the compression's keys / values are not read when the compressed cache is given
  if (!q || (!k_cmp_in && (!kv.kc || !kv.vc)) || !kv.ks || !kv.vs || !kv.kw || !kv.vw || !gates)
    return fail(NSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!k_cmp_in && dm.Nc > 0 && (!w_k || !w_v)) return fail(NSA_ERR_INVALID_ARG, "NULL compression weights");
  if (!aligned16(q) || !aligned16(kv.kc) || !aligned16(kv.vc) || !aligned16(kv.ks) || !aligned16(kv.vs) ||
      !aligned16(kv.kw) || !aligned16(kv.vw) || !aligned16(out) || !aligned16(o_cmp) || !aligned16(o_slc) ||
      !aligned16(o_swa) || !aligned16(k_cmp_in) || !aligned16(v_cmp_in) || !aligned16(workspace))
    return fail(NSA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  // the decode kernels score a block once for the selection and the window branch
  if (use_decode(dtype, dm) && !(kv.ks == kv.kw && kv.vs == kv.vw))
    return fail(NSA_ERR_UNSUPPORTED, "one query row per sequence needs one K/V for selection and window");
  if (!cmp_on_fast(dtype, dm, !k_cmp_in && cmp_group_supported(dm)) && dm.Ns > 16384)
    return fail(NSA_ERR_UNSUPPORTED, "generic kernels handle at most 16384 selection blocks");
  if (!workspace) return fail(NSA_ERR_INVALID_ARG, "NULL workspace");
  int64_t rows = fit_chunk_rows(dm, dtype, workspace_bytes);
  if (rows == 0)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                layer_ws_rows(dm, dtype, kChunkAlign));
  hipStream_t s = (hipStream_t)stream;
  const LayerIO io{q, kv, k_cmp_in, v_cmp_in, gates, is_video, out, o_cmp, o_slc, o_swa, block_idx_out};
  g_nacc = 0;
  if (rows >= dm.Tq) return layer_pass(dm, dtype, io, w_k, w_v, layer_ws(dm, dtype), workspace, true, s);
  // as few chunks as fit, of equal size (a multiple of 64 rows, at most `rows`)
  {
    const int64_t nch = (dm.Tq + rows - 1) / rows;
    const int64_t even = ((dm.Tq + nch - 1) / nch + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
    rows = even < rows ? even : rows;
  }

  // Row chunks of at most `rows` rows, one batch element at a time (the rows of one element are
  // contiguous in every [B, q_len, ...] tensor).
  Dims c = chunk_dims(dm, rows);
  const LayerWs w = layer_ws(c, dtype);
  // every chunk's scratch within the carve, checked before the first launch
  for (int64_t r0 = 0; r0 < dm.Tq; r0 += rows) {
    c.Tq = dm.Tq - r0 < rows ? dm.Tq - r0 : rows;
    c.q0 = dm.q0 + r0;
    if (!ws_fits(layer_ws(c, dtype), w))
      return fail(NSA_ERR_UNSUPPORTED, "internal: scratch of rows %lld..%lld exceeds its chunk layout",
                  (long long)r0, (long long)(r0 + c.Tq));
  }
  const int64_t qrow = (int64_t)dm.Hq * dm.D * esize(dtype);  // bytes per query row of q / out / o_*
  auto off = [](const void* p, int64_t bytes) -> const void* { return p ? (const char*)p + bytes : nullptr; };
  auto offm = [](void* p, int64_t bytes) -> void* { return p ? (char*)p + bytes : nullptr; };
  for (int64_t b = 0; b < dm.B; ++b) {
    const int64_t kvb = b * dm.T * dm.Hkv * dm.D * esize(dtype);
    const int64_t kcb = b * dm.Nc * dm.Hkv * dm.D * esize(dtype);
    for (int64_t r0 = 0; r0 < dm.Tq; r0 += rows) {
      c.Tq = dm.Tq - r0 < rows ? dm.Tq - r0 : rows;
      c.q0 = dm.q0 + r0;
      const int64_t rb = b * dm.Tq + r0;  // row index into [B, q_len, ...]
      LayerIO ic;
      ic.q = off(q, rb * qrow);
      ic.kv = BranchKV{off(kv.kc, kvb), off(kv.vc, kvb), off(kv.ks, kvb), off(kv.vs, kvb), off(kv.kw, kvb),
                       off(kv.vw, kvb)};
      ic.kc_in = off(k_cmp_in, kcb);
      ic.vc_in = off(v_cmp_in, kcb);
      ic.gates = gates + rb * dm.Hq * 3;
      ic.vid = is_video ? is_video + rb : nullptr;
      ic.out = offm(out, rb * qrow);
      ic.o_cmp = offm(o_cmp, rb * qrow);
      ic.o_slc = offm(o_slc, rb * qrow);
      ic.o_swa = offm(o_swa, rb * qrow);
      ic.idx_out = block_idx_out ? block_idx_out + rb * dm.Hkv * dm.n : nullptr;
      st = layer_pass(c, dtype, ic, w_k, w_v, w, workspace, r0 == 0, s);
      if (st != NSA_OK) return st;
      if (g_profiling) {
        st = prof_accumulate();
        if (st != NSA_OK) return st;
      }
    }
  }
  return NSA_OK;
}

}  // namespace

extern "C" {

int32_t nsa_hybrid_layer_fwd(const void* q, const void* k, const void* v, const void* k_cmp_in,
                             const void* v_cmp_in, const float* w_k, const float* w_v, const float* gates,
                             const uint8_t* is_video, int32_t dtype, const nsa_shape* shape,
                             const nsa_params* params, void* out, void* o_cmp, void* o_slc, void* o_swa,
                             int32_t* block_idx_out, void* workspace, size_t workspace_bytes, void* stream) {
  return layer_fwd(q, BranchKV{k, v, k, v, k, v}, k_cmp_in, v_cmp_in, w_k, w_v, gates, is_video, dtype, shape,
                   params, out, o_cmp, o_slc, o_swa, block_idx_out, workspace, workspace_bytes, stream);
}

int32_t nsa_hybrid_layer_fwd_branch_kv(const void* q, const void* k_c, const void* v_c, const void* k_s,
                                       const void* v_s, const void* k_w, const void* v_w, const void* k_cmp_in,
                                       const void* v_cmp_in, const float* w_k, const float* w_v,
                                       const float* gates, const uint8_t* is_video, int32_t dtype,
                                       const nsa_shape* shape, const nsa_params* params, void* out, void* o_cmp,
                                       void* o_slc, void* o_swa, int32_t* block_idx_out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return layer_fwd(q, BranchKV{k_c, v_c, k_s, v_s, k_w, v_w}, k_cmp_in, v_cmp_in, w_k, w_v, gates, is_video,
                   dtype, shape, params, out, o_cmp, o_slc, o_swa, block_idx_out, workspace, workspace_bytes,
                   stream);
}

// Shape of a decode batch: one query row per sequence at its own length.
static int decode_dims(const nsa_shape* shape, const nsa_params* params, int32_t dtype, const int32_t* page_table,
                       int32_t max_pages, int64_t num_pages, Dims* dm) {
  if (!shape) return fail(NSA_ERR_INVALID_ARG, "shape must not be NULL");
  if (shape->q_len != 1) return fail(NSA_ERR_INVALID_ARG, "q_len must be 1 (one query row per sequence)");
  if (shape->kv_len < 1) return fail(NSA_ERR_INVALID_ARG, "kv_len (the per-sequence capacity) must be >= 1");
  nsa_shape sh = *shape;
  sh.q_start = sh.kv_len - 1;
  int st = check_dims(&sh, params, dtype, dm, true);
  if (st != NSA_OK) return st;
  if (page_table) {
    if (max_pages < 1 || (int64_t)max_pages * kPageRows < dm->T)
      return fail(NSA_ERR_INVALID_ARG, "max_pages (%d) x %d rows must cover kv_len (%lld)", max_pages, kPageRows,
                  (long long)dm->T);
    if (num_pages < 1) return fail(NSA_ERR_INVALID_ARG, "num_pages must be >= 1");
  }
  if (!use_decode(dtype, *dm))
    return fail(NSA_ERR_UNSUPPORTED,
                "decode kernels cover bf16, head_dim 128, cmp_block 32, cmp_stride 16, sel_block 64, 4..8 query "
                "heads per KV head and kv_len >= cmp_block (generic kernels not forced)");
  return NSA_OK;
}

static size_t decode_ws_bytes(const Dims& dm) {
  return round_up(decode_workspace(dm)) + round_up((size_t)dm.B * dm.Hkv * dm.n * 4);
}

size_t nsa_decode_workspace_size(const nsa_shape* shape, const nsa_params* params, int32_t dtype) {
  Dims dm;
  if (decode_dims(shape, params, dtype, nullptr, 0, 0, &dm) != NSA_OK) return 0;
  return decode_ws_bytes(dm);
}

int32_t nsa_decode_fwd(const void* q, const void* k, const void* v, const void* k_cmp, const void* v_cmp,
                       const float* gates, const uint8_t* is_video, int32_t dtype, const nsa_shape* shape,
                       const nsa_params* params, const int32_t* kv_lens, const int32_t* page_table,
                       int32_t max_pages, int64_t num_pages, void* out, void* o_cmp, void* o_slc, void* o_swa,
                       int32_t* block_idx_out, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  Dims dm;
  int st = decode_dims(shape, params, dtype, page_table, max_pages, num_pages, &dm);
  if (st != NSA_OK) return st;
  if (!out) return fail(NSA_ERR_INVALID_ARG, "out must not be NULL");
  if (dm.B == 0) return NSA_OK;
  if (!q || !k || !v || !k_cmp || !v_cmp || !gates) return fail(NSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_cmp) || !aligned16(v_cmp) ||
      !aligned16(out) || !aligned16(o_cmp) || !aligned16(o_slc) || !aligned16(o_swa) || !aligned16(workspace))
    return fail(NSA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  const size_t need = decode_ws_bytes(dm);
  if (workspace_bytes < need)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (!workspace) return fail(NSA_ERR_INVALID_ARG, "NULL workspace");
  DecVar dv;
  dv.lens = kv_lens;
  dv.pages = page_table;
  dv.max_pages = page_table ? max_pages : 0;
  dv.num_pages = page_table ? num_pages : 0;
  char* p = (char*)workspace;
  int32_t* idx = block_idx_out ? block_idx_out : (int32_t*)p;
  p += round_up((size_t)dm.B * dm.Hkv * dm.n * 4);
  hipError_t e = launch_decode_fast(dm, dv, q, k_cmp, nullptr, v_cmp, nullptr, k, v, is_video, gates, out, o_cmp,
                                    o_slc, o_swa, idx, nullptr, nullptr, p, (hipStream_t)stream, nullptr);
  if (e != hipSuccess) return hip_fail(e, "decode kernels");
  return NSA_OK;
}

int32_t nsa_decode_fwd_noalloc(const void* q, const void* k, const void* v, const void* k_cmp, const void* v_cmp,
                               const float* gates, const uint8_t* is_video, int32_t dtype, const nsa_shape* shape,
                               const nsa_params* params, const int32_t* kv_lens, const int32_t* page_table,
                               int32_t max_pages, int64_t num_pages, void* out, void* o_cmp, void* o_slc,
                               void* o_swa, int32_t* block_idx_out, void* stream) {
  g_err[0] = 0;
  Dims dm;
  int st = decode_dims(shape, params, dtype, page_table, max_pages, num_pages, &dm);
  if (st != NSA_OK) return st;
  if (!out) return fail(NSA_ERR_INVALID_ARG, "out must not be NULL");
  if (dm.B == 0) return NSA_OK;
  if (!q || !k || !v || !k_cmp || !v_cmp || !gates) return fail(NSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_cmp) || !aligned16(v_cmp) ||
      !aligned16(out) || !aligned16(o_cmp) || !aligned16(o_slc) || !aligned16(o_swa))
    return fail(NSA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  const size_t need = decode_ws_bytes(dm);
  if (need > noalloc_scratch_bytes())
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL,
                "this decode batch needs %zu bytes of scratch; the library's device array holds %zu "
                "(use nsa_decode_fwd with a caller workspace)", need, noalloc_scratch_bytes());
  void* ws = nullptr;
  size_t ws_bytes = 0;
  hipError_t e = noalloc_scratch(&ws, &ws_bytes);
  if (e != hipSuccess) return hip_fail(e, "scratch address (hipGetSymbolAddress)");
  DecVar dv;
  dv.lens = kv_lens;
  dv.pages = page_table;
  dv.max_pages = page_table ? max_pages : 0;
  dv.num_pages = page_table ? num_pages : 0;
  char* p = (char*)ws;
  int32_t* idx = block_idx_out ? block_idx_out : (int32_t*)p;
  p += round_up((size_t)dm.B * dm.Hkv * dm.n * 4);
  e = launch_decode_fast(dm, dv, q, k_cmp, nullptr, v_cmp, nullptr, k, v, is_video, gates, out, o_cmp, o_slc, o_swa,
                         idx, nullptr, nullptr, p, (hipStream_t)stream, nullptr);
  if (e != hipSuccess) return hip_fail(e, "decode kernels");
  return NSA_OK;
}

int32_t nsa_compress_append(const void* k, const void* v, int32_t dtype, int64_t batch, int64_t kv_len,
                            int32_t num_kv_heads, int32_t head_dim, const float* w_k, const float* w_v,
                            int32_t cmp_block, int32_t cmp_stride, const int32_t* kv_lens, const int32_t* page_table,
                            int32_t max_pages, int64_t num_pages, int32_t n_new, void* k_cmp, void* v_cmp,
                            void* stream) {
  g_err[0] = 0;
  if (dtype != NSA_F32 && dtype != NSA_BF16) return fail(NSA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (batch < 0 || kv_len < 1 || num_kv_heads <= 0 || head_dim <= 0 || cmp_block <= 0 || cmp_stride <= 0)
    return fail(NSA_ERR_INVALID_ARG, "sizes must be positive (batch >= 0)");
  if (n_new < 0) return fail(NSA_ERR_INVALID_ARG, "n_new must be >= 0");
  if (kv_len > ((int64_t)1 << 31)) return fail(NSA_ERR_UNSUPPORTED, "kv_len above 2^31");
  if (dtype != NSA_BF16 || head_dim != 128)
    return fail(NSA_ERR_UNSUPPORTED, "compressed-cache append covers bf16 with head_dim 128");
  if (page_table && (max_pages < 1 || (int64_t)max_pages * kPageRows < kv_len || num_pages < 1))
    return fail(NSA_ERR_INVALID_ARG, "page table: max_pages x %d rows must cover kv_len and num_pages >= 1",
                kPageRows);
  Dims dm{};
  dm.B = batch;
  dm.T = kv_len;
  dm.Tq = 1;
  dm.q0 = kv_len - 1;
  dm.Hkv = num_kv_heads;
  dm.Hq = num_kv_heads;
  dm.G = 1;
  dm.D = head_dim;
  dm.l = cmp_block;
  dm.d = cmp_stride;
  dm.Nc = ncmp(kv_len, cmp_block, cmp_stride);
  if (dm.Nc == 0 || batch == 0 || n_new == 0) return NSA_OK;
  // no sequence holds more than kv_len tokens, so no block completes earlier than that
  if ((int64_t)n_new > kv_len) n_new = (int32_t)kv_len;
  if (!k || !v || !w_k || !w_v || !k_cmp || !v_cmp) return fail(NSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cmp) || !aligned16(v_cmp))
    return fail(NSA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  DecVar dv;
  dv.lens = kv_lens;
  dv.pages = page_table;
  dv.max_pages = page_table ? max_pages : 0;
  dv.num_pages = page_table ? num_pages : 0;
  hipError_t e = launch_compress_append(dm, dv, k, v, w_k, w_v, k_cmp, v_cmp, n_new, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "compressed-cache append kernel");
  return NSA_OK;
}

int32_t nsa_gate_proj(const void* x, const void* w_g, const float* b_g, int32_t dtype, int64_t batch,
                      int64_t seq_len, int32_t hidden, int32_t num_q_heads, float* gates, void* stream) {
  g_err[0] = 0;
  if (dtype != NSA_F32 && dtype != NSA_BF16) return fail(NSA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (batch < 0 || seq_len < 0 || hidden <= 0 || num_q_heads <= 0)
    return fail(NSA_ERR_INVALID_ARG, "sizes must be positive (batch, seq_len >= 0)");
  const int N = 3 * num_q_heads;
  if (dtype != NSA_BF16 || !gate_proj_supported(hidden, N))
    return fail(NSA_ERR_UNSUPPORTED, "gate projection covers bf16, hidden a multiple of 64, num_q_heads <= 32");
  const int64_t R = batch * seq_len;
  if (R == 0) return NSA_OK;
  if (!x || !w_g || !gates) return fail(NSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(x) || !aligned16(w_g) || !aligned16(gates))
    return fail(NSA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  hipError_t e = launch_gate_proj(x, w_g, b_g, gates, R, hidden, N, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "gate projection kernel");
  return NSA_OK;
}

// Backward workspace: enough for either set of kernels when the matrix-core one applies (it also
// needs 16-byte aligned tensors, which only the call sees).
static size_t bwd_need(int32_t dtype, const Dims& dm) {
  const size_t gen = bwd_workspace(dm);
  if (g_force_generic.load() || !bwd_fast_supported(dtype, dm)) return gen;
  const size_t fast = bwd_fast_workspace(dm);
  return fast > gen ? fast : gen;
}

size_t nsa_hybrid_layer_bwd_workspace_size(const nsa_shape* shape, const nsa_params* params, int32_t dtype) {
  Dims dm;
  if (check_dims(shape, params, dtype, &dm, true) != NSA_OK) return 0;
  return bwd_need(dtype, dm);
}

int32_t nsa_hybrid_layer_bwd(const void* q, const void* k, const void* v, const float* w_k, const float* w_v,
                             const float* gates, const uint8_t* is_video, const int32_t* block_idx,
                             const void* d_out, int32_t dtype, const nsa_shape* shape, const nsa_params* params,
                             float* dq, float* dk, float* dv, float* d_gates, float* dw_k, float* dw_v,
                             void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  Dims dm;
  int st = check_dims(shape, params, dtype, &dm, true);
  if (st != NSA_OK) return st;
  if (dm.B == 0 || dm.Tq == 0) return NSA_OK;
  if (!q || !k || !v || !gates || !block_idx || !d_out || !dq || !dk || !dv || !d_gates || !dw_k || !dw_v)
    return fail(NSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (dm.Nc > 0 && (!w_k || !w_v)) return fail(NSA_ERR_INVALID_ARG, "NULL compression weights");
  const bool fast = !g_force_generic.load() && bwd_fast_supported(dtype, dm) && aligned16(q) && aligned16(k) &&
                    aligned16(v) && aligned16(d_out) && aligned16(dq) && aligned16(dk) && aligned16(dv);
  if (!fast && !bwd_supported(dm))
    return fail(NSA_ERR_UNSUPPORTED, "backward kernels cover head_dim 64, 128, 192, 256");
  const size_t need = bwd_need(dtype, dm);
  if (workspace_bytes < need)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (need > 0 && !workspace) return fail(NSA_ERR_INVALID_ARG, "NULL workspace");
  hipError_t e = fast ? launch_layer_bwd_fast(dm, q, k, v, w_k, w_v, gates, is_video, block_idx, d_out, dq, dk, dv,
                                              d_gates, dw_k, dw_v, workspace, (hipStream_t)stream)
                      : launch_layer_bwd(dtype, dm, q, k, v, w_k, w_v, gates, is_video, block_idx, d_out, dq, dk,
                                         dv, d_gates, dw_k, dw_v, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "backward kernels");
  return NSA_OK;
}

}  // extern "C"
