/*
 * nsa.h -- C ABI of the MI355X (gfx950) forward pass of VideoNSA's hybrid
 * attention layer: dense causal attention for text rows, Native Sparse
 * Attention (three gated branches) for video rows.
 *
 * Sources (cited by page title and section):
 *  [A] "VideoNSA: Native Sparse Attention Scales Video Understanding"
 *      (shd-paper.top digest), English abstract: hardware-aware hybrid
 *      attention, dense for text, NSA for video.
 *  [B] top168.com digest of the same paper, section 一: the compression branch
 *      merges neighbouring content into representative tokens; the selection
 *      branch scores every segment by importance and attends to the chosen
 *      ones in detail; the sliding-window branch keeps the latest tokens; a
 *      learned weighting mixes the three per head.
 *  [C] "VideoNSA：重新定义视频理解的稀疏注意力机制" (vcloud.csdn.net), section
 *      2.2 (CMP / SLC / SWA) and section 3.1 (three gate values per head).
 *  [D] mind-verse.de, "Innovative Ansätze zur Verbesserung des
 *      Videoverständnisses in KI-Modellen", section "VideoNSA: Ein innovativer
 *      Ansatz": dense attention for text, NSA for video.
 * The pages name the branches but give no formulas; the exact definitions
 * stated with each call below are the plain readings of them.
 *
 * General rules for every call
 *  - Tensor pointers are DEVICE memory owned by the caller; the library never
 *    allocates, frees, synchronises or prints.  Scratch memory, where needed,
 *    is a caller-owned workspace whose size the matching *_workspace_size call
 *    reports.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null
 *    stream) and returns an nsa_status.  Arguments are validated before any
 *    launch; on failure nothing is launched and nsa_last_error() describes it.
 *  - nsa_hybrid_layer_fwd(_branch_kv) and nsa_sparse_attn_fwd may run their
 *    window pass (window branch and text rows) on a second stream that the
 *    library creates once per calling thread and device (default priority,
 *    kept until the process ends): it is forked from `stream` after earlier
 *    work there and joined back into `stream` before the call's last kernel,
 *    so all of the call's work is ordered after what precedes it on `stream`
 *    and complete before what follows.  The first call of a thread made while
 *    `stream` is being captured into a graph, every call while phase timing
 *    is on, and calls whose `stream` belongs to another device than the
 *    current one keep to `stream` alone.
 *  - Layouts are row-major and token-major:
 *      q, o_* , out   [B, q_len, Hq, D]      (dtype)
 *      k, v           [B, kv_len, Hkv, D]    (dtype)
 *      k_cmp, v_cmp   [B, Nc, Hkv, D]        (dtype)
 *      lse            [B, q_len, Hq]          fp32, natural log
 *      importance     [B, q_len, Hkv, Ns]     fp32
 *      block_idx      [B, q_len, Hkv, top_n]  int32, ascending, -1 padded
 *      gates          [B, q_len, Hq, 3]       fp32 (cmp, slc, swa)
 *      is_video       [B, q_len]              uint8 (non-zero = video row);
 *                                             NULL means every row is video
 *    with Nc = floor((kv_len - cmp_block) / cmp_stride) + 1 (0 when
 *    kv_len < cmp_block) and Ns = ceil(kv_len / sel_block).
 *  - Row r of q sits at absolute token position q_start + r.  Head h reads KV
 *    head h / G with G = Hq / Hkv (GQA groups of consecutive heads).
 *  - Calls are reentrant; concurrent calls must use disjoint outputs.
 */
#ifndef NSA_H
#define NSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define NSA_OK 0
#define NSA_ERR_INVALID_ARG (-1)         /* bad pointer, size or parameter */
#define NSA_ERR_UNSUPPORTED (-2)         /* valid, but no kernel covers it   */
#define NSA_ERR_HIP (-3)                 /* a HIP runtime / launch error     */
#define NSA_ERR_WORKSPACE_TOO_SMALL (-4) /* workspace smaller than required  */

/* Element types of q / k / v / compressed k, v / branch outputs. */
#define NSA_F32 0
#define NSA_BF16 1

typedef struct {
  int64_t batch;     /* B                                              */
  int64_t q_len;     /* rows of q                                      */
  int64_t kv_len;    /* tokens of k / v                                */
  int64_t q_start;   /* absolute position of q's row 0; q_start + q_len <= kv_len */
  int32_t num_q_heads;  /* Hq                                          */
  int32_t num_kv_heads; /* Hkv, divides Hq                             */
  int32_t head_dim;     /* D                                           */
} nsa_shape;

typedef struct {
  int32_t cmp_block;  /* l: tokens per compressed block (e.g. 32)      */
  int32_t cmp_stride; /* d: stride between compressed blocks (e.g. 16) */
  int32_t sel_block;  /* l': tokens per selection block (e.g. 64)      */
  int32_t top_n;      /* n: selection blocks per (row, KV group)       */
  int32_t n_init;     /* leading blocks always selected (e.g. 1)       */
  int32_t n_local;    /* most recent blocks always selected (e.g. 2)   */
  int32_t window;     /* w: sliding-window length in tokens            */
  float scale;        /* softmax scale; 0 means 1/sqrt(D)              */
} nsa_params;

/* Name of a status code (static string). */
const char* nsa_status_string(int32_t status);

/* Message of the calling thread's last failed call ("" if none). */
const char* nsa_last_error(void);

/* Nc and Ns as defined above. */
int64_t nsa_num_cmp_blocks(int64_t kv_len, int32_t cmp_block, int32_t cmp_stride);
int64_t nsa_num_sel_blocks(int64_t kv_len, int32_t sel_block);

/*
 * nsa_compress_kv -- compression-branch keys and values ([B] section 一, [C]
 * section 2.2: neighbouring tokens merged into one block token).
 * Each compressed token is the positional weighted sum of its block:
 *   k_cmp[b, i, h, :] = sum_{m < cmp_block} w_k[m] * k[b, i*cmp_stride + m, h, :]
 * and likewise v_cmp with w_v.  Accumulation is fp32; results are rounded
 * once to dtype.  w_k, w_v: device fp32 [cmp_block].  Writes Nc blocks; with
 * Nc = 0 it launches nothing.  Supported: head_dim a multiple of 8, <= 256.
 */
int32_t nsa_compress_kv(const void* k, const void* v, int32_t dtype, int64_t batch, int64_t kv_len,
                        int32_t num_kv_heads, int32_t head_dim, const float* w_k, const float* w_v,
                        int32_t cmp_block, int32_t cmp_stride, void* k_cmp, void* v_cmp, void* stream);

/*
 * nsa_cmp_attn_scores -- compression-branch attention and block importance
 * for the video rows ([B] section 一: the selection branch scores segments by
 * importance; the score is taken from the compression branch's attention).
 * For row t (absolute position) and head h:
 *   C(t) = { i < Nc : i*cmp_stride + cmp_block - 1 <= t }   (whole block <= t)
 *   p_i = softmax_i(scale * <q_t,h , k_cmp_i>) over C(t),  o_cmp = sum p_i v_cmp_i,
 *   lse = log sum_i exp(scale * <q, k_cmp_i>);  C(t) empty -> o_cmp = 0, lse = -inf.
 *   importance[t, g, j] = sum_{h in group g} sum_{i in C(t)} frac(i, j) * p_{h,i}
 * where frac(i, j) is the share of compressed block i's tokens that lie in
 * selection block j.  For a video row every candidate j <= t / sel_block is
 * written (0 where nothing contributes); later blocks are left untouched.
 * Text rows are skipped: their outputs are left untouched.
 * o_cmp and lse may be NULL.  importance may be NULL only if o_cmp is given.
 * Supported: head_dim <= 256 and a multiple of 8; top_n <= 32 is not needed here.
 */
int32_t nsa_cmp_attn_scores(const void* q, const void* k_cmp, const void* v_cmp, int32_t dtype,
                            const nsa_shape* shape, const nsa_params* params, const uint8_t* is_video,
                            void* o_cmp, float* lse, float* importance, void* stream);

/*
 * nsa_topk_blocks -- selection of the top-n blocks per (video row, KV group).
 * Candidates are J(t) = {0 .. t / sel_block}.  The forced blocks
 *   F(t) = ({0 .. n_init-1} U {jt-n_local+1 .. jt}) intersected with J(t)
 * are always taken and count inside top_n; the remaining places go to the
 * free candidates by (importance descending, index ascending).  The set is
 * written ascending and padded with -1.  Text rows are skipped.
 * Errors: top_n < n_init + n_local, or top_n > 32 (UNSUPPORTED).
 */
int32_t nsa_topk_blocks(const float* importance, const nsa_shape* shape, const nsa_params* params,
                        const uint8_t* is_video, int32_t* block_idx, void* stream);

/*
 * nsa_sparse_attn_fwd -- selection and sliding-window branches, the gated
 * combine of the video rows, and dense causal attention of the text rows.
 *  SLC: keys u <= t whose selection block u / sel_block is in block_idx[t, g]
 *       ([B] section 一, [C] section 2.2: attend in full to the chosen blocks).
 *  SWA: keys u in [max(0, t - window + 1), t] ([B] section 一).
 *  out (video rows) = g_cmp*o_cmp + g_slc*o_slc + g_swa*o_swa with the given
 *       gate values, no normalisation ([B] section 一, [C] section 3.1).
 *  out (text rows)  = softmax(scale * q K_{<=t}^T) V_{<=t} over every token,
 *       ungated ([A] abstract, [D]).
 * o_slc, o_swa, out may each be NULL (at least one given).  out needs o_cmp
 * and gates.  block_idx must hold valid sets (entries < Ns, ascending, the
 * block of t among them, -1 for unused places) for every video row; an entry
 * after the block of t holds no key u <= t and contributes nothing.
 * workspace: device scratch of nsa_sparse_attn_workspace_size() bytes (may
 * be NULL when that size is 0).
 */
size_t nsa_sparse_attn_workspace_size(const nsa_shape* shape, const nsa_params* params, int32_t dtype);
int32_t nsa_sparse_attn_fwd(const void* q, const void* k, const void* v, int32_t dtype, const nsa_shape* shape,
                            const nsa_params* params, const int32_t* block_idx, const uint8_t* is_video,
                            const void* o_cmp, const float* gates, void* out, void* o_slc, void* o_swa,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * nsa_hybrid_layer_fwd -- the whole layer: compression (unless k_cmp_in and
 * v_cmp_in give a precomputed compressed cache), compression-branch attention
 * with block importance, top-n selection, selection and window branches, the
 * gated combine for video rows, dense causal attention for text rows.
 * Prefill: q_start = 0, q_len = kv_len.  Decode: q_len = 1,
 * q_start = kv_len - 1 with the compressed cache passed in.
 * out is required; o_cmp / o_slc / o_swa / block_idx_out may be NULL (when
 * given they receive the branch outputs and the chosen blocks of the video
 * rows).  workspace: device scratch; the size depends on the kernels the call
 * dispatches to, so query it after any nsa_set_force_generic change.
 * Row chunks: a prefill on the MFMA path (bf16, head_dim 128, cmp_block 32 /
 * stride 16, and sel_block 64 with 4..8 query heads per KV head or sel_block
 * 32 or 128 with 4..7) may run as passes over chunks of query rows.  Every stage except the compression of K / V is
 * independent across rows, so the results are bit-identical to one pass; each
 * batch element's K / V are compressed once.  The call takes the largest chunk
 * (all rows, else a multiple of 64) whose scratch fits workspace_bytes, and
 * fails with NSA_ERR_WORKSPACE_TOO_SMALL when not even 64 rows fit (any
 * other dispatch needs the one-pass size).
 * nsa_hybrid_layer_workspace_size_rows: the scratch when at most
 * rows_per_chunk query rows run in one pass (0: all rows; < 0: returns 0).
 * nsa_hybrid_layer_workspace_size: the size for the default chunk: all rows
 * when their scratch stays within 7 GiB, else the largest chunk that does,
 * rounded down to a multiple of 16384 rows when it is at least that long.
 * Both return 0 for invalid arguments.
 */
size_t nsa_hybrid_layer_workspace_size(const nsa_shape* shape, const nsa_params* params, int32_t dtype);
size_t nsa_hybrid_layer_workspace_size_rows(const nsa_shape* shape, const nsa_params* params, int32_t dtype,
                                            int64_t rows_per_chunk);
int32_t nsa_hybrid_layer_fwd(const void* q, const void* k, const void* v, const void* k_cmp_in,
                             const void* v_cmp_in, const float* w_k, const float* w_v, const float* gates,
                             const uint8_t* is_video, int32_t dtype, const nsa_shape* shape,
                             const nsa_params* params, void* out, void* o_cmp, void* o_slc, void* o_swa,
                             int32_t* block_idx_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode over a batch of sequences of different lengths, with an optional
 * paged K / V cache.  The same layer as nsa_hybrid_layer_fwd ([A] abstract,
 * [B] section 一, [C] sections 2.2 and 3.1), one query row per sequence:
 * sequence b holds L_b tokens and its query sits at position t = L_b - 1;
 * every definition above applies with kv_len replaced by L_b (C(t), the
 * candidate blocks 0 .. t / sel_block, the window, the dense text rows).
 *  shape      q_len = 1; kv_len = the per-sequence capacity Lmax (q_start is
 *             ignored); k_cmp / v_cmp hold Nc(Lmax) blocks per sequence.
 *  kv_lens    device int32 [B]: L_b (clamped to [1, kv_len]); NULL means
 *             every sequence holds kv_len tokens.
 *  page_table device int32 [B, max_pages] or NULL.  NULL: k, v are
 *             [B, kv_len, Hkv, D].  Otherwise k, v are a page pool
 *             [num_pages, 64, Hkv, D]; token u of sequence b is row u % 64 of
 *             page page_table[b, u / 64] (ids clamped into [0, num_pages)).
 *             max_pages * 64 must cover kv_len.
 *  k_cmp, v_cmp [B, Nc(kv_len), Hkv, D]: blocks i < Nc(L_b) must be current
 *             (nsa_compress_kv, or nsa_compress_append after each step).
 *  q, gates, out, o_* are [B, 1, Hq, ...]; is_video [B] (NULL: all video);
 *  block_idx_out [B, 1, Hkv, top_n] or NULL.  lse and importance are not
 *  produced.  Covers bf16, head_dim 128, cmp_block 32, cmp_stride 16,
 *  sel_block 64, 4..8 query heads per KV head, kv_len >= 32; anything else is
 *  NSA_ERR_UNSUPPORTED.  workspace: nsa_decode_workspace_size() bytes.
 */
size_t nsa_decode_workspace_size(const nsa_shape* shape, const nsa_params* params, int32_t dtype);
int32_t nsa_decode_fwd(const void* q, const void* k, const void* v, const void* k_cmp, const void* v_cmp,
                       const float* gates, const uint8_t* is_video, int32_t dtype, const nsa_shape* shape,
                       const nsa_params* params, const int32_t* kv_lens, const int32_t* page_table,
                       int32_t max_pages, int64_t num_pages, void* out, void* o_cmp, void* o_slc, void* o_swa,
                       int32_t* block_idx_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * nsa_decode_fwd_noalloc -- nsa_decode_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments, outputs and kernels, without the
 * workspace arguments.  Its scratch is a device array inside the library, 64
 * MiB per GPU, held from the library's first use on that GPU until the process
 * ends; the call allocates nothing.  A batch whose workspace
 * (nsa_decode_workspace_size) exceeds that array is rejected with
 * NSA_ERR_WORKSPACE_TOO_SMALL before any launch (16 sequences of 64K tokens
 * need about 11 MB).  Every call on a GPU uses the same array: calls that
 * overlap in time on one GPU (concurrent streams or threads) race and must be
 * ordered by the caller.
 */
int32_t nsa_decode_fwd_noalloc(const void* q, const void* k, const void* v, const void* k_cmp, const void* v_cmp,
                               const float* gates, const uint8_t* is_video, int32_t dtype, const nsa_shape* shape,
                               const nsa_params* params, const int32_t* kv_lens, const int32_t* page_table,
                               int32_t max_pages, int64_t num_pages, void* out, void* o_cmp, void* o_slc,
                               void* o_swa, int32_t* block_idx_out, void* stream);

/*
 * nsa_compress_append -- incremental update of a compressed cache ([B]
 * section 一, [C] section 2.2; the weighted block sum of nsa_compress_kv).
 * After n_new tokens were appended to every sequence (kv_lens[b] = L_b
 * counts them; NULL means kv_len), writes every compressed block i whose last
 * token i*cmp_stride + cmp_block - 1 lies in [L_b - n_new, L_b - 1], with the
 * same fp32 sums and rounding as nsa_compress_kv, so the cache equals a full
 * recompression of the first L_b tokens.  Other blocks are left untouched.
 * k, v, kv_lens, page_table, max_pages, num_pages are as for nsa_decode_fwd;
 * k_cmp, v_cmp are [B, Nc(kv_len), Hkv, D].  n_new = 0 launches nothing.
 * Covers bf16 with head_dim 128 (else NSA_ERR_UNSUPPORTED).
 */
int32_t nsa_compress_append(const void* k, const void* v, int32_t dtype, int64_t batch, int64_t kv_len,
                            int32_t num_kv_heads, int32_t head_dim, const float* w_k, const float* w_v,
                            int32_t cmp_block, int32_t cmp_stride, const int32_t* kv_lens, const int32_t* page_table,
                            int32_t max_pages, int64_t num_pages, int32_t n_new, void* k_cmp, void* v_cmp,
                            void* stream);

/*
 * nsa_gate_proj -- the per-head branch gates from each token's hidden state,
 * computed in front of the layer ([B] section 一: a learned weighting mixes
 * the three branches per head; [C] section 3.1: three gate values per head
 * from the token's features).  Plain per-token reading, a linear map followed
 * by the logistic function:
 *   gates[b, t, h, c] = 1 / (1 + exp(-(b_g[f] + sum_k x[b, t, k] * w_g[f, k]))),
 *   f = 3 h + c, c = 0 (cmp), 1 (slc), 2 (swa)
 * x [B, seq_len, hidden] (dtype), w_g [3 * num_q_heads, hidden] (dtype, the
 * weight of a linear layer), b_g [3 * num_q_heads] fp32 or NULL (no bias),
 * gates [B, seq_len, num_q_heads, 3] fp32 -- the gates argument of the layer.
 * Products are accumulated in fp32.  Covers bf16 with hidden a multiple of 64
 * and num_q_heads <= 32 (else NSA_ERR_UNSUPPORTED).
 */
int32_t nsa_gate_proj(const void* x, const void* w_g, const float* b_g, int32_t dtype, int64_t batch,
                      int64_t seq_len, int32_t hidden, int32_t num_q_heads, float* gates, void* stream);

/*
 * nsa_hybrid_layer_fwd_branch_kv -- the same layer with independent keys and
 * values per branch, as in Native Sparse Attention, where each branch has its
 * own key/value projections ([B] section 一 names three separate branches;
 * [C] section 2.2).  k_c / v_c feed the compression (ignored when k_cmp_in /
 * v_cmp_in are given), k_s / v_s the selection branch, k_w / v_w the
 * sliding-window branch and the dense attention of text rows; the block
 * importance still comes from the compression branch.  All six are
 * [B, kv_len, Hkv, D]; they may alias each other (all equal gives
 * nsa_hybrid_layer_fwd).  Workspace as nsa_hybrid_layer_workspace_size().
 * One query row per sequence (decode shapes on the MFMA path) needs
 * k_s == k_w and v_s == v_w (else NSA_ERR_UNSUPPORTED).
 */
int32_t nsa_hybrid_layer_fwd_branch_kv(const void* q, const void* k_c, const void* v_c, const void* k_s,
                                       const void* v_s, const void* k_w, const void* v_w, const void* k_cmp_in,
                                       const void* v_cmp_in, const float* w_k, const float* w_v,
                                       const float* gates, const uint8_t* is_video, int32_t dtype,
                                       const nsa_shape* shape, const nsa_params* params, void* out, void* o_cmp,
                                       void* o_slc, void* o_swa, int32_t* block_idx_out, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * nsa_hybrid_layer_bwd -- backward pass of nsa_hybrid_layer_fwd: gradients of
 * the loss sum(d_out * out) ([B] section 一 and [C] sections 2.2 / 3.1 define
 * the forward; the selection is non-differentiable, so the chosen blocks are
 * an input and pass no gradient).  Per branch of a video row (and the single
 * dense branch of a text row, gate 1), with P the probabilities over the
 * branch's keys and E = sum_u P_u <d_out, v_u>:
 *   d_gates = E,  ds_u = gate P_u (<d_out, v_u> - E),  dq += scale sum ds_u k_u,
 *   dk_u += scale ds_u q,  dv_u += gate P_u d_out;
 * compressed keys / values pass their gradients back through the weighted block
 * sum: dk[i*d + m] += w_k[m] dk_cmp[i], dw_k[m] = sum_i <dk_cmp[i], k[i*d + m]>
 * (likewise v).  Compression is recomputed from k, v in fp32.
 *  q, d_out [B, q_len, Hq, D] (dtype); k, v [B, kv_len, Hkv, D] (dtype);
 *  w_k, w_v [cmp_block] fp32; gates [B, q_len, Hq, 3] fp32; is_video as for
 *  the forward; block_idx [B, q_len, Hkv, top_n] int32 (the forward's choice).
 *  Outputs, all fp32 and required: dq [B, q_len, Hq, D], dk, dv
 *  [B, kv_len, Hkv, D], d_gates [B, q_len, Hq, 3] (0 for text rows), dw_k,
 *  dw_v [cmp_block] (summed over the batch).  bf16 with head_dim 128, 1..8 heads
 *  per KV head, selection blocks of 32, 64 or 128 tokens and 16-byte aligned
 *  tensors: matrix-core kernels, whose atomic adds make the last bits of dk and
 *  dv depend on scheduling; otherwise generic kernels: head_dim a multiple
 *  of 64 up to 256 (else NSA_ERR_UNSUPPORTED), fp32 or bf16.  workspace:
 *  nsa_hybrid_layer_bwd_workspace_size() bytes (enough for either set).
 */
size_t nsa_hybrid_layer_bwd_workspace_size(const nsa_shape* shape, const nsa_params* params, int32_t dtype);
int32_t nsa_hybrid_layer_bwd(const void* q, const void* k, const void* v, const float* w_k, const float* w_v,
                             const float* gates, const uint8_t* is_video, const int32_t* block_idx,
                             const void* d_out, int32_t dtype, const nsa_shape* shape, const nsa_params* params,
                             float* dq, float* dk, float* dv, float* d_gates, float* dw_k, float* dw_v,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Debug / test switch: 1 forces the generic (non-MFMA) kernels, 0 restores the
 * default dispatch.  Returns the previous value.  Process-wide. */
int32_t nsa_set_force_generic(int32_t on);

/* Measurement aid.  nsa_profile_enable(1) makes every later
 * nsa_hybrid_layer_fwd record a HIP event on its stream at each phase
 * boundary (compress | compression branch + importance | top-n | window and
 * text rows | selection + combine); nsa_profile_read waits for the last event
 * of the most recent call and writes the phase durations in ms (returns their
 * count, or a negative status).  While it is on, the window pass runs in order
 * on the caller's stream (no second stream), so each phase is timed alone.
 * Process-wide, not for concurrent use. */
int32_t nsa_profile_enable(int32_t on);
int32_t nsa_profile_read(float* ms, int32_t max_phases);

#ifdef __cplusplus
}
#endif
#endif /* NSA_H */
