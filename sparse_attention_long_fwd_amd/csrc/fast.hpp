// MFMA (bf16, gfx950) kernels of the hybrid layer: declarations.
#pragma once
#include "common.hpp"

// True when the MFMA kernels cover this problem: bf16, head_dim 128, compressed block 32 /
// stride 16, selection block 64 with 4 <= G <= 8, or selection block 32 or 128 with 4 <= G <= 7.
bool fast_supported(int32_t dtype, const Dims& dm);

// Scratch bytes the MFMA selection/window path needs.
size_t fast_sparse_workspace(const Dims& dm);

// Compression branch + importance.  kh/vh: compressed keys/values (bf16, row-major).  When they
// come from an fp32 sum: kl8/ksc the fp8 low parts and scales of the keys (launch_compress_k8),
// vl the bf16 low parts of the values.  o (bf16) and o32 (fp32) are optional copies of the branch
// output; imp (optional) the block importance.
hipError_t launch_cmp_fast(const Dims& dm, const void* q, const void* kh, const void* kl8, const void* ksc,
                           const void* vh, const void* vl, const uint8_t* vid, void* o, float* o32, float* lse,
                           float* imp, hipStream_t s);

// Compressed keys split for launch_cmp_fast: bf16 high parts [B, Nc, Hkv, 128] in hi,
// fp8 low parts (k8_lo_bytes) in lo8, their scales (k8_sc_bytes) in sc.
size_t k8_lo_bytes(const Dims& dm);
size_t k8_sc_bytes(const Dims& dm);
hipError_t launch_compress_k8(const Dims& dm, const void* k, const float* w_k, void* hi, void* lo8, void* sc,
                              hipStream_t s);

// Compression branch + importance on the group kernel (one wave per 16 rows x all 4..7 query heads
// of a KV head), for keys and values compressed from the raw k / v: launch_compress_kv16 writes them
// as fp16 key and value tiles with power-of-two range scales (kv16_tiles_bytes(dm) bytes), which
// launch_cmp_group reads.  lse (required) receives the log-sum-exp of the video rows.
bool cmp_group_supported(const Dims& dm);
size_t kv16_tiles_bytes(const Dims& dm);
hipError_t launch_compress_kv16(const Dims& dm, const void* k, const float* w_k, const void* v, const float* w_v,
                                void* out, hipStream_t s);
hipError_t launch_cmp_group(const Dims& dm, const void* q, const void* kv16, const uint8_t* vid, void* o_bf,
                            float* o32, float* lse, float* imp, hipStream_t s);

// Window branch, text rows, selection branch and the gated combine of the compression output
// o_cmp (fp32 when ocmp_f32, else bf16), the selection output and the window output (bf16, in
// o_swa or the workspace).  ws: fast_sparse_workspace(dm) bytes.  ks / vs: keys and values
// of the selection branch; kw / vw: of the window branch and text rows.  forced_local: idx comes
// from the layer's own top-n, so each video row's last min(n_local, jt + 1) entries are its forced
// local blocks jt - n_local + 1 .. jt (the window pass may then take them over).
// concurrent: the window pass runs on the calling thread's side stream (side_stream) beside the
// selection kernels; otherwise the two passes run in order on s (mark is called between them).
hipError_t launch_sparse_fast(const Dims& dm, const void* q, const void* ks, const void* vs, const void* kw,
                              const void* vw, const int32_t* idx,
                              const uint8_t* vid, const void* o_cmp, bool ocmp_f32, const float* gates, void* out,
                              void* o_slc, void* o_swa, void* ws, hipStream_t s,
                              void (*mark)(hipStream_t) = nullptr, bool forced_local = false,
                              bool concurrent = false);

// The calling thread's second stream on the current device (non-blocking, default priority) and a
// fork / join event pair.  The window pass (window branch, dense text rows, the forced local
// selection partials) reads only q, k, v and the row flags, so it can run there beside the top-n
// and the selection kernels; only the selection merge reads its outputs.  Created on the first
// call outside stream capture and kept until the process ends; null when that fails, the first
// call comes during a capture, or the caller's stream belongs to another device than the current
// one (the passes then run in order on the caller's stream).
struct SideStream {
  hipStream_t s;
  hipEvent_t fork, join;
};
SideStream* side_stream(hipStream_t caller);
// The two passes of launch_sparse_fast.  With side, the window pass runs on side->s once the
// caller's stream reaches the launch (side->fork) and records side->join when done; the selection
// pass's merge waits for side->join on the caller's stream.  Both passes take the same side (or
// null), the same workspace and the same o_swa: the window output of the video rows in bf16 goes
// there when given, else to the workspace, and the combine reads it back.
hipError_t launch_sparse_window(const Dims& dm, const void* q, const void* ks, const void* vs, const void* kw,
                                const void* vw, const uint8_t* vid, void* out, void* o_swa, void* ws, hipStream_t s,
                                const SideStream* side, bool forced_local);
// Make s wait for the window pass forked onto side (no-op for a null side); every error return after
// a fork calls it, so no work of the call is left running unordered beside the caller's stream.
hipError_t join_side_stream(const SideStream* side, hipStream_t s);
hipError_t launch_sparse_select(const Dims& dm, const void* q, const void* ks, const void* vs, const void* kw,
                                const void* vw, const int32_t* idx, const uint8_t* vid, const void* o_cmp,
                                bool ocmp_f32, const float* gates, void* out, void* o_slc, const void* o_swa,
                                void* ws, hipStream_t s, const SideStream* side, bool forced_local);

// The kept (row, slot) pairs of the video rows bucketed by chosen block (every pair whose block holds a
// key at or before its row): chunk c of (batch, group) bg covers block chunk_blk[bg * cap_c + c]
// (-1: unused) and its 32 pairs pairs[(bg * cap_c + c) * 32 + i] = (row << 5) | slot (-1 past the
// list's end); a block's chunks are consecutive from cfirst[bg * Ns + j].  The arrays sit at the
// start of ws (slc_bucket_bytes(dm) bytes).
struct SlcPairLists {
  const int* chunk_blk;
  const int* pairs;
  const int* cfirst;  // [bg][Ns]: the first chunk of each block's list
  int cap_c;
};
size_t slc_bucket_bytes(const Dims& dm);
hipError_t launch_slc_pair_lists(const Dims& dm, const int32_t* idx, const uint8_t* vid, void* ws, SlcPairLists* pl,
                                 hipStream_t s);

// Window / text-row flash kernel: swa_bf the bf16 window output of the video rows (may be NULL),
// text: output of text rows (NULL: skip them); ws: flash_workspace(dm).
// local_ml / local_o (both or neither): the selection partial arrays of the selection kernels;
// when given, the window pass also forms each video row's selection partial over its forced local
// blocks (local_fusable(dm) must hold) and stores it in the row's first local slot (the others
// are marked empty).
hipError_t launch_flash_fast(const Dims& dm, const void* q, const void* k, const void* v, const uint8_t* vid,
                             void* swa_bf, void* text, void* ws, hipStream_t s,
                             void* local_ml = nullptr, void* local_o = nullptr);
// The forced local blocks of every video row lie inside its window and the query tiles of 32 rows
// never straddle a 64-token block.
bool local_fusable(const Dims& dm);
size_t flash_workspace(const Dims& dm);

// Gate values g = sigmoid(x w^T + b): x [R, K] bf16, w [N, K] bf16, b [N] fp32 or null, g [R, N] fp32.
bool gate_proj_supported(int64_t K, int N);
hipError_t launch_gate_proj(const void* x, const void* w, const float* bias, float* g, int64_t R, int64_t K, int N,
                            hipStream_t s);

// Decode path (one query row per sequence, split over the compressed keys).
// Variable-length batches: lens[b] tokens in sequence b (the query at lens[b] - 1), dm.T the
// capacity; pages (optional) maps 64-token page i of sequence b to pool page pages[b * max_pages
// + i] of a [num_pages, 64, Hkv, D] cache.  All null: every sequence holds dm.T tokens of a
// contiguous [B, T, Hkv, D] cache, the query at dm.q0.
// Rows of one page of a paged K / V cache ([num_pages, kPageRows, Hkv, D]): one selection block.
constexpr int kPageRows = 64;
struct DecVar {
  const int32_t* lens = nullptr;
  const int32_t* pages = nullptr;
  int max_pages = 0;
  int64_t num_pages = 0;
};
bool decode_supported(const Dims& dm);
size_t decode_workspace(const Dims& dm);
hipError_t launch_decode_fast(const Dims& dm, const DecVar& dv, const void* q, const void* kh, const void* kl,
                              const void* vh, const void* vl, const void* k, const void* v, const uint8_t* vid,
                              const float* gates, void* out, void* o_cmp, void* o_slc, void* o_swa, int32_t* idx,
                              float* lse, float* imp, void* ws, hipStream_t s, void (*mark)(hipStream_t));
// Compressed cache update after n_new tokens were appended to every sequence: the blocks whose
// last token is among them (per sequence), from the (possibly paged) K / V cache.
hipError_t launch_compress_append(const Dims& dm, const DecVar& dv, const void* k, const void* v, const float* w_k,
                                  const float* w_v, void* kc, void* vc, int n_new, hipStream_t s);

// Scratch of nsa_decode_fwd_noalloc: the current device's copy of a file-scope device array
// (address from hipGetSymbolAddress, kept per device) and its size.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);
size_t noalloc_scratch_bytes();
