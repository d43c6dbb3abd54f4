// Dispatch of the MFMA path: coverage test, workspace sizes, launch order.
#include "fast_common.hpp"

size_t slc_block_workspace(const Dims& dm);
void slc_partial_arrays(const Dims& dm, void* ws, void** ml, void** o);
hipError_t launch_slc_block(const Dims& dm, const void* q, const void* k, const void* v, const int32_t* idx,
                            const uint8_t* vid, const void* ocmp, bool ocmp_f32, const void* swa,
                            const float* gates, void* out, void* o_slc, void* ws, hipStream_t s,
                            bool local_fused, hipEvent_t before_merge);

// Block-major selection packs (row, slot) into 32 bits: rows below 2^26.  Selection blocks of 64
// tokens for 4..8 query heads per KV head; of 32 or 128 tokens for 4..7 (the group kernel of the
// compression branch).
bool fast_supported(int32_t dtype, const Dims& dm) {
  const bool ls_ok = dm.ls == 64 || ((dm.ls == 32 || dm.ls == 128) && dm.G <= 7);
  return dtype == 1 && dm.D == 128 && dm.l == 32 && dm.d == 16 && ls_ok && dm.G >= 4 && dm.G <= 8 &&
         dm.n <= 32 && dm.Tq < ((int64_t)1 << 26);
}

static size_t rup(size_t x) { return (x + 255) & ~(size_t)255; }

// [window output of the video rows, bf16 (the caller's o_swa instead when given)][split partials of
// long text rows][block-major selection]
static size_t swa_bytes(const Dims& dm) { return rup((size_t)dm.B * dm.Tq * dm.Hq * dm.D * 2); }

size_t fast_sparse_workspace(const Dims& dm) {
  return swa_bytes(dm) + rup(flash_workspace(dm)) + rup(slc_block_workspace(dm));
}

// The window pass takes over the forced local blocks of the selection (they lie inside the window
// and are scored there anyway) when the layer chose the blocks and the keys are shared.
static bool fuse_local(const Dims& dm, const void* ks, const void* vs, const void* kw, const void* vw,
                       bool forced_local) {
  return forced_local && ks == kw && vs == vw && local_fusable(dm);
}

SideStream* side_stream(hipStream_t caller) {
  struct Slot {
    SideStream ss{};
    bool tried = false, ok = false;
  };
  constexpr int kMaxDev = 64;
  thread_local Slot tab[kMaxDev];
  // only for a stream of the current device (the side stream is created there)
  int dev = 0;
  hipDevice_t sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  if (hipStreamGetDevice(caller, &sdev) != hipSuccess || sdev != dev) return nullptr;
  Slot& sl = tab[dev];
  if (!sl.tried) {
    // no stream or event creation while the caller's stream is being captured
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    sl.tried = true;
    sl.ok = hipStreamCreateWithFlags(&sl.ss.s, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&sl.ss.fork, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&sl.ss.join, hipEventDisableTiming) == hipSuccess;
  }
  return sl.ok ? &sl.ss : nullptr;
}

hipError_t launch_sparse_window(const Dims& dm, const void* q, const void* ks, const void* vs, const void* kw,
                                const void* vw, const uint8_t* vid, void* out, void* o_swa, void* ws, hipStream_t s,
                                const SideStream* side, bool forced_local) {
  void* swa = o_swa ? o_swa : ws;
  char* fws = (char*)ws + swa_bytes(dm);
  char* sws = fws + rup(flash_workspace(dm));
  void *lml = nullptr, *lo = nullptr;
  if (fuse_local(dm, ks, vs, kw, vw, forced_local)) slc_partial_arrays(dm, sws, &lml, &lo);
  hipStream_t sw = s;
  if (side) {
    hipError_t e = hipEventRecord(side->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
    if (e != hipSuccess) return e;
    sw = side->s;
  }
  // window branch (bf16, read by the combine) and dense text rows; the join event
  // is recorded even when the launch failed, so that the caller can always rejoin the side stream
  hipError_t e = launch_flash_fast(dm, q, kw, vw, vid, swa, out, fws, sw, lml, lo);
  if (side) {
    const hipError_t ej = hipEventRecord(side->join, sw);
    if (e == hipSuccess) e = ej;
  }
  return e;
}

hipError_t join_side_stream(const SideStream* side, hipStream_t s) {
  return side ? hipStreamWaitEvent(s, side->join, 0) : hipSuccess;
}

hipError_t launch_sparse_select(const Dims& dm, const void* q, const void* ks, const void* vs, const void* kw,
                                const void* vw, const int32_t* idx, const uint8_t* vid, const void* o_cmp,
                                bool ocmp_f32, const float* gates, void* out, void* o_slc, const void* o_swa,
                                void* ws, hipStream_t s, const SideStream* side, bool forced_local) {
  const void* swa = o_swa ? o_swa : ws;
  char* sws = (char*)ws + swa_bytes(dm) + rup(flash_workspace(dm));
  // selection branch and the gated combine of video rows
  return launch_slc_block(dm, q, ks, vs, idx, vid, o_cmp, ocmp_f32, swa, gates, out, o_slc, sws, s,
                          fuse_local(dm, ks, vs, kw, vw, forced_local), side ? side->join : nullptr);
}

hipError_t launch_sparse_fast(const Dims& dm, const void* q, const void* ks, const void* vs, const void* kw,
                              const void* vw, const int32_t* idx,
                              const uint8_t* vid, const void* o_cmp, bool ocmp_f32, const float* gates, void* out,
                              void* o_slc, void* o_swa, void* ws, hipStream_t s, void (*mark)(hipStream_t),
                              bool forced_local, bool concurrent) {
  const SideStream* side = concurrent ? side_stream(s) : nullptr;
  hipError_t e = launch_sparse_window(dm, q, ks, vs, kw, vw, vid, out, o_swa, ws, s, side, forced_local);
  if (e == hipSuccess) {
    if (mark && !side) mark(s);
    e = launch_sparse_select(dm, q, ks, vs, kw, vw, idx, vid, o_cmp, ocmp_f32, gates, out, o_slc, o_swa, ws, s,
                             side, forced_local);
  }
  // on failure the caller's stream still waits for the window pass (a no-op once the merge did)
  if (e != hipSuccess) (void)join_side_stream(side, s);
  return e;
}
