// ssm_prefill.hip -- launch planning for prefill and decode: the choice of prefill
// decomposition, and the split of a call into launches over batch rows.
#include "ssm_internal.h"

namespace ssm {

hipError_t launch_sequential(const ScanArgs& a, hipStream_t s);
hipError_t launch_windowed(const ScanArgs& a, hipStream_t s);
hipError_t launch_decode_rows(const ScanArgs& a, hipStream_t s);
bool windowed_supported(const ScanArgs& a);

// The windowed scan spreads each channel over a whole wave, so it fills the GPU even for one
// batch row of a 2048-channel slice; it needs d_state == 16.  Everything else runs one lane per
// channel.  The choice depends on d_state and chunk_hint only, never on the batch or channel
// count, so a channel slice run alone reproduces the full run bit for bit.
int choose_prefill_variant(const ScanArgs& a) {
  if (a.chunk_hint == kSequential) return kSequential;
  if (windowed_supported(a)) return kWindowed;
  return kSequential;
}

size_t prefill_workspace_bytes(const ScanArgs& a) {
  (void)a;
  return 0;
}

// A launch's work-items must stay below 2^32 per grid dimension.  The widest kernel here
// takes 64 work-items per channel (one wave) plus a ragged workgroup of at most 16 waves, so
// each launch covers at most kLaunchItems / (64 (D + 16)) batch rows; d_inner <= 2^24 keeps
// that at least one.
constexpr int64_t kLaunchItems = int64_t(1) << 31;

int64_t rows_per_launch(const ScanArgs& a) {
  const int64_t n = kLaunchItems / (64 * (a.D + 16));
  return n < 1 ? 1 : n;
}

// Batch rows [b0, b0 + nb) of a call as a call of their own.  Every per-row tensor moves to
// row b0; with a cache pool the cache is shared and only the slot and length maps move.
// Channels are never split, so every channel computes exactly as in one launch.
ScanArgs batch_rows(const ScanArgs& a, int64_t b0, int64_t nb) {
  ScanArgs r = a;
  const int64_t es = a.bf16 ? 2 : 4;
  const int64_t seq = b0 * a.D * a.L * es, bc = b0 * a.L * a.N * es;
  auto at = [](const void* p, int64_t bytes) -> const char* {
    return p ? static_cast<const char*>(p) + bytes : nullptr;
  };
  r.B = nb;
  r.x = at(a.x, seq);
  r.dt = at(a.dt, seq);
  r.z = at(a.z, seq);
  r.y = const_cast<char*>(at(a.y, seq));
  r.Bm = at(a.Bm, bc);
  r.Cm = at(a.Cm, bc);
  if (a.slots) {
    r.slots = a.slots + b0;
    if (a.seqlens) r.seqlens = a.seqlens + b0;
  } else {
    const int64_t hs = b0 * a.D * a.N * 4, cs = b0 * a.D * 3 * 4;
    r.h0 = reinterpret_cast<const float*>(at(a.h0, hs));
    r.h_out = reinterpret_cast<float*>(const_cast<char*>(at(a.h_out, hs)));
    r.conv0 = reinterpret_cast<const float*>(at(a.conv0, cs));
    r.conv_out = reinterpret_cast<float*>(const_cast<char*>(at(a.conv_out, cs)));
    if (a.seqlens) r.seqlens = a.seqlens + b0;
  }
  return r;
}

template <typename Launch>
hipError_t over_batch_rows(const ScanArgs& a, hipStream_t s, Launch launch) {
  const int64_t step = rows_per_launch(a);
  if (step >= a.B) return launch(a, s);
  for (int64_t b0 = 0; b0 < a.B; b0 += step) {
    const hipError_t e = launch(batch_rows(a, b0, a.B - b0 < step ? a.B - b0 : step), s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_prefill(const ScanArgs& a, void* workspace, hipStream_t s) {
  (void)workspace;
  const bool windowed = choose_prefill_variant(a) == kWindowed;
  return over_batch_rows(a, s, windowed ? launch_windowed : launch_sequential);
}

hipError_t launch_decode(const ScanArgs& a, hipStream_t s) { return over_batch_rows(a, s, launch_decode_rows); }

}  // namespace ssm
