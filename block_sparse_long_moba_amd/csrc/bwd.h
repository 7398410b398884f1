// Internal declarations of the backward-pass kernels (bf16, d = 128).
#pragma once

#include "moba_internal.h"

namespace moba {

constexpr size_t kBwdZeroBytes = 256;  // zero area of a backward workspace
constexpr int kKvKeys = 256;            // keys per dK/dV workgroup (8 waves x 32)

// Splitting of large bins in the dK/dV stage: a bin of r rows is processed in
// ceil(r / seg_rows) segments (own-block rows with the first), each by its own
// workgroups; a split bin's segments write fp32 partials that a second kernel
// sums in segment order. seg_rows (a multiple of 32) defaults to 262144 and
// can be set with the environment variable MOBA_DKDV_SEGMENT_ROWS.
struct DkdvSplit {
  int64_t seg_rows;     // rows per segment
  int64_t extra_bound;  // bound on the segments beyond the first, over all bins
  int64_t nch;          // key chunks of a block
};
DkdvSplit dkdv_split(int64_t T, int Hp, int k, int B);

// Regions of a backward workspace after D, from `base` on.
struct BwdExtra {
  size_t zeros, ext_off, slot_off, part, end;
};
BwdExtra bwd_extra(size_t base, int64_t nbins, const DkdvSplit &sp);

// Extra buffers of the backward pass, next to the forward-pass Work of the
// same plan (its vt region is unused).
struct BwdWork {
  float *dq_part;  // [T*Hp*k][d] fp32 partial dQ of each (row, head, slot), scale applied
  float *delta;    // [Hq][T] D = <dO, O> of each (row, head)
  void *zeros;     // 256 bytes, zeroed by launch_bwd_dkdv
  uint32_t *ext_off;   // [nbins + 1] prefix of the segments beyond the first per bin
  uint32_t *slot_off;  // [nbins + 1] prefix of the partial slots (split bins only)
  float *part;         // [2 extra_bound][nch][256 keys][d] dK (scaled), then as much dV
};

struct BwdIo {
  const void *q, *k, *v, *dout;
  const float *lse;  // [Hq][T], natural log
  void *dq, *dk, *dv;
};

hipError_t launch_bwd_delta(const Problem &pb, const void *out, const void *dout, float *delta,
                            hipStream_t s);
// which: 1 = own-block rows, 2 = earlier-block rows, 3 = both
hipError_t launch_bwd_dq(const Problem &pb, const Work &w, const BwdWork &bw, const BwdIo &io,
                         int g0, int which, hipStream_t s);
hipError_t launch_bwd_dq_sum(const Problem &pb, const Work &w, const BwdWork &bw,
                             const BwdIo &io, int g0, hipStream_t s);
hipError_t launch_bwd_dkdv(const Problem &pb, const Work &w, const BwdWork &bw, const BwdIo &io,
                           int g0, hipStream_t s);

}  // namespace moba
