// Internal declarations of the backward-pass kernels (bf16, d = 128).
#pragma once

#include "moba_internal.h"

namespace moba {

constexpr size_t kBwdZeroBytes = 256;  // zero area at the end of a backward workspace

// Extra buffers of the backward pass, next to the forward-pass Work of the
// same plan (its vt region is unused).
struct BwdWork {
  float *dq_part;  // [T*Hp*k][d] fp32 partial dQ of each (row, head, slot), scale applied
  float *delta;    // [Hq][T] D = <dO, O> of each (row, head)
  void *zeros;     // 256 bytes, zeroed by launch_bwd_dkdv
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
