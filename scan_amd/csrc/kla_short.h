// kla_short.h -- the short-sequence forward (internal to the library).
#pragma once

#include "kla_internal.h"

namespace kla {

// Short sequences (1 <= T <= kShortTMax, dk == dv in {16, 32, 64, 128}): each
// (b,h) keeps its state in registers for the whole sequence and crosses HBM
// once each way (prefill into cached states, multi-token decode).  Small
// heads share a workgroup.
constexpr int kShortTMax = 32;
bool fwd_short_supported(int dk, int dv, int T);
hipError_t launch_fwd_short(const FwdArgs& a, int dtype, int cov, hipStream_t s);

}  // namespace kla
