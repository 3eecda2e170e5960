// kla_residual.h -- the residual-write forward (internal to the library).
#pragma once

#include "kla_internal.h"

namespace kla {

// Residual-write forward for dk == dv in {16, 32, 64, 128}, T >= 1.  The
// state passes as FwdArgs::eta0 / etaT, holding the posterior mean m (not
// the information l*m); l0 / lT are the precision as in the KLA forward.
bool fwd_residual_supported(int dk, int dv);
// Value tiles per (b,h) (1 or 2; 2 only for dk 64 / 128); FwdArgs::n_vtiles.
int fwd_residual_vtiles(int B, int H, int dk);
hipError_t launch_fwd_residual(const FwdArgs& a, int dtype, int cov, hipStream_t s);

// The chunked matrix-core forward (diagonal or isotropic, dk == dv in
// {64, 128}); its own value tiles of 64 columns (FwdArgs::n_vtiles is
// ignored).  KLA_RES_IMPL=block sends these shapes to the block kernel instead.
bool fwd_residual_chunk_supported(int dk, int dv, int cov, int dtype);
hipError_t launch_fwd_residual_chunk(const FwdArgs& a, int dtype, int cov, hipStream_t s);

}  // namespace kla
