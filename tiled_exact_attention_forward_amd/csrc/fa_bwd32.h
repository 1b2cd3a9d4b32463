// fa_bwd32.h -- the float32 backward (fa_bwd32.hip), called by the C ABI for FA_F32 inputs.
#pragma once
#include "fa_launch.h"

namespace teaf {

// dQ, dK, dV of the float32 forward; same arguments, workspace layout and kernel order as
// launch_backward (a.dtype is FA_F32, a.d 64 or 128, a.mask 0..4 or the block-sparse id).
hipError_t launch_backward32(const BwdArgs &a, hipStream_t stream);

}  // namespace teaf
