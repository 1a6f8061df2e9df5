// FP8 e4m3 attention forward (gfx950): not implemented yet.
#include "fa_launch.hpp"

namespace fa {

hipError_t launch_fwd_fp8(const FwdParams&, int, bool, hipStream_t) { return hipErrorNotSupported; }

}  // namespace fa
