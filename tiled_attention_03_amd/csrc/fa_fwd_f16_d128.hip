// Forward kernel instances for f16 inputs, head_dim 128 (one translation
// unit per (dtype, head_dim) so that the instances compile in parallel).
#include "fa_fwd_kernel.h"

namespace fa {
hipError_t launch_fwd_f16_d128(const Params &p, hipStream_t s) { return launch_d<_Float16, 128>(p, s); }
}  // namespace fa
