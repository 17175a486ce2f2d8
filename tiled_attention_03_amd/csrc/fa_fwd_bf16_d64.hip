// Forward kernel instances for bf16 inputs, head_dim 64 (one translation
// unit per (dtype, head_dim) so that the instances compile in parallel).
#include "fa_fwd_kernel.h"

namespace fa {
hipError_t launch_fwd_bf16_d64(const Params &p, hipStream_t s) { return launch_d<__bf16, 64>(p, s); }
}  // namespace fa
