// Forward dispatch, bf16/f16 MFMA path: the kernel is fa_fwd_kernel.h, its
// instances live in one translation unit per (dtype, head_dim).
#include "fa_launch.h"

namespace fa {

hipError_t launch_fwd_mfma(const Params &p, int dtype, hipStream_t s) {
  if (dtype == FA_BF16) {
    if (p.D == 64) return launch_fwd_bf16_d64(p, s);
    if (p.D == 128) return launch_fwd_bf16_d128(p, s);
  } else if (dtype == FA_F16) {
    if (p.D == 64) return launch_fwd_f16_d64(p, s);
    if (p.D == 128) return launch_fwd_f16_d128(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
