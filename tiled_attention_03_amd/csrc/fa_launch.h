// Host-side launchers of the libfa kernels.  Each returns the result of
// hipGetLastError() after its launches; the caller has validated the
// problem (sizes, pointers, supported head_dim) beforehand.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_common.h"

namespace fa {

// Run-time switches read from the environment at each call (host side only):
//   FA_LOG=1   every call prints the kernel instance it launches and its grid
//              on stderr (one line per launch);
//   FA_TILE=   workgroup shape, for sweeps: "auto" (default: the short-query
//              forward and backward where they apply, else one-wave forward
//              workgroups for S_q <= 32 and four-wave ones otherwise),
//              "short" (the same as auto), "wg4" (four-wave forward
//              workgroups for every S_q, and the key and query passes for
//              every backward), "wg1" (one-wave list-based forward
//              workgroups for every S_q whose key range fits their lists,
//              and the key and query passes for every backward).
// Unknown FA_TILE values count as "auto".  The choice never changes results
// beyond rounding order.
enum { kTileAuto = 0, kTileWg4 = 1, kTileWg1 = 2, kTileShort = 3 };
bool log_enabled();
int tile_override();
void log_launch(const char *what, const char *instance, long long grid, int block,
                const Params &p);

// Forward, bf16/f16 MFMA path (D = 64 or 128), and its per-(dtype, D) instances.
hipError_t launch_fwd_mfma(const Params &p, int dtype, hipStream_t s);
hipError_t launch_fwd_bf16_d64(const Params &p, hipStream_t s);
hipError_t launch_fwd_bf16_d128(const Params &p, hipStream_t s);
hipError_t launch_fwd_f16_d64(const Params &p, hipStream_t s);
hipError_t launch_fwd_f16_d128(const Params &p, hipStream_t s);
// Forward, fp8 (OCP e4m3) inputs, D = 64 or 128: a pre-pass writes the
// permuted V^T tiles into p.vt, then the MFMA kernel; O is bf16.
hipError_t launch_fwd_fp8(const Params &p, hipStream_t s);
size_t fwd_fp8_workspace_bytes(const Params &p);
// Forward, fp32 path (D = 32, 64 or 128): fp32 FMA throughout.
hipError_t launch_fwd_f32(const Params &p, hipStream_t s);

// Backward step 1 (any dtype): delta_i = sum_d dO_id O_id.
hipError_t launch_bwd_prep(const Params &p, int dtype, hipStream_t s);
// Backward step 2: dK, dV (key-tile pass).  The producer/consumer form
// serves the problems bwd_kv_split_eligible accepts (causal rule with or
// without ALiBi, or no mask or bias; dropout allowed, no bias gradient);
// launch_bwd_kv_mfma picks it for them and the one-role pass otherwise.
hipError_t launch_bwd_kv_mfma(const Params &p, int dtype, hipStream_t s);
bool bwd_kv_split_eligible(const Params &p);
hipError_t launch_bwd_kv_split(const Params &p, int dtype, hipStream_t s);
hipError_t launch_bwd_kv_f32(const Params &p, hipStream_t s);
// Backward step 3: dQ (query-tile pass), written in dtype/layout.
hipError_t launch_bwd_q_mfma(const Params &p, int dtype, hipStream_t s);
// Zeroes n_words 32-bit words at dst (16-byte aligned): a fill kernel, not a
// memset node, so that it behaves inside captured graphs.
hipError_t launch_zero_words(void *dst, int64_t n_words, hipStream_t s);
hipError_t launch_bwd_q_f32(const Params &p, hipStream_t s);
// Backward for short query blocks (S_q <= 32, causal / padding masks, ALiBi
// or no bias, no dropout, gradients in the input dtype): dQ, dK and dV in one
// pass per (batch, head).  Selected by fa_bwd when bwd_short_fits() and
// FA_TILE is "auto" or "short"; the step entry points keep their own passes.
bool bwd_short_fits(const Params &p, int dtype);
hipError_t launch_bwd_short(const Params &p, int dtype, hipStream_t s);

// MaxSim late-interaction scores (see fa_maxsim in include/fa.h).
struct MaxSimParams {
  const void *q, *d;               // [B, Lq, D], [B, Ld, D]
  const uint8_t *q_valid, *d_valid;  // [B, Lq], [B, Ld] or null
  float *rowmax;                   // [B, Lq]
  float *score;                    // [B]
  int B, Lq, Ld, D;
};
constexpr int kMaxSimMaxDim = 1024;     // D: multiple of 128, at most this
constexpr int kMaxSimMaxDocs = 16384;   // L_d at most this
hipError_t launch_maxsim(const MaxSimParams &p, int dtype, hipStream_t s);

}  // namespace fa
