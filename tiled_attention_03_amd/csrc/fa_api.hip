// C ABI of libfa: argument validation, parameter block, dispatch.
// The contract of every entry point is documented in include/fa.h.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "fa_launch.h"

using namespace fa;

namespace fa {

// The switches are read at every call (getenv is cheap next to a launch), so
// a process may change them between calls.
bool log_enabled() {
  const char *lg = getenv("FA_LOG");
  return lg && *lg && strcmp(lg, "0") != 0;
}

int tile_override() {
  const char *tl = getenv("FA_TILE");
  if (tl && strcmp(tl, "wg4") == 0) return kTileWg4;
  if (tl && strcmp(tl, "wg1") == 0) return kTileWg1;
  if (tl && strcmp(tl, "short") == 0) return kTileShort;
  return kTileAuto;
}

void log_launch(const char *what, const char *instance, long long grid, int block,
                const Params &p) {
  static std::mutex mu;
  std::lock_guard<std::mutex> lk(mu);
  const char *masks[4] = {"causal", "explicit", "modality", "padding"};
  char mk[64] = "";
  for (int i = 0; i < 4; ++i)
    if (p.mask_flags & (1u << i)) {
      if (mk[0]) strcat(mk, "+");
      strcat(mk, masks[i]);
    }
  fprintf(stderr,
          "[libfa] %s: B=%d H=%d S_q=%d S_k=%d D=%d masks=%s pse=%s dropout=%d -> %s grid=%lld "
          "block=%d\n",
          what, p.B, p.H, p.Sq, p.Sk, p.D, mk[0] ? mk : "none",
          p.pse_kind == FA_PSE_ALIBI ? "alibi" : p.pse_kind == FA_PSE_DENSE ? "dense" : "none",
          p.dropout, instance, grid, block);
}

}  // namespace fa

namespace {

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

bool head_dim_supported(int dtype, int d) {
  if (dtype == FA_F32) return d == 32 || d == 64 || d == 128;
  return d == 64 || d == 128;
}

// True when the problem holds no work at all (B, H or S_q is zero).
bool empty_problem(const fa_problem *p) {
  return p->batch == 0 || p->head_num == 0 || p->seq_q == 0;
}

// Checks everything that does not involve tensor pointers.
fa_status check_problem(const fa_problem *p) {
  if (!p) return FA_ERR_INVALID_ARG;
  if (p->batch < 0 || p->head_num < 0 || p->seq_q < 0 || p->seq_k < 0 || p->head_dim <= 0)
    return FA_ERR_INVALID_ARG;
  if (p->layout != FA_BNSD && p->layout != FA_BSH) return FA_ERR_INVALID_ARG;
  if (p->dtype != FA_F32 && p->dtype != FA_F16 && p->dtype != FA_BF16 && p->dtype != FA_FP8_E4M3)
    return FA_ERR_INVALID_ARG;
  if (!isfinite(p->scale)) return FA_ERR_INVALID_ARG;
  // the kernels take a row's max over raw scores and then scale it, which
  // needs scale >= 0
  if (p->scale < 0.f) return FA_ERR_UNSUPPORTED;
  if (!(p->keep_prob > 0.f && p->keep_prob <= 1.f)) return FA_ERR_INVALID_ARG;   // NaN too
  if (p->keep_prob < 1.f && (p->dtype == FA_F32 || p->dtype == FA_FP8_E4M3))
    return FA_ERR_UNSUPPORTED;
  if (p->reserved0 != 0) return FA_ERR_INVALID_ARG;
  if (p->dpse) {
    if (p->pse_kind != FA_PSE_DENSE || !aligned16(p->dpse)) return FA_ERR_INVALID_ARG;
    if (p->dtype == FA_F32 || p->dtype == FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  }
  if (!head_dim_supported(p->dtype, p->head_dim)) return FA_ERR_UNSUPPORTED;
  const uint32_t known = FA_MASK_CAUSAL | FA_MASK_EXPLICIT | FA_MASK_MODALITY | FA_MASK_PADDING;
  if (p->mask_flags & ~known) return FA_ERR_INVALID_ARG;
  if (p->pse_kind != FA_PSE_NONE && p->pse_kind != FA_PSE_ALIBI && p->pse_kind != FA_PSE_DENSE)
    return FA_ERR_INVALID_ARG;
  // sizes whose indices must fit the kernels' 32-bit counters, each product
  // bounded before it enters the next, so none leaves 64-bit range: B·H and
  // H·D, then one (batch, head) span of Q/K-shaped tensors below 2 GiB (the
  // kernels address it with 32-bit byte offsets), then B·H·S_q rows
  const int64_t bh = (int64_t)p->batch * p->head_num;
  const int64_t hd = (int64_t)p->head_num * p->head_dim;
  if (bh > INT32_MAX || hd > INT32_MAX) return FA_ERR_UNSUPPORTED;
  {
    const int64_t es = p->dtype == FA_F32 ? 4 : 2;
    const int64_t rs = p->layout == FA_BSH ? hd : p->head_dim;
    const int64_t lim = ((int64_t)1 << 31) / es;   // elements
    if ((int64_t)p->seq_q * rs >= lim || (int64_t)p->seq_k * rs >= lim) return FA_ERR_UNSUPPORTED;
  }
  if (bh * p->seq_q > INT32_MAX) return FA_ERR_UNSUPPORTED;
  if (empty_problem(p)) return FA_OK;
  if (p->mask_flags & FA_MASK_EXPLICIT) {
    if (!p->explicit_mask) return FA_ERR_INVALID_ARG;
    if (p->em_stride_b < 0 || p->em_stride_h < 0 || p->em_stride_q < 0) return FA_ERR_INVALID_ARG;
  }
  if (p->mask_flags & FA_MASK_MODALITY) {
    if (!p->q_modality || !p->k_modality) return FA_ERR_INVALID_ARG;
    if (p->num_modalities < 1 || p->num_modalities > 8) return FA_ERR_INVALID_ARG;
  }
  if ((p->mask_flags & FA_MASK_PADDING) && !p->key_valid) return FA_ERR_INVALID_ARG;
  if (p->pse_kind == FA_PSE_ALIBI && !p->alibi_slopes) return FA_ERR_INVALID_ARG;
  if (p->pse_kind == FA_PSE_DENSE) {
    if (!p->pse) return FA_ERR_INVALID_ARG;
    if (p->pse_dtype != FA_F32 && p->pse_dtype != FA_F16 && p->pse_dtype != FA_BF16)
      return FA_ERR_INVALID_ARG;
    if (p->pse_stride_b < 0 || p->pse_stride_h < 0 || p->pse_stride_q < 0)
      return FA_ERR_INVALID_ARG;
  }
  return FA_OK;
}

// A tensor pointer that must be present (and 16-byte aligned for vector loads).
bool tensor_ok(const void *ptr) { return ptr != nullptr && aligned16(ptr); }
// K/V-shaped tensors may be absent when S_k == 0.
bool ktensor_ok(const fa_problem *p, const void *ptr) {
  return p->seq_k == 0 ? (ptr == nullptr || aligned16(ptr)) : tensor_ok(ptr);
}

Params make_params(const fa_problem *p) {
  Params r;
  memset(&r, 0, sizeof(r));
  const int64_t B = p->batch, H = p->head_num, Sq = p->seq_q, Sk = p->seq_k, D = p->head_dim;
  r.B = (int)B; r.H = (int)H; r.Sq = (int)Sq; r.Sk = (int)Sk; r.D = (int)D;
  if (p->layout == FA_BNSD) {
    r.q_sb = H * Sq * D; r.q_sh = Sq * D; r.q_ss = D;
    r.k_sb = H * Sk * D; r.k_sh = Sk * D; r.k_ss = D;
  } else {
    r.q_sb = Sq * H * D; r.q_sh = D; r.q_ss = H * D;
    r.k_sb = Sk * H * D; r.k_sh = D; r.k_ss = H * D;
  }
  r.scale = p->scale;
  r.scale_log2 = p->scale * kLog2e;
  r.mask_flags = p->mask_flags;
  r.em = p->explicit_mask;
  r.em_sb = p->em_stride_b; r.em_sh = p->em_stride_h; r.em_sq = p->em_stride_q;
  r.qmod = p->q_modality; r.kmod = p->k_modality;
  r.num_modalities = p->num_modalities;
  r.allow_diag = p->modality_allow_diag != 0;
  uint64_t bits = 0;
  if (p->mask_flags & FA_MASK_MODALITY) {
    const int M = p->num_modalities;
    for (int a = 0; a < M; ++a)
      for (int c = 0; c < M; ++c)
        if (p->modality_allow[a * M + c]) bits |= 1ull << (a * 8 + c);
  }
  r.allow_bits = bits;
  r.key_valid = p->key_valid;
  r.pse_kind = p->pse_kind;
  r.pse_dtype = p->pse_dtype;
  r.alibi_slopes = p->alibi_slopes;
  r.pse = p->pse;
  r.pse_sb = p->pse_stride_b; r.pse_sh = p->pse_stride_h; r.pse_sq = p->pse_stride_q;
  r.grad_f32 = p->grad_f32 != 0 && p->dtype != FA_F32;
  r.dpse = p->dpse;
  if (p->keep_prob < 1.f) {
    // keep iff word < floor(keep_prob * 2^32); keep_prob * 2^32 is exact in double
    r.dropout = 1;
    r.drop_thr = (uint32_t)floor((double)p->keep_prob * 4294967296.0);
    r.seed_lo = (uint32_t)(p->dropout_seed & 0xffffffffu);
    r.seed_hi = (uint32_t)(p->dropout_seed >> 32);
    r.inv_keep = 1.f / p->keep_prob;
  }
  return r;
}

size_t delta_bytes(const fa_problem *p) {
  return round256((size_t)p->batch * p->head_num * p->seq_q * sizeof(float));
}

fa_status hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

fa_status workspace_ok(const fa_problem *p, const void *ws, size_t bytes) {
  if (p->dtype == FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;   // no fp8 backward
  if (bytes < delta_bytes(p)) return FA_ERR_WORKSPACE;
  if (!tensor_ok(ws)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

void bind_workspace(Params &r, void *ws) { r.delta = (float *)ws; }

// ---- device scratch of the allocation-free backward (fa_bwd_noalloc): the
// row terms D_i live in this array instead of a caller workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  Host code
// never passes the array's name to a kernel or a copy (on the host it is a
// stand-in, not a device address): it uses the address hipGetSymbolAddress
// returns for the current device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void *scratch_ptr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

// The scratch array's device address on the current device.
fa_status current_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::call_once(scratch_once[dev], [dev] {
    void *ptr = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (scratch_err[dev] != hipSuccess || !scratch_ptr[dev]) return FA_ERR_HIP;
  *out = scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char *fa_status_str(fa_status s) {
  // a C caller may pass any int; read it as one (a load of an out-of-range
  // value as the enum type would be undefined in C++)
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_HIP: return "HIP error";
    case FA_ERR_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

fa_status fa_fwd(const fa_problem *p, const void *q, const void *k, const void *v, void *o,
                 float *lse, hipStream_t stream) {
  fa_status st = check_problem(p);
  if (st != FA_OK) return st;
  if (p->dtype == FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;   // fa_fwd_fp8
  if (empty_problem(p)) return FA_OK;
  if (!tensor_ok(q) || !ktensor_ok(p, k) || !ktensor_ok(p, v) || !tensor_ok(o) || !lse)
    return FA_ERR_INVALID_ARG;
  Params r = make_params(p);
  r.q = q; r.k = k; r.v = v; r.o = o; r.lse = lse;
  if (p->dtype == FA_F32) return hip_status(launch_fwd_f32(r, stream));
  return hip_status(launch_fwd_mfma(r, p->dtype, stream));
}

fa_status fa_bwd_workspace_size(const fa_problem *p, size_t *bytes) {
  if (!bytes) return FA_ERR_INVALID_ARG;
  fa_status st = check_problem(p);
  if (st != FA_OK) return st;
  if (p->dtype == FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  *bytes = empty_problem(p) ? 0 : delta_bytes(p);
  return FA_OK;
}

fa_status fa_bwd_prep(const fa_problem *p, const void *o, const void *dout, void *workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  fa_status st = check_problem(p);
  if (st != FA_OK || empty_problem(p)) return st;
  if (!tensor_ok(o) || !tensor_ok(dout)) return FA_ERR_INVALID_ARG;
  if ((st = workspace_ok(p, workspace, workspace_bytes)) != FA_OK) return st;
  Params r = make_params(p);
  r.o = (void *)o; r.dout = dout;
  bind_workspace(r, workspace);
  return hip_status(launch_bwd_prep(r, p->dtype, stream));
}

// S_q == 0 with keys: no query attends to any key, so dK = dV = 0.
bool keys_without_queries(const fa_problem *p) {
  return p->batch > 0 && p->head_num > 0 && p->seq_q == 0 && p->seq_k > 0;
}

fa_status zero_kv_grads(const fa_problem *p, void *dk, void *dv, hipStream_t stream) {
  if (!ktensor_ok(p, dk) || !ktensor_ok(p, dv)) return FA_ERR_INVALID_ARG;
  const int64_t esize = (p->dtype == FA_F32 || p->grad_f32) ? 4 : 2;
  const int64_t words = (int64_t)p->batch * p->head_num * p->seq_k * p->head_dim * esize / 4;
  hipError_t e = launch_zero_words(dk, words, stream);
  if (e == hipSuccess) e = launch_zero_words(dv, words, stream);
  return hip_status(e);
}

fa_status fa_bwd_main(const fa_problem *p, const void *q, const void *k, const void *v,
                      const float *lse, const void *dout, void *dk, void *dv,
                      const void *workspace, size_t workspace_bytes, hipStream_t stream) {
  fa_status st = check_problem(p);
  if (st != FA_OK) return st;
  if (keys_without_queries(p)) return zero_kv_grads(p, dk, dv, stream);
  if (empty_problem(p)) return FA_OK;
  if (!tensor_ok(q) || !ktensor_ok(p, k) || !ktensor_ok(p, v) || !lse || !tensor_ok(dout) ||
      !ktensor_ok(p, dk) || !ktensor_ok(p, dv))
    return FA_ERR_INVALID_ARG;
  if ((st = workspace_ok(p, workspace, workspace_bytes)) != FA_OK) return st;
  Params r = make_params(p);
  r.q = q; r.k = k; r.v = v; r.lse = (float *)lse; r.dout = dout; r.dk = dk; r.dv = dv;
  bind_workspace(r, (void *)workspace);
  if (p->dtype == FA_F32) return hip_status(launch_bwd_kv_f32(r, stream));
  return hip_status(launch_bwd_kv_mfma(r, p->dtype, stream));
}

fa_status fa_bwd_post(const fa_problem *p, const void *q, const void *k, const void *v,
                      const float *lse, const void *dout, void *dq, const void *workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  fa_status st = check_problem(p);
  if (st != FA_OK || empty_problem(p)) return st;
  if (!tensor_ok(q) || !ktensor_ok(p, k) || !ktensor_ok(p, v) || !lse || !tensor_ok(dout) ||
      !tensor_ok(dq))
    return FA_ERR_INVALID_ARG;
  if ((st = workspace_ok(p, workspace, workspace_bytes)) != FA_OK) return st;
  Params r = make_params(p);
  r.q = q; r.k = k; r.v = v; r.lse = (float *)lse; r.dout = dout; r.dq = dq;
  bind_workspace(r, (void *)workspace);
  if (p->dtype == FA_F32) return hip_status(launch_bwd_q_f32(r, stream));
  return hip_status(launch_bwd_q_mfma(r, p->dtype, stream));
}

fa_status fa_bwd(const fa_problem *p, const void *q, const void *k, const void *v, const void *o,
                 const float *lse, const void *dout, void *dq, void *dk, void *dv,
                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
  fa_status st = check_problem(p);
  if (st != FA_OK) return st;
  if (keys_without_queries(p)) return zero_kv_grads(p, dk, dv, stream);
  if (empty_problem(p)) return FA_OK;
  // validate every pointer before the first launch
  if (!tensor_ok(q) || !ktensor_ok(p, k) || !ktensor_ok(p, v) || !tensor_ok(o) || !lse ||
      !tensor_ok(dout) || !tensor_ok(dq) || !ktensor_ok(p, dk) || !ktensor_ok(p, dv))
    return FA_ERR_INVALID_ARG;
  if ((st = workspace_ok(p, workspace, workspace_bytes)) != FA_OK) return st;
  if ((st = fa_bwd_prep(p, o, dout, workspace, workspace_bytes, stream)) != FA_OK) return st;
  {
    // short query blocks: dQ, dK and dV in one pass per (batch, head)
    Params r = make_params(p);
    r.q = q; r.k = k; r.v = v; r.lse = (float *)lse; r.dout = dout;
    r.dq = dq; r.dk = dk; r.dv = dv;
    bind_workspace(r, workspace);
    if (bwd_short_fits(r, p->dtype)) return hip_status(launch_bwd_short(r, p->dtype, stream));
  }
  if ((st = fa_bwd_main(p, q, k, v, lse, dout, dk, dv, workspace, workspace_bytes, stream)) != FA_OK)
    return st;
  return fa_bwd_post(p, q, k, v, lse, dout, dq, workspace, workspace_bytes, stream);
}

fa_status fa_bwd_noalloc(const fa_problem *p, const void *q, const void *k, const void *v,
                         const void *o, const float *lse, const void *dout, void *dq, void *dk,
                         void *dv, hipStream_t stream) {
  fa_status st = check_problem(p);
  if (st != FA_OK) return st;
  if (p->dtype == FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  if (keys_without_queries(p)) return zero_kv_grads(p, dk, dv, stream);
  if (empty_problem(p)) return FA_OK;
  if (!tensor_ok(q) || !ktensor_ok(p, k) || !ktensor_ok(p, v) || !tensor_ok(o) || !lse ||
      !tensor_ok(dout) || !tensor_ok(dq) || !ktensor_ok(p, dk) || !ktensor_ok(p, dv))
    return FA_ERR_INVALID_ARG;
  if (delta_bytes(p) > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  void *ws = nullptr;
  if ((st = current_scratch(&ws)) != FA_OK) return st;
  return fa_bwd(p, q, k, v, o, lse, dout, dq, dk, dv, ws, FA_NOALLOC_SCRATCH_BYTES, stream);
}

fa_status fa_fwd_fp8_workspace_size(const fa_problem *p, size_t *bytes) {
  if (!bytes) return FA_ERR_INVALID_ARG;
  fa_status st = check_problem(p);
  if (st != FA_OK) return st;
  if (p->dtype != FA_FP8_E4M3) return FA_ERR_INVALID_ARG;
  if (empty_problem(p)) { *bytes = 0; return FA_OK; }
  *bytes = round256(fwd_fp8_workspace_bytes(make_params(p)));
  return FA_OK;
}

fa_status fa_fwd_fp8(const fa_problem *p, const void *q, const void *k, const void *v,
                     float q_descale, float k_descale, float v_descale, void *o, float *lse,
                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
  fa_status st = check_problem(p);
  if (st != FA_OK) return st;
  if (p->dtype != FA_FP8_E4M3) return FA_ERR_INVALID_ARG;
  if (!(isfinite(q_descale) && q_descale > 0.f) || !(isfinite(k_descale) && k_descale > 0.f) ||
      !(isfinite(v_descale) && v_descale > 0.f))
    return FA_ERR_INVALID_ARG;
  if (empty_problem(p)) return FA_OK;
  if (!tensor_ok(q) || !ktensor_ok(p, k) || !ktensor_ok(p, v) || !tensor_ok(o) || !lse)
    return FA_ERR_INVALID_ARG;
  Params r = make_params(p);
  const size_t need = fwd_fp8_workspace_bytes(r);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (need > 0 && !tensor_ok(workspace)) return FA_ERR_INVALID_ARG;
  r.q = q; r.k = k; r.v = v; r.o = o; r.lse = lse;
  r.fp8_qk = q_descale * k_descale;
  r.fp8_v = v_descale;
  r.vt = workspace;
  return hip_status(launch_fwd_fp8(r, stream));
}

fa_status fa_maxsim(const fa_maxsim_problem *p, const void *q, const void *d, float *rowmax,
                    float *score, hipStream_t stream) {
  if (!p) return FA_ERR_INVALID_ARG;
  if (p->batch < 0 || p->len_q < 0 || p->len_d < 0 || p->dim <= 0 || p->pad0 != 0)
    return FA_ERR_INVALID_ARG;
  if (p->dtype != FA_F32 && p->dtype != FA_F16 && p->dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (p->dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (p->dim % 128 != 0 || p->dim > kMaxSimMaxDim || p->len_d > kMaxSimMaxDocs)
    return FA_ERR_UNSUPPORTED;
  const int64_t b_pad = ((int64_t)p->batch + 7) / 8 * 8;
  if (b_pad * (((int64_t)p->len_q + 31) / 32) > INT32_MAX || (int64_t)p->batch * p->len_q > INT32_MAX)
    return FA_ERR_UNSUPPORTED;
  if (p->batch == 0) return FA_OK;
  if (!score || ((uintptr_t)score & 3u)) return FA_ERR_INVALID_ARG;
  if (p->len_q > 0 && (!tensor_ok(q) || !rowmax || ((uintptr_t)rowmax & 3u)))
    return FA_ERR_INVALID_ARG;
  if (p->len_q > 0 && p->len_d > 0 && !tensor_ok(d)) return FA_ERR_INVALID_ARG;
  MaxSimParams r;
  memset(&r, 0, sizeof(r));
  r.q = q; r.d = d; r.q_valid = p->q_valid; r.d_valid = p->d_valid;
  r.rowmax = rowmax; r.score = score;
  r.B = p->batch; r.Lq = p->len_q; r.Ld = p->len_d; r.D = p->dim;
  return hip_status(launch_maxsim(r, p->dtype, stream));
}

}  // extern "C"
