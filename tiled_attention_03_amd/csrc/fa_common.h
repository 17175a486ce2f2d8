// Shared device-side definitions for the libfa kernels (gfx950 only).
//
// Parameter block passed by value to every kernel, element conversions, and
// the per-element mask / bias rules of the operator (see include/fa.h for
// their definition and sources).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The raw-unit ALiBi forms divide the slope by c_log2 = scale * log2(e); at
// or below this c_log2 that quotient could overflow, and the tiles take the
// per-element path instead.
constexpr float kRawMinC = 1e-20f;

struct Params {
  // tensors (device pointers)
  const void *q, *k, *v;
  void *o;
  float *lse;
  const void *dout;
  void *dq, *dk, *dv;
  float *delta;    // float32 [B,H,Sq]: delta_i = sum_d dO_id O_id
  // element strides: batch, head, row (last dim contiguous)
  int64_t q_sb, q_sh, q_ss;   // Q, O, dO, dQ
  int64_t k_sb, k_sh, k_ss;   // K, V, dK, dV
  int B, H, Sq, Sk, D;
  float scale;        // multiplies Q K^T
  float scale_log2;   // scale * log2(e)
  uint32_t mask_flags;
  // explicit mask
  const uint8_t *em;
  int64_t em_sb, em_sh, em_sq;
  // modality mask: bit (mq*8 + mk) of allow_bits set = allowed
  const int8_t *qmod, *kmod;
  uint64_t allow_bits;
  int allow_diag;
  int num_modalities;
  // padding
  const uint8_t *key_valid;
  // bias
  int pse_kind;
  int pse_dtype;
  const float *alibi_slopes;
  const void *pse;
  int64_t pse_sb, pse_sh, pse_sq;
  // dropout (keep_prob < 1): keep iff a Philox word < drop_thr; kept
  // probabilities are scaled by inv_keep
  int dropout;
  uint32_t drop_thr;
  uint32_t seed_lo, seed_hi;
  float inv_keep;
  // gradient outputs: float32 instead of the input dtype
  int grad_f32;
  // optional bias gradient, float32 contiguous [B, H, Sq, Sk]
  float *dpse;
  // fp8 forward: descale products (q * k and v) and the permuted V^T workspace
  float fp8_qk, fp8_v;
  void *vt;
};

// Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): each round multiplies counter words
// 0 and 2 by the round constants, and the new counter is (hi(w2*M1) ^ c1 ^ k0,
// lo(w2*M1), hi(w0*M0) ^ c3 ^ k1, lo(w0*M0)); the key is bumped by the Weyl
// constants between rounds.  Each product is one 32x32 -> 64-bit multiply
// (v_mad_u64_u32) rather than separate high and low halves.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)M0 * c[0];
    const uint64_t p1 = (uint64_t)M1 * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
    k0 += W0;
    k1 += W1;
  }
}

// Keep bits of keys 4*(j/4) .. 4*(j/4) + 3 for query i of head (b, h): bit t
// is set iff word t of the Philox output for counter (j/4, i, h, b), under
// the seed as key, is below the threshold.  One call serves four keys.
__device__ __forceinline__ uint32_t dropout_keep4(const Params &p, int b, int h, int i, int j) {
  uint32_t w[4] = {(uint32_t)(j >> 2), (uint32_t)i, (uint32_t)h, (uint32_t)b};
  philox4x32_10(w, p.seed_lo, p.seed_hi);
  return (uint32_t)(w[0] < p.drop_thr) | ((uint32_t)(w[1] < p.drop_thr) << 1) |
         ((uint32_t)(w[2] < p.drop_thr) << 2) | ((uint32_t)(w[3] < p.drop_thr) << 3);
}

// The factor for keep bit `bit`: inv_keep if kept, else 0.
__device__ __forceinline__ float dropout_scale(const Params &p, uint32_t bit) {
  return bit ? p.inv_keep : 0.f;
}

// ------------------------------------------------------------------------
// element conversion

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<__bf16>(__bf16 x) { return (float)x; }
template <> __device__ __forceinline__ float to_f32<_Float16>(_Float16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// float -> bf16 / f16 conversions round to nearest even.
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }

// Two floats -> one dword holding two 16-bit values (lo in bits 0..15), RNE.
template <typename T> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<__bf16>(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
template <> __device__ __forceinline__ uint32_t pack2<_Float16>(float lo, float hi) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resource over [base, base + bytes): loads at offsets past the end
// return zeros (no fault), which is how tile tails are zero-filled.  Offsets
// are 32-bit, so callers keep one (batch, head) span below 2 GiB.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
// Bytes spanned by `rows` rows of `d` elements at row stride `stride` elements.
__device__ __forceinline__ uint32_t span_bytes(int rows, int64_t stride, int d, int esize) {
  return rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * stride + d) * esize) : 0u;
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete before it arrives, so after the barrier every wave sees every
// other wave's LDS writes.  Outstanding global loads, stores and atomics are
// not waited for (a plain __syncthreads() fence would wait for them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// ------------------------------------------------------------------------
// mask and bias rules, one element at a time (partial tiles only)

__device__ __forceinline__ bool modality_ok(const Params &p, int mq, int mk, int i, int j) {
  bool ok = (p.allow_bits >> ((unsigned)(mq * 8 + mk))) & 1ull;
  return ok || (p.allow_diag && i == j);
}

// Everything except the S_k bound, which the tile loops handle
// arithmetically.  No early exit: the loads of the different rules do not
// depend on each other, so the loads of a whole unrolled block of elements
// can be in flight together.
__device__ __forceinline__ bool allowed_elem(const Params &p, int b, int h, int i, int j) {
  const uint32_t f = p.mask_flags;
  bool ok = !(f & FA_MASK_CAUSAL) || j <= i;
  if (f & FA_MASK_PADDING) ok &= p.key_valid[(int64_t)b * p.Sk + j] != 0;
  if (f & FA_MASK_MODALITY) {
    const int mq = p.qmod[(int64_t)b * p.Sq + i];
    const int mk = p.kmod[(int64_t)b * p.Sk + j];
    ok &= modality_ok(p, mq, mk, i, j);
  }
  if (f & FA_MASK_EXPLICIT)
    ok &= p.em[(int64_t)b * p.em_sb + (int64_t)h * p.em_sh + (int64_t)i * p.em_sq + j] != 0;
  return ok;
}

// The same rules (all but the causal rule) for a block of 32 elements at
// once, built from wave-wide votes instead of one global load per element.
// Every lane of the wave must call it (it votes).
//
// col_querymask: the lane's key j against the 32 queries [i0, i0 + 32): bit c
// set iff query i0 + c < S_q may attend key j.  key_ok: key j exists and is
// valid (padding); col_allow: the query modalities allowed to see key j's
// modality (bit mq set = allowed).  Only the bits of the lane's own queries
// (c = 8q + 4g + t) carry the explicit mask.
__device__ __forceinline__ uint32_t col_querymask(const Params &p, int b, int h, int j, int i0,
                                                  bool key_ok, uint32_t col_allow, int l) {
  const uint32_t f = p.mask_flags;
  const int i = i0 + (l & 31);
  const bool in = i < p.Sq;
  uint32_t m = (uint32_t)__ballot(in);
  if (f & FA_MASK_MODALITY) {
    const int mq = in ? p.qmod[(int64_t)b * p.Sq + i] : -1;
    uint32_t allowed = 0u;
    for (int mm = 0; mm < p.num_modalities; ++mm) {
      const uint32_t qm = (uint32_t)__ballot(mq == mm);
      if ((col_allow >> mm) & 1u) allowed |= qm;
    }
    if (p.allow_diag && j >= i0 && j < i0 + 32) allowed |= 1u << (j - i0);
    m &= allowed;
  }
  if (!key_ok) m = 0u;
  if ((f & FA_MASK_EXPLICIT) && m) {
    const uint8_t *col = p.em + (int64_t)b * p.em_sb + (int64_t)h * p.em_sh + j;
    const int g = (l >> 5) & 1;
    uint32_t ex = 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = 8 * q + 4 * g + t;
        if (i0 + c < p.Sq && col[(int64_t)(i0 + c) * p.em_sq]) ex |= 1u << c;
      }
    m &= ex;
  }
  return m;
}

// Dense bias element (natural units, unscaled).
__device__ __forceinline__ float dense_bias(const Params &p, int b, int h, int i, int j) {
  int64_t off = (int64_t)b * p.pse_sb + (int64_t)h * p.pse_sh + (int64_t)i * p.pse_sq + j;
  if (p.pse_dtype == FA_F32) return ((const float *)p.pse)[off];
  if (p.pse_dtype == FA_BF16) return (float)((const __bf16 *)p.pse)[off];
  return (float)((const _Float16 *)p.pse)[off];
}

}  // namespace fa
