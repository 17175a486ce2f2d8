// Backward attention, bf16/f16 inputs, MFMA on gfx950.
//
// Recompute-based gradient (FlashAttentionScore replacement guide, section
// 2: gradients are formed without the N x N matrix, from O(N) saved
// statistics).  Only O and the row LSE come from the forward; every P tile is
// recomputed as P = exp2(S * scale * log2 e + bias * log2 e - LSE * log2 e).
//
// Workgroup = 4 waves owning BNB = 128 consecutive keys (32 per wave) of one
// (batch, head); it walks the query blocks of 32 rows that can see those keys
// (causal: from the diagonal down).  Per query block, per wave:
//
//   S  = Q  . K^T    A = Q  tile (LDS, row-major)    B = K rows (VGPRs)
//   dP = dO . V^T    A = dO tile (LDS, row-major)    B = V rows (VGPRs)
//   P  = exp2(...), dS = P * (dP - delta_i)          (fp32, in registers)
//   dV += P^T . dO   A = P^T from the S accumulators B = dO^T tile (LDS)
//   dK += dS^T . Q   A = dS^T from registers         B = Q^T tile (LDS)
//   dQ  = dS . K     A = dS of all 128 keys (LDS)    B = K^T (VGPRs)
//
// In the 32x32 accumulator layout lane l holds key l%32 of the wave and 16
// query rows, which is exactly the A-operand layout of P^T / dS^T for the dV
// and dK products (keys as rows, queries as the contraction index), so those
// two need no data movement.  dQ contracts over keys instead, so dS goes
// through LDS once; each wave then forms dQ for one 32-column block of D over
// the workgroup's keys and adds it to the float32 accumulator with hardware
// float atomics.  Q^T and dO^T tiles use the same bits-2-and-3 swapped
// position order inside each 16-row chunk as the forward's V^T tile.
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int NWB = 4;      // waves per workgroup
constexpr int BNB = 128;    // keys per workgroup
constexpr int BMB = 32;     // queries per iteration

template <typename T> struct MfmaB;
template <> struct MfmaB<__bf16> {
  static __device__ __forceinline__ f32x16 mac(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct MfmaB<_Float16> {
  static __device__ __forceinline__ f32x16 mac(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

__device__ __forceinline__ int chunk_pos_b(int u) {
  return (u & 3) | ((u & 4) << 1) | ((u & 8) >> 1);
}
__device__ __forceinline__ uint32_t lo_h(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_h(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

template <int D>
struct BwdCfg {
  static constexpr int NT = NWB * 64;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int QP = D + 8;      // row-major Q / dO tile pitch
  static constexpr int TP = BMB + 8;    // transposed tile pitch
  static constexpr int SP = BNB + 8;    // dS tile pitch
  static constexpr int WPD = NWB / DB;  // waves sharing one dQ column block
  static constexpr int NCH = (BNB / 16) / WPD;  // 16-key chunks per wave for dQ
  static constexpr int UNITS = (BMB / 4) * (D / 8);  // 4-row x 8-col units per tile
};

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void bwd_mfma_kernel(Params p, int n_ktiles) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[BMB * C::QP];
  __shared__ __attribute__((aligned(16))) uint16_t Gs[BMB * C::QP];
  __shared__ __attribute__((aligned(16))) uint16_t QTs[D * C::TP];
  __shared__ __attribute__((aligned(16))) uint16_t GTs[D * C::TP];
  __shared__ __attribute__((aligned(16))) uint16_t dSs[BMB * C::SP];
  __shared__ float lse_s[BMB], dlt_s[BMB];

  const int BH = p.B * p.H;
  const int lin = blockIdx.x;
  const int kt = lin / BH;          // key tile 0 has the most causal work: first
  const int bh = lin % BH;
  const int b = bh / p.H, h = bh % p.H;
  const int j0 = kt * BNB;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 5, lr = l & 31;
  const int jw = j0 + 32 * w;
  const int my_j = jw + lr;
  const uint32_t flags = p.mask_flags;
  const bool causal = flags & FA_MASK_CAUSAL;
  const bool elem_mask_any = flags & (FA_MASK_PADDING | FA_MASK_MODALITY | FA_MASK_EXPLICIT);

  const int64_t qoff = b * p.q_sb + h * p.q_sh;
  const int64_t koff = b * p.k_sb + h * p.k_sh;
  const T *Qg = (const T *)p.q + qoff;
  const T *Gg = (const T *)p.dout + qoff;
  const T *Kg = (const T *)p.k + koff;
  const T *Vg = (const T *)p.v + koff;
  const int64_t rbase = ((int64_t)b * p.H + h) * p.Sq;

  // ---- resident operands: K and V rows of this lane's key, K^T for dQ
  u32x4 kf[C::KS], vf[C::KS];
#pragma unroll
  for (int t = 0; t < C::KS; ++t) {
    if (my_j < p.Sk) {
      kf[t] = *(const u32x4 *)(Kg + (int64_t)my_j * p.k_ss + 16 * t + 8 * g);
      vf[t] = *(const u32x4 *)(Vg + (int64_t)my_j * p.k_ss + 16 * t + 8 * g);
    } else {
      kf[t] = vf[t] = u32x4{0, 0, 0, 0};
    }
  }
  const int dbq = w % C::DB;                 // dQ column block of this wave
  const int c0 = (w / C::DB) * C::NCH;       // first 16-key chunk of this wave for dQ
  u32x4 ktf[C::NCH];
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    uint16_t e[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int j = j0 + 16 * (c0 + c) + 8 * g + s;
      e[s] = (j < p.Sk) ? ((const uint16_t *)Kg)[(int64_t)j * p.k_ss + 32 * dbq + lr] : 0;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) ktf[c][s] = (uint32_t)e[2 * s] | ((uint32_t)e[2 * s + 1] << 16);
  }

  f32x16 dv[C::DB], dk[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dv[db] = dk[db] = f32x16{};

  const float sl2 = (p.pse_kind == FA_PSE_ALIBI) ? p.alibi_slopes[h] * kLog2e : 0.f;

  // query blocks that can see this key tile
  const int it_begin = causal ? (j0 / BMB) : 0;
  const int it_end = (p.Sq + BMB - 1) / BMB;

  // ---- staging of one query block: Q, dO row-major and transposed, LSE, delta
  u32x4 ld[4];
  auto gload = [&](int it) {
    const int i0 = it * BMB;
    const int u = tid % C::UNITS;
    const int which = tid / C::UNITS;  // 0: Q, 1: dO, else idle
    const int i4 = u / (D / 8), col8 = u % (D / 8);
    const T *src = which == 0 ? Qg : Gg;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 4 * i4 + r;
      if (which < 2 && i < p.Sq)
        ld[r] = *(const u32x4 *)(src + (int64_t)i * p.q_ss + col8 * 8);
      else
        ld[r] = u32x4{0, 0, 0, 0};
    }
  };
  float ls_reg = 0.f;
  auto gload_stats = [&](int it) {
    const int i = it * BMB + (tid & 31);
    if (tid < 32) {
      const float v = i < p.Sq ? p.lse[rbase + i] : -INFINITY;
      ls_reg = (v == -INFINITY) ? INFINITY : v * kLog2e;   // dead rows: P = 0
    } else if (tid < 64) {
      ls_reg = i < p.Sq ? p.delta[rbase + i] : 0.f;
    }
  };
  auto sstore = [&]() {
    const int u = tid % C::UNITS;
    const int which = tid / C::UNITS;
    if (which < 2) {
      const int i4 = u / (D / 8), col8 = u % (D / 8);
      uint16_t *nat = which == 0 ? Qs : Gs;
      uint16_t *tr = which == 0 ? QTs : GTs;
#pragma unroll
      for (int r = 0; r < 4; ++r) *(u32x4 *)(&nat[(4 * i4 + r) * C::QP + col8 * 8]) = ld[r];
      const int pos = 16 * (i4 >> 2) + chunk_pos_b(4 * (i4 & 3));
      uint16_t *dst = &tr[(col8 * 8) * C::TP + pos];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t a0 = ld[0][e2], a1 = ld[1][e2], a2 = ld[2][e2], a3 = ld[3][e2];
        *(u32x2 *)(dst + (2 * e2) * C::TP) = u32x2{lo_h(a0, a1), lo_h(a2, a3)};
        *(u32x2 *)(dst + (2 * e2 + 1) * C::TP) = u32x2{hi_h(a0, a1), hi_h(a2, a3)};
      }
    }
    if (tid < 32) lse_s[tid] = ls_reg;
    else if (tid < 64) dlt_s[tid - 32] = ls_reg;
  };

  if (it_begin < it_end) {
    gload(it_begin);
    gload_stats(it_begin);
    sstore();
  }
  __syncthreads();

  for (int it = it_begin; it < it_end; ++it) {
    const bool has_next = it + 1 < it_end;
    if (has_next) {
      gload(it + 1);
      gload_stats(it + 1);
    }
    const int i0 = it * BMB;
    // wave-level classification of this (query block, 32 keys) tile
    bool skip = jw >= p.Sk;
    bool need_mask = elem_mask_any || (jw + 32 > p.Sk) || (i0 + BMB > p.Sq);
    if (causal) {
      if (jw > i0 + BMB - 1) skip = true;
      if (jw + 31 > i0) need_mask = true;
    }
    if (!skip) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < C::KS; ++t) {
        const u32x4 aq = *(const u32x4 *)(&Qs[lr * C::QP + 16 * t + 8 * g]);
        const u32x4 ag = *(const u32x4 *)(&Gs[lr * C::QP + 16 * t + 8 * g]);
        s = MfmaB<T>::mac(aq, kf[t], s);
        dp = MfmaB<T>::mac(ag, vf[t], dp);
      }
      // P and dS; element r: query i0 + 8(r/4) + 4g + r%4, key my_j
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = 8 * (r >> 2) + 4 * g + (r & 3);
        const int i = i0 + il;
        float t = s[r] * p.scale_log2;
        if (p.pse_kind == FA_PSE_ALIBI) t -= sl2 * fabsf((float)(i - my_j));
        else if (p.pse_kind == FA_PSE_DENSE && i < p.Sq && my_j < p.Sk)
          t += dense_bias(p, b, h, i, my_j) * kLog2e;
        float pr = exp2_fast(t - lse_s[il]);
        if (need_mask) {
          bool ok = i < p.Sq && my_j < p.Sk;
          if (ok) ok = allowed_elem(p, b, h, i, my_j);
          if (!ok) pr = 0.f;
        }
        s[r] = pr;
        dp[r] = pr * (dp[r] - dlt_s[il]);
      }
      // dV += P^T dO, dK += dS^T Q (contraction over the 32 queries)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int r0 = 8 * c;
        u32x4 pp, pd;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          pp[q2] = pack2<T>(s[r0 + 2 * q2], s[r0 + 2 * q2 + 1]);
          pd[q2] = pack2<T>(dp[r0 + 2 * q2], dp[r0 + 2 * q2 + 1]);
        }
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const u32x4 bg = *(const u32x4 *)(&GTs[(32 * db + lr) * C::TP + 16 * c + 8 * g]);
          const u32x4 bq = *(const u32x4 *)(&QTs[(32 * db + lr) * C::TP + 16 * c + 8 * g]);
          dv[db] = MfmaB<T>::mac(pp, bg, dv[db]);
          dk[db] = MfmaB<T>::mac(pd, bq, dk[db]);
        }
      }
      // dS (rounded) to LDS, row = query, column = key of the workgroup
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = 8 * (r >> 2) + 4 * g + (r & 3);
        const uint32_t v = pack2<T>(dp[r], 0.f);
        dSs[il * C::SP + 32 * w + lr] = (uint16_t)(v & 0xffffu);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = 8 * (r >> 2) + 4 * g + (r & 3);
        dSs[il * C::SP + 32 * w + lr] = 0;
      }
    }
    lds_barrier();
    // dQ(block) += dS . K over this wave's key chunks, column block dbq
    {
      f32x16 dq0 = f32x16{}, dq1 = f32x16{};   // two independent MFMA chains
#pragma unroll
      for (int c = 0; c < C::NCH; c += 2) {
        const u32x4 a0 = *(const u32x4 *)(&dSs[lr * C::SP + 16 * (c0 + c) + 8 * g]);
        const u32x4 a1 = *(const u32x4 *)(&dSs[lr * C::SP + 16 * (c0 + c + 1) + 8 * g]);
        dq0 = MfmaB<T>::mac(a0, ktf[c], dq0);
        dq1 = MfmaB<T>::mac(a1, ktf[c + 1], dq1);
      }
      const f32x16 dq = dq0 + dq1;
      float *dst = p.dq_acc + (rbase + i0) * D + 32 * dbq + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = 8 * (r >> 2) + 4 * g + (r & 3);
        if (i0 + il < p.Sq) unsafeAtomicAdd(dst + (int64_t)il * D, dq[r]);
      }
    }
    if (has_next) sstore();
    lds_barrier();
  }

  // ---- write dK (scaled) and dV; element r: key jw + 8(r/4) + 4g + r%4, column 32db + lr
  T *DKg = (T *)p.dk + koff;
  T *DVg = (T *)p.dv + koff;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = jw + 8 * (r >> 2) + 4 * g + (r & 3);
      if (j < p.Sk) {
        DKg[(int64_t)j * p.k_ss + 32 * db + lr] = from_f32<T>(dk[db][r] * p.scale);
        DVg[(int64_t)j * p.k_ss + 32 * db + lr] = from_f32<T>(dv[db][r]);
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_t(const Params &p, hipStream_t s) {
  const int n_ktiles = (p.Sk + BNB - 1) / BNB;
  const int64_t blocks = (int64_t)n_ktiles * p.B * p.H;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_mfma_kernel<T, D>), dim3((unsigned)blocks), dim3(NWB * 64), 0, s, p,
                     n_ktiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_mfma(const Params &p, int dtype, hipStream_t s) {
  if (dtype == FA_BF16) {
    if (p.D == 64) return launch_t<__bf16, 64>(p, s);
    if (p.D == 128) return launch_t<__bf16, 128>(p, s);
  } else if (dtype == FA_F16) {
    if (p.D == 64) return launch_t<_Float16, 64>(p, s);
    if (p.D == 128) return launch_t<_Float16, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
