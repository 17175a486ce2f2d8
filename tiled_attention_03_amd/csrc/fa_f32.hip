// fp32 attention path and the dtype-generic backward prep pass.
//
// The fp32 path keeps every product and sum in fp32 FMA (no bf16/xf32
// shortcut).  One query row (forward, dQ) or one key row (dK/dV) is owned by
// D/32 adjacent lanes, each holding 32 of the row's D elements; dot products
// are finished with xor-shuffles inside that lane group.  Key (or query)
// tiles of 32 rows are staged through LDS and read as broadcasts.
//
// Forward: the online softmax of the FlashAttentionScore guide (section 2):
// running max m and running sum l per row, the accumulator rescaled by
// exp(m_old - m_new) whenever the max grows, so the S x S matrix is never
// stored.  Backward: P is recomputed from the saved LSE, then
// dP = dO.v, dS = P (dP - delta), dQ += dS k (query-owned kernel) and
// dV += P dO, dK += dS q (key-owned kernel): no atomics, deterministic.
// The prep pass forms delta_i = sum_d dO_id O_id for every dtype.
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kTile = 32;  // rows per LDS tile

template <int D>
struct RowSplit {
  static constexpr int TPR = D / 32;         // lanes per row
  static constexpr int ROWS = 256 / TPR;     // rows per 256-thread workgroup
};

template <int TPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ float bias_nat(const Params &p, int b, int h, int i, int j) {
  float bias = 0.f;
  if (p.pse_kind == FA_PSE_ALIBI) bias = -p.alibi_slopes[h] * fabsf((float)(i - j));
  else if (p.pse_kind == FA_PSE_DENSE) bias = dense_bias(p, b, h, i, j);
  return bias;
}

template <int D>
__device__ __forceinline__ void stage_rows(float (*dst)[D], const float *src, int64_t row_stride,
                                           int r0, int nrows_total) {
  for (int idx = threadIdx.x; idx < kTile * D; idx += 256) {
    int r = idx / D, c = idx % D;
    int rr = r0 + r;
    dst[r][c] = (rr < nrows_total) ? src[(int64_t)rr * row_stride + c] : 0.f;
  }
}

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(Params p) {
  constexpr int TPR = RowSplit<D>::TPR, ROWS = RowSplit<D>::ROWS;
  __shared__ float Ks[kTile][D];
  __shared__ float Vs[kTile][D];
  const int bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int i = blockIdx.x * ROWS + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  const float *Q = (const float *)p.q + b * p.q_sb + h * p.q_sh;
  const float *K = (const float *)p.k + b * p.k_sb + h * p.k_sh;
  const float *V = (const float *)p.v + b * p.k_sb + h * p.k_sh;
  float q[32], acc[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    q[e] = (i < p.Sq) ? Q[(int64_t)i * p.q_ss + part * 32 + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int k0 = 0; k0 < p.Sk; k0 += kTile) {
    __syncthreads();
    stage_rows<D>(Ks, K, p.k_ss, k0, p.Sk);
    stage_rows<D>(Vs, V, p.k_ss, k0, p.Sk);
    __syncthreads();
    const int nk = min(kTile, p.Sk - k0);
    for (int jj = 0; jj < nk; ++jj) {
      const int j = k0 + jj;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) s = fmaf(q[e], Ks[jj][part * 32 + e], s);
      s = group_sum<TPR>(s);
      if (i >= p.Sq || !allowed_elem(p, b, h, i, j)) continue;
      const float t = s * p.scale + bias_nat(p, b, h, i, j);
      if (t > m) {
        const float a = expf(m - t);
        l *= a;
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[e] *= a;
        m = t;
      }
      const float pe = expf(t - m);
      l += pe;
#pragma unroll
      for (int e = 0; e < 32; ++e) acc[e] = fmaf(pe, Vs[jj][part * 32 + e], acc[e]);
    }
  }
  if (i < p.Sq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float *O = (float *)p.o + b * p.q_sb + h * p.q_sh + (int64_t)i * p.q_ss + part * 32;
#pragma unroll
    for (int e = 0; e < 32; ++e) O[e] = acc[e] * inv;
    if (part == 0) p.lse[((int64_t)b * p.H + h) * p.Sq + i] = l > 0.f ? m + logf(l) : -INFINITY;
  }
}

// dQ = scale * sum_j dS_ij k_j, one query row per lane group.
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(Params p) {
  constexpr int TPR = RowSplit<D>::TPR, ROWS = RowSplit<D>::ROWS;
  __shared__ float Ks[kTile][D];
  __shared__ float Vs[kTile][D];
  const int bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int i = blockIdx.x * ROWS + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  const float *Q = (const float *)p.q + b * p.q_sb + h * p.q_sh;
  const float *dO = (const float *)p.dout + b * p.q_sb + h * p.q_sh;
  const float *K = (const float *)p.k + b * p.k_sb + h * p.k_sh;
  const float *V = (const float *)p.v + b * p.k_sb + h * p.k_sh;
  float q[32], g[32], acc[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    q[e] = (i < p.Sq) ? Q[(int64_t)i * p.q_ss + part * 32 + e] : 0.f;
    g[e] = (i < p.Sq) ? dO[(int64_t)i * p.q_ss + part * 32 + e] : 0.f;
    acc[e] = 0.f;
  }
  const int64_t row = ((int64_t)b * p.H + h) * p.Sq + i;
  const float lse = (i < p.Sq) ? p.lse[row] : -INFINITY;
  const float dl = (i < p.Sq) ? p.delta[row] : 0.f;
  const bool live = lse != -INFINITY;
  for (int k0 = 0; k0 < p.Sk; k0 += kTile) {
    __syncthreads();
    stage_rows<D>(Ks, K, p.k_ss, k0, p.Sk);
    stage_rows<D>(Vs, V, p.k_ss, k0, p.Sk);
    __syncthreads();
    const int nk = min(kTile, p.Sk - k0);
    for (int jj = 0; jj < nk; ++jj) {
      const int j = k0 + jj;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        s = fmaf(q[e], Ks[jj][part * 32 + e], s);
        dp = fmaf(g[e], Vs[jj][part * 32 + e], dp);
      }
      s = group_sum<TPR>(s);
      dp = group_sum<TPR>(dp);
      if (!live || !allowed_elem(p, b, h, i, j)) continue;
      const float P = expf(s * p.scale + bias_nat(p, b, h, i, j) - lse);
      const float ds = P * (dp - dl);
#pragma unroll
      for (int e = 0; e < 32; ++e) acc[e] = fmaf(ds, Ks[jj][part * 32 + e], acc[e]);
    }
  }
  if (i < p.Sq) {
    float *out = (float *)p.dq + b * p.q_sb + h * p.q_sh + (int64_t)i * p.q_ss + part * 32;
#pragma unroll
    for (int e = 0; e < 32; ++e) out[e] = acc[e] * p.scale;
  }
}

// dK, dV, one key row per lane group.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(Params p) {
  constexpr int TPR = RowSplit<D>::TPR, ROWS = RowSplit<D>::ROWS;
  __shared__ float Qs[kTile][D];
  __shared__ float Gs[kTile][D];
  __shared__ float Ls[kTile], Ds[kTile];
  const int bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int j = blockIdx.x * ROWS + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  const float *Q = (const float *)p.q + b * p.q_sb + h * p.q_sh;
  const float *dO = (const float *)p.dout + b * p.q_sb + h * p.q_sh;
  const float *K = (const float *)p.k + b * p.k_sb + h * p.k_sh;
  const float *V = (const float *)p.v + b * p.k_sb + h * p.k_sh;
  float kr[32], vr[32], dk[32], dv[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    kr[e] = (j < p.Sk) ? K[(int64_t)j * p.k_ss + part * 32 + e] : 0.f;
    vr[e] = (j < p.Sk) ? V[(int64_t)j * p.k_ss + part * 32 + e] : 0.f;
    dk[e] = dv[e] = 0.f;
  }
  const int64_t rbase = ((int64_t)b * p.H + h) * p.Sq;
  for (int i0 = 0; i0 < p.Sq; i0 += kTile) {
    __syncthreads();
    stage_rows<D>(Qs, Q, p.q_ss, i0, p.Sq);
    stage_rows<D>(Gs, dO, p.q_ss, i0, p.Sq);
    if (threadIdx.x < kTile) {
      const int ii = i0 + threadIdx.x;
      Ls[threadIdx.x] = ii < p.Sq ? p.lse[rbase + ii] : -INFINITY;
      Ds[threadIdx.x] = ii < p.Sq ? p.delta[rbase + ii] : 0.f;
    }
    __syncthreads();
    const int nq = min(kTile, p.Sq - i0);
    for (int ii = 0; ii < nq; ++ii) {
      const int i = i0 + ii;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        s = fmaf(Qs[ii][part * 32 + e], kr[e], s);
        dp = fmaf(Gs[ii][part * 32 + e], vr[e], dp);
      }
      s = group_sum<TPR>(s);
      dp = group_sum<TPR>(dp);
      const float lse = Ls[ii];
      if (j >= p.Sk || lse == -INFINITY || !allowed_elem(p, b, h, i, j)) continue;
      const float P = expf(s * p.scale + bias_nat(p, b, h, i, j) - lse);
      const float ds = P * (dp - Ds[ii]);
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        dv[e] = fmaf(P, Gs[ii][part * 32 + e], dv[e]);
        dk[e] = fmaf(ds, Qs[ii][part * 32 + e], dk[e]);
      }
    }
  }
  if (j < p.Sk) {
    float *DK = (float *)p.dk + b * p.k_sb + h * p.k_sh + (int64_t)j * p.k_ss + part * 32;
    float *DV = (float *)p.dv + b * p.k_sb + h * p.k_sh + (int64_t)j * p.k_ss + part * 32;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      DK[e] = dk[e] * p.scale;
      DV[e] = dv[e];
    }
  }
}

// ---------------------------------------------------------------------------
// dtype-generic passes: 8 elements of a row per lane.

template <typename T>
__global__ __launch_bounds__(256) void bwd_prep_kernel(Params p) {
  const int lanes_per_row = p.D / 8;
  const int rows_per_block = 256 / lanes_per_row;
  const int bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int i = blockIdx.x * rows_per_block + threadIdx.x / lanes_per_row;
  const int part = threadIdx.x % lanes_per_row;
  float acc = 0.f;
  const int64_t row = ((int64_t)b * p.H + h) * p.Sq + i;
  if (i < p.Sq) {
    const int64_t off = b * p.q_sb + h * p.q_sh + (int64_t)i * p.q_ss + part * 8;
    const T *O = (const T *)p.o + off;
    const T *G = (const T *)p.dout + off;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(to_f32<T>(O[e]), to_f32<T>(G[e]), acc);
  }
  for (int off = 1; off < lanes_per_row; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (i < p.Sq && part == 0) p.delta[row] = acc;
}

template <int D>
hipError_t fwd_f32_d(const Params &p, hipStream_t s) {
  dim3 grid((p.Sq + RowSplit<D>::ROWS - 1) / RowSplit<D>::ROWS, p.B * p.H);
  hipLaunchKernelGGL(fwd_f32_kernel<D>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_kv_f32_d(const Params &p, hipStream_t s) {
  if (p.Sk == 0) return hipSuccess;
  dim3 gk((p.Sk + RowSplit<D>::ROWS - 1) / RowSplit<D>::ROWS, p.B * p.H);
  hipLaunchKernelGGL(bwd_dkdv_f32_kernel<D>, gk, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_q_f32_d(const Params &p, hipStream_t s) {
  dim3 gq((p.Sq + RowSplit<D>::ROWS - 1) / RowSplit<D>::ROWS, p.B * p.H);
  hipLaunchKernelGGL(bwd_dq_f32_kernel<D>, gq, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_prep_t(const Params &p, hipStream_t s) {
  const int rows_per_block = 256 / (p.D / 8);
  dim3 grid((p.Sq + rows_per_block - 1) / rows_per_block, p.B * p.H);
  hipLaunchKernelGGL(bwd_prep_kernel<T>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const Params &p, hipStream_t s) {
  switch (p.D) {
    case 32: return fwd_f32_d<32>(p, s);
    case 64: return fwd_f32_d<64>(p, s);
    case 128: return fwd_f32_d<128>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_kv_f32(const Params &p, hipStream_t s) {
  switch (p.D) {
    case 32: return bwd_kv_f32_d<32>(p, s);
    case 64: return bwd_kv_f32_d<64>(p, s);
    case 128: return bwd_kv_f32_d<128>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_q_f32(const Params &p, hipStream_t s) {
  switch (p.D) {
    case 32: return bwd_q_f32_d<32>(p, s);
    case 64: return bwd_q_f32_d<64>(p, s);
    case 128: return bwd_q_f32_d<128>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_prep(const Params &p, int dtype, hipStream_t s) {
  if (dtype == FA_F32) return launch_prep_t<float>(p, s);
  if (dtype == FA_F16) return launch_prep_t<_Float16>(p, s);
  return launch_prep_t<__bf16>(p, s);
}

}  // namespace fa
