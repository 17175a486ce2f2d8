// MaxSim late-interaction scores (retrieval page, "Layer 2: semantic
// modelling"): rowmax[b, i] = max over valid document tokens j of q_i . d_j,
// score[b] = (sum of rowmax over valid query tokens) / L_q.
//
// The work is one streaming pass over the document embeddings: every
// document row is read once and dotted with the 32 query rows of a block,
// so at the shapes of a late-interaction workload (32 query tokens, hundreds
// of document tokens, D = 768) the kernel is bound by HBM, not by the
// products.  The products still run on MFMA (32x32x16, fp32 accumulation):
// the document rows go straight from HBM into operand registers, with no LDS
// staging.
//
// Workgroup = (sample b, block of 32 query tokens), NW = 16 waves.  Wave w
// owns document tiles (32 tokens each) w, w + NW, w + 2 NW, ...  With the
// tiles dealt out this way every wave of the grid carries (nearly) the same
// number of tiles, whatever each sample's document length: under a
// saturated HBM all waves stream at about the same rate, so they also finish
// together (with whole samples per wave group, the longest samples would set
// the end).  The query blocks of one sample share their blockIdx modulo 8,
// i.e. one XCD, so with several query blocks the documents come from L2 after
// the first pass.
//  1. Each wave reads the validity bytes of its tiles (one byte per lane, two
//     tiles per load), and lists, in wave-private LDS, the tiles that hold at
//     least one valid token: padding is never read.  Meanwhile the query
//     block is copied to LDS by direct-to-LDS loads (swizzled rows; rows past
//     L_q are zeros).
//  2. A tile is consumed in blocks of 64 dimensions; RING blocks are in
//     flight ahead of the one being multiplied, across the wave's tiles.  The
//     products are 16x16x32 MFMAs, S^T = D Q^T per 16 documents and 16
//     queries: their A operand takes 16 document rows (lane l: row l % 16,
//     8 dimensions at 8 (l / 16)), so one 16-byte load per lane reads 16 rows
//     x 64 contiguous bytes.  Loads that each touch 32 rows (the 32x32x16
//     operand) streamed at about 30 GB/s per workgroup, half the rate of
//     loads of the same bytes over fewer rows.  Lane l holds query column
//     l % 16 and 4 document rows of each product, so a tile's masked max is
//     a per-lane max over registers, then over the 4 lanes of a column.
//  3. The two lanes of a query column and the NW waves are merged; rowmax is
//     written, and with a single query block the score as well (fixed-order
//     sum; the result is bitwise repeatable).  With several query blocks a
//     second small kernel forms the scores from rowmax.
//
// Within a 64-dimension block, k-step t covers dimensions 32t .. 32t + 31:
// lane quarter k = l / 16 holds dimensions 32t + 8k .. 32t + 8k + 7 of its
// row, on both operands.
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

template <typename T> struct Mfma16;
template <> struct Mfma16<__bf16> {
  static __device__ __forceinline__ f32x4 mac(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mfma16<_Float16> {
  static __device__ __forceinline__ f32x4 mac(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

constexpr int kMsNW = 16;          // waves per workgroup
constexpr int kMsRing = 4;         // 64-dimension blocks in flight per wave
constexpr int kMsTilesPerWave = (kMaxSimMaxDocs / 32 + kMsNW - 1) / kMsNW;
constexpr uint32_t kOutOfRange = 0x80000000u;   // past any buffer: loads return 0

template <typename T, int NW, int RING>
__global__ __launch_bounds__(NW * 64) void maxsim_kernel(MaxSimParams p, int n_qb) {
  extern __shared__ __attribute__((aligned(16))) uint16_t Qs[];   // [32][D], swizzled
  __shared__ int16_t tlist[NW][kMsTilesPerWave];
  __shared__ uint32_t tmask[NW][kMsTilesPerWave];
  __shared__ float part[NW][32];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // blockIdx = (b_hi * n_qb + qb) * 8 + b_lo with b = 8 b_hi + b_lo
  const int x = __builtin_amdgcn_readfirstlane((int)blockIdx.x);
  const int b_lo = x & 7, y = x >> 3;
  const int b_hi = y / n_qb, qb = y - b_hi * n_qb;
  const int b = b_hi * 8 + b_lo;
  if (b >= p.B) return;                      // padding of the grid to whole groups of 8
  const int D = p.D, nch = D >> 3;           // 16-byte chunks per row
  const uint32_t rowb = (uint32_t)D * 2u;    // bytes per row
  const int n_dt = (p.Ld + 31) >> 5;         // document tiles
  const int n_mine = n_dt > w ? (n_dt - w + NW - 1) / NW : 0;   // tiles dealt to this wave

  // 1a. this wave's tiles, two per load: lanes 0-31 tile 2k, lanes 32-63 tile 2k+1
  //     (all validity loads are issued before the first ballot)
  bool okv[(kMsTilesPerWave + 1) / 2];
#pragma unroll
  for (int k = 0; k < (kMsTilesPerWave + 1) / 2; ++k) {
    okv[k] = false;
    if (2 * k < n_mine) {
      const int t = w + NW * (2 * k + (lane >> 5));
      const int j = t * 32 + (lane & 31);
      bool ok = 2 * k + (lane >> 5) < n_mine && j < p.Ld;
      if (ok && p.d_valid) ok = p.d_valid[(int64_t)b * p.Ld + j] != 0;
      okv[k] = ok;
    }
  }

  // 1b. query block -> LDS: physical chunk position pc of row r holds logical
  // chunk pc ^ swz(r); wave instruction i fills LDS bytes [1024 i, 1024 i + 1024)
  {
    const int q0 = qb * 32;
    const int rows = min(32, p.Lq - q0);
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc((const T *)p.q + ((int64_t)b * p.Lq + q0) * D, (uint32_t)rows * rowb);
    const int n_inst = D >> 4;               // 32 rows * D * 2 bytes / 1 KB
    for (int i = w; i < n_inst; i += NW) {
      const int pch = i * 64 + lane;
      const int r = pch / nch, pc = pch - r * nch;
      const uint32_t src = (uint32_t)r * rowb + (uint32_t)((pc ^ swz<128>(r)) << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rq, (__attribute__((address_space(3))) void *)(Qs + i * 512), 16, src, 0, 0, 0);
    }
  }

  // 1c. list the wave's tiles that hold a valid token (wave-private LDS)
  int my_tiles = 0;
#pragma unroll
  for (int k = 0; k < (kMsTilesPerWave + 1) / 2; ++k) {
    if (2 * k < n_mine) {
      const uint64_t bal = __ballot(okv[k]);
      const uint32_t mk[2] = {(uint32_t)bal, (uint32_t)(bal >> 32)};
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (mk[h]) {
          if (lane == 0) {
            tlist[w][my_tiles] = (int16_t)(w + NW * (2 * k + h));
            tmask[w][my_tiles] = mk[h];
          }
          ++my_tiles;
        }
    }
  }

  // 2. stream the wave's tiles
  const int nblk = D >> 6;                   // 64-dimension blocks per row
  const int total = my_tiles * nblk;
  const __amdgpu_buffer_rsrc_t rd =
      make_rsrc((const T *)p.d + (int64_t)b * p.Ld * D, (uint32_t)p.Ld * rowb);
  const int quad = lane >> 4, r16 = lane & 15;
  // document operand: row r16 of a 16-document group, 16 bytes at 16 quad
  const uint32_t lane_off = (uint32_t)r16 * rowb + (uint32_t)quad * 16u;

  // byte offset of the first row of the wave's ordinal-th listed tile (or past the end)
  auto tile_base = [&](int ordinal) -> uint32_t {
    if (ordinal >= my_tiles) return kOutOfRange;
    const int t = __builtin_amdgcn_readfirstlane((int)tlist[w][ordinal]);
    return (uint32_t)t * 32u * rowb;
  };

  // ring slot: operand (dg, t) at [2 dg + t] for document group dg, k-step t
  u32x4 ring[RING][4];
  int is_ord = 0, is_kb = 0;                 // issue side: tile ordinal, block
  uint32_t is_base = tile_base(0);
  auto issue = [&](u32x4 (&dst)[4]) __attribute__((always_inline)) {
    const uint32_t off = is_base + lane_off + (uint32_t)is_kb * 128u;
#pragma unroll
    for (int dg = 0; dg < 2; ++dg)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        dst[2 * dg + t] = buf_load16(rd, off + (uint32_t)dg * 16u * rowb + 64u * t);
    if (++is_kb == nblk) {
      is_kb = 0;
      is_base = tile_base(++is_ord);
    }
  };

#pragma unroll
  for (int s = 0; s < RING - 1; ++s) issue(ring[s]);
  vm_wait_barrier();                         // the query block is in LDS

  // accumulators (dg, qg): lane l holds query 16 qg + l % 16 and documents
  // 16 dg + 4 quad + i, i = 0..3
  f32x4 acc[2][2];
#pragma unroll
  for (int dg = 0; dg < 2; ++dg)
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) acc[dg][qg] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};      // per query group
  uint32_t q_row[2];
  int q_swz[2];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    q_row[qg] = (uint32_t)(16 * qg + r16) * rowb;
    q_swz[qg] = swz<128>(16 * qg + r16);
  }
  int c_ord = 0, c_kb = 0;                   // compute side

  for (int n0 = 0; n0 < total; n0 += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      issue(ring[(r + RING - 1) % RING]);
      if (n0 + r < total) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int c = c_kb * 8 + t * 4 + quad;
#pragma unroll
          for (int qg = 0; qg < 2; ++qg) {
            const u32x4 bq =
                *(const u32x4 *)((const char *)Qs + q_row[qg] + ((c ^ q_swz[qg]) << 4));
#pragma unroll
            for (int dg = 0; dg < 2; ++dg)
              acc[dg][qg] = Mfma16<T>::mac(ring[r][2 * dg + t], bq, acc[dg][qg]);
          }
        }
        if (++c_kb == nblk) {
          // tile done: masked max over its 32 documents, then start afresh
          const uint32_t vm = __builtin_amdgcn_readfirstlane(tmask[w][c_ord]);
#pragma unroll
          for (int dg = 0; dg < 2; ++dg)
#pragma unroll
            for (int qg = 0; qg < 2; ++qg)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int jj = 16 * dg + 4 * quad + i;
                if ((vm >> jj) & 1u) m[qg] = fmaxf(m[qg], acc[dg][qg][i]);
                acc[dg][qg][i] = 0.f;
              }
          c_kb = 0;
          ++c_ord;
        }
      }
    }
  }

  // 3. merge the four lanes of each query column, then the waves: lane q < 32
  //    ends up with query q's max
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    m[qg] = fmaxf(m[qg], __shfl_xor(m[qg], 16, 64));
    m[qg] = fmaxf(m[qg], __shfl_xor(m[qg], 32, 64));
  }
  if (lane < 32) part[w][lane] = lane < 16 ? m[0] : m[1];
  __syncthreads();
  if (w == 0 && lane < 32) {
    float rm = part[0][lane];
#pragma unroll
    for (int v = 1; v < NW; ++v) rm = fmaxf(rm, part[v][lane]);
    const int i = qb * 32 + lane;
    bool valid = i < p.Lq;
    if (valid && p.q_valid) valid = p.q_valid[(int64_t)b * p.Lq + i] != 0;
    if (!valid) rm = -INFINITY;
    if (i < p.Lq) p.rowmax[(int64_t)b * p.Lq + i] = rm;
    if (n_qb == 1) {
      // fixed-order tree over the 32 query tokens
      float sum = valid ? rm : 0.f;
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      if (lane == 0) p.score[b] = sum / (float)p.Lq;
    }
  }
}

// score[b] from rowmax when L_q is not a single block (L_q == 0 or L_q > 32).
constexpr int kRedThreads = 256;
__global__ __launch_bounds__(kRedThreads) void maxsim_score_kernel(MaxSimParams p) {
  __shared__ float red[kRedThreads];
  const int b = blockIdx.x, tid = threadIdx.x;
  float sum = 0.f;
  for (int i = tid; i < p.Lq; i += kRedThreads) {
    bool valid = true;
    if (p.q_valid) valid = p.q_valid[(int64_t)b * p.Lq + i] != 0;
    if (valid) sum += p.rowmax[(int64_t)b * p.Lq + i];
  }
  red[tid] = sum;
  __syncthreads();
#pragma unroll
  for (int o = kRedThreads / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) p.score[b] = p.Lq > 0 ? red[0] / (float)p.Lq : 0.f;
}

template <typename T>
hipError_t launch_t(const MaxSimParams &p, hipStream_t s) {
  const int n_qb = (p.Lq + 31) / 32;
  const int b_pad = (p.B + 7) / 8 * 8;
  if (n_qb > 0)
    hipLaunchKernelGGL((maxsim_kernel<T, kMsNW, kMsRing>), dim3((unsigned)(b_pad * n_qb)),
                       dim3(kMsNW * 64), (size_t)32 * p.D * 2, s, p, n_qb);
  if (n_qb != 1)
    hipLaunchKernelGGL(maxsim_score_kernel, dim3((unsigned)p.B), dim3(kRedThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_maxsim(const MaxSimParams &p, int dtype, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  if (dtype == FA_BF16) return launch_t<__bf16>(p, s);
  if (dtype == FA_F16) return launch_t<_Float16>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
