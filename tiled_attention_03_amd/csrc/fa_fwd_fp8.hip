// Forward pass with fp8 inputs (page 1, tuning section: pure fp8 as the
// experimental precision).  Q, K, V are OCP e4m3 bytes with per-tensor
// descale factors (value = byte * descale); O is bf16 and LSE float32, as for
// the 16-bit forward.
//
// Products run on gfx950's 32x32x64 fp8 MFMA (fp32 accumulation), whose two
// operands take the same lane layout: lane l supplies row (or column) l % 32
// and 32 consecutive bytes of the contraction for lane half l / 32.
//  * S^T = K Q^T: a K row and a Q row each give 32 contiguous bytes per
//    64-dimension k-step (row reads; Q stays in registers).
//  * O^T += V^T P^T: P^T comes from the lane's own score registers, rounded
//    to e4m3 (the lazy rescale keeps p = exp2(t - m_run) <= 2^8, inside
//    e4m3's range of 448; l sums the unrounded p).  A lane's 32 P values are
//    the keys 32 kb + 8 (r / 4) + 4 g + r % 4 of its half g, in register order;
//    V^T must present the same keys in the same order, so a pre-pass writes V
//    transposed and permuted per 64-key tile: byte 32 g + 16 kb + r of row d
//    holds V[key 32 kb + 8 (r / 4) + 4 g + r % 4][d].  Both operands are then
//    plain 32-byte row reads.
// The online softmax, the per-wave tile classes (dead / fast / general) and
// the mask and bias rules are those of the 16-bit forward; tiles are visited
// one per step with the next tile's loads in flight.
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kBN = 64;            // keys per tile
constexpr float kTau8 = 8.f;       // lazy rescale threshold (base-2 units)
enum : int { kFast8 = 0, kGen8 = 1, kDead8 = 2 };   // a wave's class of a tile

__device__ __forceinline__ f32x16 mac_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // scale bytes 127 = 2^0 (E8M0): the plain product
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16-byte chunk swizzles: K rows of D bytes, V^T rows of 64 bytes.  Each makes
// the 32-byte operand reads of 16 consecutive rows hit 16 distinct bank groups.
template <int D> __device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
__device__ __forceinline__ int swz_v(int r) { return (r >> 2) & 3; }

// The key held at byte position pos (0..63) of a permuted V^T tile row.
__device__ __forceinline__ int vt_key(int pos) {
  const int g = pos >> 5, kb = (pos >> 4) & 1, r = pos & 15;
  return 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
}

// N direct-to-LDS loads of 1 KB, wave load k into dst + 1024 (k * NW + w),
// lane offsets off[k] + base (the base in the per-lane offset, so that the
// buffer's range check turns rows past the end into zeros).
template <int N, int NW>
__device__ __forceinline__ void lds_loads(uint8_t *dst, __amdgpu_buffer_rsrc_t rs,
                                          const uint32_t (&off)[N], uint32_t base, int w) {
#pragma unroll
  for (int k = 0; k < N; ++k)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void *)(dst + 1024 * (k * NW + w)), 16,
        off[k] + base, 0, 0, 0);
}

// Pre-pass: V [keys][D] (bytes) -> per 64-key tile, V^T [D][64] permuted.
template <int D>
__global__ __launch_bounds__(256) void vt_prep_kernel(Params p, int n_kt) {
  __shared__ __attribute__((aligned(16))) uint8_t vb[kBN * D];
  const int kt = blockIdx.x % n_kt, bh = blockIdx.x / n_kt;
  const int b = bh / p.H, h = bh % p.H;
  const uint8_t *Vg = (const uint8_t *)p.v + b * p.k_sb + h * p.k_sh;
  const auto Vr = make_rsrc(Vg, span_bytes(p.Sk, p.k_ss, D, 1));
  const int tid = threadIdx.x;
  for (int c = tid; c < kBN * D / 16; c += 256) {
    const int key = c / (D / 16), part = c % (D / 16);
    const int j = kt * kBN + key;
    const uint32_t off = j < p.Sk ? (uint32_t)((int64_t)j * p.k_ss + 16 * part) : 0x80000000u;
    *(u32x4 *)(vb + key * D + 16 * part) = buf_load16(Vr, off);
  }
  __syncthreads();
  uint8_t *dst = (uint8_t *)p.vt + ((int64_t)bh * n_kt + kt) * D * kBN;
  for (int c = tid; c < D * kBN / 16; c += 256) {
    const int d = c >> 2, q = c & 3;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t x = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) x |= (uint32_t)vb[vt_key(16 * q + 4 * e + t) * D + d] << (8 * t);
      w[e] = x;
    }
    *(u32x4 *)(dst + d * kBN + 16 * q) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void fwd_fp8_kernel(Params p, int n_qtiles, int n_kt) {
  constexpr int BM = 32 * NW;       // query rows per workgroup
  constexpr int KS = D / 64;        // k-steps of S^T
  constexpr int DB = D / 32;        // 32-row blocks of O^T
  constexpr int KI = kBN * D / 1024 / NW;   // K tile: 1 KB wave loads per wave
  constexpr int VI = D * kBN / 1024 / NW;   // V^T tile: likewise
  static_assert(KI >= 1 && VI >= 1, "tile must split over the waves");
  __shared__ __attribute__((aligned(16))) uint8_t K0[kBN * D], K1[kBN * D], K2[kBN * D];
  __shared__ __attribute__((aligned(16))) uint8_t V0[D * kBN], V1[D * kBN], V2[D * kBN];
  __shared__ int kv_range[2];

  const int BH = p.B * p.H;
  const int lin = blockIdx.x;
  const int qt = n_qtiles - 1 - lin / BH;   // longest causal rows first
  const int bh = lin % BH;
  const int b = bh / p.H, h = bh % p.H;
  const int q0 = qt * BM;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, g = l >> 5, lr = l & 31;
  const int qw = q0 + 32 * w;
  const int my_i = qw + lr;
  const uint32_t flags = p.mask_flags;
  const bool causal = flags & FA_MASK_CAUSAL;
  const bool f_pad = flags & FA_MASK_PADDING, f_mod = flags & FA_MASK_MODALITY;
  const bool f_exp = flags & FA_MASK_EXPLICIT;
  const bool alibi = p.pse_kind == FA_PSE_ALIBI;
  const bool dense = p.pse_kind == FA_PSE_DENSE;

  // ---- key range of this workgroup
  int k_lo = 0, k_hi = p.Sk;
  if (causal) k_hi = min(k_hi, q0 + BM);
  if (f_pad) {
    if (tid == 0) { kv_range[0] = p.Sk; kv_range[1] = 0; }
    __syncthreads();
    int lo = p.Sk, hi = 0;
    const uint8_t *kv = p.key_valid + (int64_t)b * p.Sk;
    for (int j = tid; j < p.Sk; j += NW * 64) {
      if (kv[j]) { lo = min(lo, j); hi = max(hi, j + 1); }
    }
    atomicMin(&kv_range[0], lo);
    atomicMax(&kv_range[1], hi);
    __syncthreads();
    k_lo = max(k_lo, kv_range[0]);
    k_hi = min(k_hi, kv_range[1]);
  }
  const int kt_begin = __builtin_amdgcn_readfirstlane(k_lo / kBN);
  const int kt_end =
      __builtin_amdgcn_readfirstlane(k_hi > k_lo ? (k_hi + kBN - 1) / kBN : k_lo / kBN);

  const uint8_t *Qg = (const uint8_t *)p.q + b * p.q_sb + h * p.q_sh;
  const uint8_t *Kg = (const uint8_t *)p.k + b * p.k_sb + h * p.k_sh;
  const uint8_t *Vt = (const uint8_t *)p.vt + (int64_t)bh * n_kt * D * kBN;
  const auto Qr = make_rsrc(Qg, span_bytes(p.Sq, p.q_ss, D, 1));
  const auto Kr = make_rsrc(Kg, span_bytes(p.Sk, p.k_ss, D, 1));
  const auto Vtr = make_rsrc(Vt, (uint32_t)(n_kt * D * kBN));
  const uint32_t krow = (uint32_t)p.k_ss;

  // ---- Q operand: row my_i, bytes 64 ks + 32 g .. + 31 (rows past S_q read as zeros)
  i32x8 qf[KS];
  {
    const uint32_t qoff = my_i < p.Sq ? (uint32_t)((int64_t)my_i * p.q_ss) : 0x80000000u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 a = buf_load16(Qr, qoff + 64 * ks + 32 * g);
      const u32x4 c = buf_load16(Qr, qoff + 64 * ks + 32 * g + 16);
      qf[ks] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                     (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
    }
  }

  // ---- tile loads straight into LDS (lane l of a wave load fills bytes 16 l of its 1 KB)
  uint32_t koff[KI], voff[VI];
#pragma unroll
  for (int k = 0; k < KI; ++k) {
    const int pb = 1024 * (k * NW + w) + 16 * l;       // physical byte in the tile
    const int row = pb / D, pc = (pb % D) >> 4;
    koff[k] = (uint32_t)row * krow + (uint32_t)((pc ^ swz_k<D>(row)) << 4);
  }
#pragma unroll
  for (int k = 0; k < VI; ++k) {
    const int pb = 1024 * (k * NW + w) + 16 * l;
    const int row = pb / kBN, pc = (pb % kBN) >> 4;
    voff[k] = (uint32_t)row * kBN + (uint32_t)((pc ^ swz_v(row)) << 4);
  }
  auto load_tile = [&](int kt, uint8_t *kd, uint8_t *vd) __attribute__((always_inline)) {
    lds_loads<KI, NW>(kd, Kr, koff, (uint32_t)kt * kBN * krow, w);
    lds_loads<VI, NW>(vd, Vtr, voff, (uint32_t)kt * D * kBN, w);
  };

  // per-lane LDS byte offsets of the operand reads (chunk c of the lane's row)
  auto read32 = [&](const uint8_t *base, int row, int rowb, int c0, int sw)
                    __attribute__((always_inline)) {
    const u32x4 a = *(const u32x4 *)(base + row * rowb + ((c0 ^ sw) << 4));
    const u32x4 c = *(const u32x4 *)(base + row * rowb + (((c0 + 1) ^ sw) << 4));
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                 (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c_log2 = p.scale_log2 * p.fp8_qk;     // raw score -> base-2 logit
  const float sl2 = alibi ? p.alibi_slopes[h] * kLog2e : 0.f;

  auto step = [&](int kt, auto buf) __attribute__((always_inline)) {
    constexpr int B = decltype(buf)::value;
    const uint8_t *ks = B ? K1 : K0;
    const uint8_t *vs = B ? V1 : V0;
    if (kt + 1 < kt_end) load_tile(kt + 1, B ? K0 : K1, B ? V0 : V1);
    const int k0 = kt * kBN;
    int cls = qw < p.Sq ? kFast8 : kDead8;
    if (dense || f_exp || f_pad || f_mod || k0 + kBN > p.Sk) cls = max(cls, (int)kGen8);
    if (causal) {
      if (k0 > qw + 31) cls = kDead8;
      else if (k0 + kBN - 1 > qw) cls = max(cls, (int)kGen8);
    }
    // ALiBi on a tile wholly below (+1) or above (-1) the diagonal of this
    // wave's rows is linear in the key: -slope |i - j| = adir * slope (j - i)
    float adir = 0.f;
    if (alibi && cls == kFast8) {
      if (k0 + kBN - 1 <= qw) adir = 1.f;
      else if (k0 >= qw + 31) adir = -1.f;
      else cls = kGen8;
    }
    if (cls != kDead8) {
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks_ = 0; ks_ < KS; ++ks_) {
        i32x8 ka[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = 32 * kb + lr;
          ka[kb] = read32(ks, row, D, 4 * ks_ + 2 * g, swz_k<D>(row));
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = mac_fp8(ka[kb], qf[ks_], s[kb]);
      }
      // base-2 logits, masks and bias; element r of block kb is key
      // k0 + 32 kb + 8 (r / 4) + 4 g + r % 4 of row my_i
      float mx = -INFINITY;
      // fast ALiBi: t = c s + a (k0 + 32 kb + 8 (r / 4) + 4 g + r % 4 - i), a = adir * slope
      const float a2 = adir * sl2;
      const float abase = a2 * (float)(k0 + 4 * g - my_i);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float t = s[kb][r] * c_log2;
          if (cls == kFast8 && alibi)
            t += fmaf(a2, (float)(32 * kb + 8 * (r >> 2) + (r & 3)), abase);
          if (cls == kGen8) {
            const int j = k0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
            bool ok = j < p.Sk && my_i < p.Sq;
            if (ok) ok = allowed_elem(p, b, h, my_i, j);
            if (ok) {
              if (alibi) t -= sl2 * fabsf((float)(my_i - j));
              else if (dense) t += dense_bias(p, b, h, my_i, j) * kLog2e;
            } else {
              t = -INFINITY;
            }
          }
          s[kb][r] = t;
          mx = fmaxf(mx, t);
        }
      mx = max_lane_pair(mx);
      float alpha = 1.f;
      const bool grow = mx > m_run + kTau8;
      if (grow) {
        alpha = exp2_fast(m_run - mx);
        m_run = mx;
      }
      if (__any(grow)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      }
      const float off = m_run == -INFINITY ? 0.f : m_run;
      float part = 0.f;
      i32x8 pk;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          float x[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            x[t] = exp2_fast(s[kb][4 * rq + t] - off);
            part += x[t];
          }
          int wd = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
          wd = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], wd, true);
          pk[4 * kb + rq] = wd;
        }
      l_run = l_run * alpha + part;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 32 * db + lr;
        const i32x8 va = read32(vs, row, kBN, 2 * g, swz_v(row));
        acc[db] = mac_fp8(va, pk, acc[db]);
      }
    }
    vm_wait_barrier();
  };

  // ---- fast range [kt_begin, f_end): full tiles that need no per-element work
  // in any wave of the workgroup, with one ALiBi direction (below every row).
  // Only without mask tensors and dense bias; the other tiles run `step`.
  int f_end = kt_begin;
  // (the fast form folds slope / c into raw scores, which needs c > 0)
  if (!dense && !f_exp && !f_pad && !f_mod && (!alibi || c_log2 > kRawMinC)) {
    f_end = min(kt_end, p.Sk / kBN);                          // full tiles
    if (causal || alibi) f_end = min(f_end, (q0 + 1) / kBN);   // k0 + 63 <= q0
    f_end = max(f_end, kt_begin);
  }
  f_end = __builtin_amdgcn_readfirstlane(f_end);

  // generic tiles [f_end, kt_end), one per step
  if (f_end < kt_end) load_tile(f_end, K0, V0);
  vm_wait_barrier();
  {
    int kt = f_end;
    for (; kt + 1 < kt_end; kt += 2) {
      step(kt, BufIdx<0>{});
      step(kt + 1, BufIdx<1>{});
    }
    if (kt < kt_end) step(kt, BufIdx<0>{});
  }

  // ---- pipelined fast phase over [kt_begin, f_end): step n computes the
  // scores of tile n+1 (MFMA) interleaved with tile n's exponentials (VALU),
  // then tile n's P V (MFMA) interleaved with tile n+1's logits and row max.
  // Three buffers: tile n (P V), tile n+1 (scores), tile n+2 (loading).
  const int n_fast = f_end - kt_begin;
  // Fast tiles lie below every row (ALiBi direction +1).  Their scores stay in
  // raw units with the key-dependent part of the bias added, u = s + ar * jr
  // (jr = 32 kb + 8 (r / 4) + r % 4, a per-register constant; ar = slope / c):
  // the base-2 logit is c u + lane_base with lane_base = slope (k0 + 4 g - i),
  // which the max and the exponent's argument take as a per-lane constant.
  const float ar = alibi ? sl2 / c_log2 : 0.f;
  float lane_base = 0.f;                // of the tile whose scores sit in the other register set
  auto fold = [&](f32x16 (&sc)[2], int k0) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float u = fmaf(ar, (float)(32 * kb + 8 * (r >> 2) + (r & 3)), sc[kb][r]);
        sc[kb][r] = u;
        mx = fmaxf(mx, u);
      }
    lane_base = (alibi ? sl2 : 0.f) * (float)(k0 + 4 * g - my_i);
    return max_lane_pair(fmaf(mx, c_log2, lane_base));
  };
  auto rescale = [&](float mx) __attribute__((always_inline)) {
    const bool grow = mx > m_run + kTau8;
    float alpha = 1.f;
    if (grow) {
      alpha = exp2_fast(m_run - mx);
      m_run = mx;
    }
    l_run *= alpha;
    if (__any(grow)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
  };
  auto kbuf = [&](auto bi) -> uint8_t * {
    constexpr int B = decltype(bi)::value;
    return B == 0 ? K0 : (B == 1 ? K1 : K2);
  };
  auto vbuf = [&](auto bi) -> uint8_t * {
    constexpr int B = decltype(bi)::value;
    return B == 0 ? V0 : (B == 1 ? V1 : V2);
  };
  auto fast_step = [&](int n, auto cur, auto nxt, auto ld, f32x16 (&sc)[2], f32x16 (&sn)[2])
                       __attribute__((always_inline)) {
    const bool has_next = n + 1 < n_fast;
    if (n + 2 < n_fast) load_tile(kt_begin + n + 2, kbuf(ld), vbuf(ld));
    // operands of the next tile's scores, all read up front
    i32x8 ka[KS][2];
    if (has_next) {
#pragma unroll
      for (int t = 0; t < KS; ++t)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = 32 * kb + lr;
          ka[t][kb] = read32(kbuf(nxt), row, D, 4 * t + 2 * g, swz_k<D>(row));
        }
    }
    // exponent argument of element u: c u + (lane_base - m_run)
    const float off = lane_base - (m_run == -INFINITY ? 0.f : m_run);
    float part = 0.f;
    i32x8 pk;
    constexpr int NG = 2 * KS;        // score MFMAs of the next tile
    constexpr int EPG = 8 / NG;       // packed dwords (4 probabilities each) per group
    static_assert(NG * EPG == 8, "the 8 packed dwords split over the groups");
    sn[0] = f32x16{};
    sn[1] = f32x16{};
    // the MFMA-dense part at raised issue priority: the other workgroup's wave on
    // this SIMD fills the gaps with its VALU work
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      if (has_next) sn[gi & 1] = mac_fp8(ka[gi >> 1][gi & 1], qf[gi >> 1], sn[gi & 1]);
#pragma unroll
      for (int e = 0; e < EPG; ++e) {
        const int dw = gi * EPG + e, kb = dw >> 2, rq = dw & 3;
        float x[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          x[t] = exp2_fast(fmaf(sc[kb][4 * rq + t], c_log2, off));
          part += x[t];
        }
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], wd, true);
        pk[dw] = wd;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += part;
    // P V of this tile, then the next tile's logits, max and rescale
    i32x8 va[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int row = 32 * db + lr;
      va[db] = read32(vbuf(cur), row, kBN, 2 * g, swz_v(row));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = mac_fp8(va[db], pk, acc[db]);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    if (has_next) rescale(fold(sn, (kt_begin + n + 1) * kBN));
    vm_wait_barrier();
  };
  if (n_fast > 0) {
    load_tile(kt_begin, K0, V0);
    if (n_fast > 1) load_tile(kt_begin + 1, K1, V1);
    vm_wait_barrier();
    f32x16 sA[2] = {f32x16{}, f32x16{}}, sB[2];
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * kb + lr;
        sA[kb] = mac_fp8(read32(K0, row, D, 4 * t + 2 * g, swz_k<D>(row)), qf[t], sA[kb]);
      }
    rescale(fold(sA, kt_begin * kBN));
    for (int n = 0; n < n_fast; n += 6) {
      fast_step(n, BufIdx<0>{}, BufIdx<1>{}, BufIdx<2>{}, sA, sB);
      if (n + 1 < n_fast) fast_step(n + 1, BufIdx<1>{}, BufIdx<2>{}, BufIdx<0>{}, sB, sA);
      if (n + 2 < n_fast) fast_step(n + 2, BufIdx<2>{}, BufIdx<0>{}, BufIdx<1>{}, sA, sB);
      if (n + 3 < n_fast) fast_step(n + 3, BufIdx<0>{}, BufIdx<1>{}, BufIdx<2>{}, sB, sA);
      if (n + 4 < n_fast) fast_step(n + 4, BufIdx<1>{}, BufIdx<2>{}, BufIdx<0>{}, sA, sB);
      if (n + 5 < n_fast) fast_step(n + 5, BufIdx<2>{}, BufIdx<0>{}, BufIdx<1>{}, sB, sA);
    }
  }

  // ---- O = acc * v_descale / l (bf16) and LSE
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (my_i < p.Sq) {
    const float inv = l_tot > 0.f ? p.fp8_v / l_tot : 0.f;
    __bf16 *Og = (__bf16 *)p.o + b * p.q_sb + h * p.q_sh + (int64_t)my_i * p.q_ss;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * g;
        u32x2 v;
        v[0] = pack2<__bf16>(acc[db][4 * rr + 0] * inv, acc[db][4 * rr + 1] * inv);
        v[1] = pack2<__bf16>(acc[db][4 * rr + 2] * inv, acc[db][4 * rr + 3] * inv);
        *(u32x2 *)(Og + d0) = v;
      }
    }
    if (g == 0)
      p.lse[((int64_t)b * p.H + h) * p.Sq + my_i] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const Params &p, hipStream_t s) {
  constexpr int NW = 4;
  const int n_kt = (p.Sk + kBN - 1) / kBN;
  if (n_kt > 0)
    hipLaunchKernelGGL((vt_prep_kernel<D>), dim3((unsigned)((int64_t)n_kt * p.B * p.H)), dim3(256),
                       0, s, p, n_kt);
  const int n_qtiles = (p.Sq + 32 * NW - 1) / (32 * NW);
  const int64_t blocks = (int64_t)n_qtiles * p.B * p.H;
  if (blocks > 0)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, NW>), dim3((unsigned)blocks), dim3(NW * 64), 0, s, p,
                       n_qtiles, n_kt);
  return hipGetLastError();
}

}  // namespace

size_t fwd_fp8_workspace_bytes(const Params &p) {
  const int64_t n_kt = (p.Sk + kBN - 1) / kBN;
  return (size_t)((int64_t)p.B * p.H * n_kt * p.D * kBN);
}

hipError_t launch_fwd_fp8(const Params &p, hipStream_t s) {
  if (p.D == 64) return launch_d<64>(p, s);
  if (p.D == 128) return launch_d<128>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
