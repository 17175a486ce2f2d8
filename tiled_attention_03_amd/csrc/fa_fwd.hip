// Forward attention, bf16/f16 inputs, MFMA on gfx950 (CDNA4).
//
// What is computed: O = Softmax(Q K^T * scale + mask + pse) V and the row
// log-sum-exp, tile by tile with an online softmax so the S_q x S_k score
// matrix never leaves registers (FlashAttentionScore replacement guide,
// section 2; the tile loop and running statistics are the "tiling + online
// softmax" of its section 1 and of the NPU FlashAttention study's flow
// description).
//
// Workgroup = NW waves; each wave owns 32 query rows, so BM = 32*NW rows per
// workgroup share one stream of K/V tiles of BN = 64 keys.  The products are
// arranged so that a lane owns ONE query row for the whole kernel:
//
//   S^T (keys x queries) = K . Q^T     v_mfma_f32_32x32x16, A = K from LDS,
//                                      B = Q^T kept in VGPRs (loaded once)
//   O^T (d x queries)   += V^T . P^T   A = V^T from LDS, B = P^T straight
//                                      from the S^T accumulators
//
// With the 32x32 accumulator layout (lane l, register r holds row
// 8*(r/4) + 4*(l/32) + r%4, column l%32), lane l holds query l%32 and half of
// the tile's keys; the other half sits in lane l^32.  Row max and row sum
// therefore need a single cross-lane exchange per tile, and the running
// statistics and the O rescale are per-lane scalars.  The P^T operand of
// the second product is the first product's accumulators rounded to 16 bits
// in place; the V^T operand comes from the row-major V tile through gfx950's
// transposing LDS read, in the key order those accumulators hold.
//
// Softmax runs in the base-2 domain: t = s * scale * log2(e) + bias * log2(e),
// p = exp2(t - m); LSE = ln(2) * (m + log2(l)).
//
// K/V tiles are double-buffered in LDS: tile n+1 is loaded from global memory
// straight into LDS (no register staging) while tile n is multiplied; one
// barrier per tile.  Tiles use the swizzled layout of fa_tile.h.
//
// Tiles with nothing visible are not visited: the causal rule bounds the
// tile range, key padding bounds it by the first/last valid key of the
// sample, and a wave whose 32 rows see none of a tile's keys skips its
// MFMAs.  Per-element mask work happens only on tiles that need it.
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int BN = 64;          // keys per tile
constexpr int kMaxTiles = 512;  // key-tile summaries kept in LDS (S_k <= 32768)
constexpr float kTau = 8.f;     // rescale O only when a row max grows by more than this (log2)

template <typename T, int D, int NW>
struct FwdCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = 32 * NW;
  static constexpr int KS = D / 16;        // k-steps of Q K^T
  static constexpr int DB = D / 32;        // 32-row blocks of O^T
};

template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void fwd_mfma_kernel(Params p, int n_qtiles) {
  using C = FwdCfg<T, D, NW>;
  __shared__ __attribute__((aligned(16))) uint16_t K0[BN * D], K1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t V0[BN * D], V1[BN * D];
  __shared__ int kv_range[2];
  __shared__ uint32_t tsum[kMaxTiles];  // per key tile: bits 0-7 modality set of valid keys,
                                        // bit 8 some key invalid or past S_k

  const int BH = p.B * p.H;
  const int lin = blockIdx.x;
  const int qt = n_qtiles - 1 - lin / BH;   // longest causal rows first
  const int bh = lin % BH;
  const int b = bh / p.H, h = bh % p.H;
  const int q0 = qt * C::BM;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 5, lr = l & 31;
  const int qw = q0 + 32 * w;
  const int my_i = qw + lr;
  const uint32_t flags = p.mask_flags;
  const bool causal = flags & FA_MASK_CAUSAL;

  const T *Qg = (const T *)p.q + b * p.q_sb + h * p.q_sh;
  const T *Kg = (const T *)p.k + b * p.k_sb + h * p.k_sh;
  const T *Vg = (const T *)p.v + b * p.k_sb + h * p.k_sh;

  // ---- key range of this workgroup
  int k_lo = 0, k_hi = p.Sk;
  if (causal) k_hi = min(k_hi, q0 + C::BM);
  if (flags & FA_MASK_PADDING) {
    if (tid == 0) { kv_range[0] = p.Sk; kv_range[1] = 0; }
    __syncthreads();
    int lo = p.Sk, hi = 0;
    const uint8_t *kv = p.key_valid + (int64_t)b * p.Sk;
    for (int j = tid; j < p.Sk; j += C::NT) {
      if (kv[j]) { lo = min(lo, j); hi = max(hi, j + 1); }
    }
    atomicMin(&kv_range[0], lo);
    atomicMax(&kv_range[1], hi);
    __syncthreads();
    k_lo = max(k_lo, kv_range[0]);
    k_hi = min(k_hi, kv_range[1]);
  }
  const int kt_begin = k_lo / BN;
  const int kt_end = k_hi > k_lo ? (k_hi + BN - 1) / BN : kt_begin;

  constexpr int ES = (int)sizeof(T);
  const auto Qr = make_rsrc(Qg, span_bytes(p.Sq, p.q_ss, D, ES));
  const auto Kr = make_rsrc(Kg, span_bytes(p.Sk, p.k_ss, D, ES));
  const auto Vr = make_rsrc(Vg, span_bytes(p.Sk, p.k_ss, D, ES));
  const uint32_t krow_b = (uint32_t)(p.k_ss * ES);   // bytes between K/V rows

  // ---- Q^T fragments (B operand), one row per lane, loaded once (rows past
  // S_q read as zeros)
  u32x4 qf[C::KS];
  {
    const uint32_t qoff = my_i < p.Sq ? (uint32_t)((int64_t)my_i * p.q_ss * ES) : 0x80000000u;
#pragma unroll
    for (int t = 0; t < C::KS; ++t) qf[t] = buf_load16(Qr, qoff + (16 * t + 8 * g) * ES);
  }

  const bool alibi = p.pse_kind == FA_PSE_ALIBI;
  const bool dense = p.pse_kind == FA_PSE_DENSE;
  const float c_log2 = p.scale_log2;
  const float sl2 = alibi ? p.alibi_slopes[h] * kLog2e : 0.f;   // slope in log2 units
  const float sl2c = alibi ? sl2 / c_log2 : 0.f;                 // slope in raw-score units
  const bool f_pad = flags & FA_MASK_PADDING, f_mod = flags & FA_MASK_MODALITY;
  const bool f_exp = flags & FA_MASK_EXPLICIT;

  // ---- per key tile summaries (padding / modality), one wave-wide vote per tile
  const int n_kt_all = (p.Sk + BN - 1) / BN;
  const bool use_summary = (f_pad || f_mod) && n_kt_all <= kMaxTiles;
  uint32_t allow_any = 0, allow_all = 0xffu;   // over the modalities of this wave's rows
  if (use_summary) {
    for (int kt = w; kt < n_kt_all; kt += NW) {
      const int j = kt * BN + l;
      bool valid = j < p.Sk;
      int m = 0;
      if (valid && f_pad) valid = p.key_valid[(int64_t)b * p.Sk + j] != 0;
      if (valid && f_mod) m = p.kmod[(int64_t)b * p.Sk + j];
      uint32_t bits = __ballot(!valid) ? 0x100u : 0u;
      if (f_mod) {
        for (int mm = 0; mm < p.num_modalities; ++mm)
          if (__ballot(valid && m == mm)) bits |= 1u << mm;
      } else if (__ballot(valid)) {
        bits |= 1u;
      }
      if (l == 0) tsum[kt] = bits;
    }
    if (f_mod) {
      const int mq = my_i < p.Sq ? p.qmod[(int64_t)b * p.Sq + my_i] : -1;
      for (int mm = 0; mm < p.num_modalities; ++mm) {
        if (__ballot(mq == mm)) {
          const uint32_t row = (uint32_t)(p.allow_bits >> (8 * mm)) & 0xffu;
          allow_any |= row;
          allow_all &= row;
        }
      }
    }
    __syncthreads();
  }

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- K and V tiles straight into LDS; rows past S_k read as zeros.
  // Key tiles are walked from the last one down: under ALiBi the largest
  // logits (the keys nearest the diagonal) come first, so the running max
  // settles early and the lazy rescale below rarely fires.
  uint32_t voff[TileGeom<D, BN, NW>::PER_WAVE];
  tile_offsets<D, BN, NW>(voff, krow_b, w, l);
  auto gload = [&](int kt, uint16_t *kdst, uint16_t *vdst) {
    const uint32_t base = (uint32_t)kt * BN * krow_b;
    tile_load<D, BN, NW>(kdst, Kr, voff, base, w);
    tile_load<D, BN, NW>(vdst, Vr, voff, base, w);
  };

  if (kt_begin < kt_end) gload(kt_end - 1, K0, V0);
  vm_wait_barrier();

  // per-lane LDS byte offsets: K rows (A operand of S^T) and V^T reads
  uint32_t ro[C::KS], to[2 * C::DB];
#pragma unroll
  for (int t = 0; t < C::KS; ++t) ro[t] = row_off<D>(lr, 2 * t + g);
#pragma unroll
  for (int db = 0; db < C::DB; ++db) tr_off<D>(&to[2 * db], 32 * db, l);

  // one key tile held in buffer B; the next tile goes into the other buffer
  auto tile_step = [&](int kt, auto buf) {
    constexpr int B = decltype(buf)::value;
    uint16_t *ks = B ? K1 : K0;
    uint16_t *vs = B ? V1 : V0;
    if (kt > kt_begin) gload(kt - 1, B ? K0 : K1, B ? V0 : V1);
    opaque(ro);
    opaque(to);
    const int k0 = kt * BN;

    // ---- wave-level tile class: skip, fast (no per-element work) or general
    bool skip = qw >= p.Sq;
    bool general = dense || f_exp || (k0 + BN > p.Sk);
    if (causal) {
      if (k0 > qw + 31) skip = true;
      else if (k0 + BN - 1 > qw) general = true;
    }
    int adir = 0;   // ALiBi on a tile wholly below (+1) or above (-1) the diagonal
    if (alibi) {
      if (k0 + BN - 1 <= qw) adir = 1;
      else if (k0 >= qw + 31) adir = -1;
      else general = true;
    }
    if (use_summary) {
      const uint32_t ts = tsum[kt];
      const uint32_t kset = ts & 0xffu;
      if (f_mod) {
        const bool diag = p.allow_diag && k0 < qw + 32 && k0 + BN > qw;
        if ((kset & allow_any) == 0 && !diag) skip = true;
        if ((kset & ~allow_all) != 0 || diag) general = true;
      } else if (kset == 0) {
        skip = true;
      }
      if (ts & 0x100u) general = true;
    } else if (f_pad || f_mod) {
      general = true;
    }

    if (!skip) {
      // S^T = K . Q^T for two 32-key blocks
      f32x16 s[2] = {f32x16{}, f32x16{}};
      // operand reads in batches ahead of their MFMAs (the scheduling fence
      // keeps the LDS latency from being exposed on each product)
#pragma unroll
      for (int t0 = 0; t0 < C::KS; t0 += 4) {
        u32x4 ka[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int jb = 0; jb < 2; ++jb) ka[t][jb] = read_row_at<D>(ks, 32 * jb, ro[t0 + t]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int jb = 0; jb < 2; ++jb) s[jb] = Mfma<T>::mac(ka[t][jb], qf[t0 + t], s[jb]);
      }
      // Logit of element r of block jb is  t = cs * s + lane_off  (base-2 units).
      // Fast tiles: cs = scale*log2(e), the ALiBi term split into a per-register
      // constant (folded into s) and a per-lane constant lane_off.
      // General tiles: s already holds t (cs = 1, lane_off = 0), -inf where masked.
      float cs = c_log2, lane_off = 0.f, mx = -INFINITY;
      if (!general) {
        if (adir != 0) {
          const float a = adir * sl2c;
#pragma unroll
          for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              s[jb][r] = fmaf(a, (float)(32 * jb + 8 * (r >> 2) + (r & 3)), s[jb][r]);
          lane_off = adir * sl2 * (float)(k0 + 4 * g - my_i);
        }
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[jb][r]);
        mx = fmaf(mx, cs, lane_off);
      } else {
        cs = 1.f;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = k0 + 32 * jb + 8 * (r >> 2) + 4 * g + (r & 3);
            float t = s[jb][r] * c_log2;
            bool ok = j < p.Sk && my_i < p.Sq;
            if (ok) ok = allowed_elem(p, b, h, my_i, j);
            if (ok) {
              if (alibi) t -= sl2 * fabsf((float)(my_i - j));
              else if (dense) t += dense_bias(p, b, h, my_i, j) * kLog2e;
            } else {
              t = -INFINITY;
            }
            s[jb][r] = t;
            mx = fmaxf(mx, t);
          }
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // lazy rescale: the reference max moves only when a row max grows by > kTau;
      // exp2(t - m_run) then stays <= 2^kTau and O, l share the same reference.
      const bool grow = mx > m_run + kTau;
      float alpha = 1.f;
      if (grow) {
        alpha = exp2_fast(m_run - mx);
        m_run = mx;
      }
      if (__any(grow)) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
      }
      const float off = lane_off - (m_run == -INFINITY ? 0.f : m_run);
      float rs = 0.f;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = exp2_fast(fmaf(s[jb][r], cs, off));
          s[jb][r] = e;
          rs += e;
        }
      }
      l_run = l_run * alpha + rs;
      // O^T += V^T . P^T over four 16-key chunks
#pragma unroll
      for (int c = 0; c < BN / 16; ++c) {
        const u32x4 pk = pack8<T>(s[c >> 1], 8 * (c & 1));
        u32x4 va[C::DB];
#pragma unroll
        for (int db = 0; db < C::DB; ++db) va[db] = read_tr_at<D>(vs, c, &to[2 * db]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc[db] = Mfma<T>::mac(va[db], pk, acc[db]);
      }
    }
    vm_wait_barrier();
  };
  int kt = kt_end - 1;
  for (; kt > kt_begin; kt -= 2) {
    tile_step(kt, BufIdx<0>{});
    tile_step(kt - 1, BufIdx<1>{});
  }
  if (kt == kt_begin) tile_step(kt, BufIdx<0>{});

  // ---- epilogue: O = acc / l, LSE
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (my_i < p.Sq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T *Og = (T *)p.o + b * p.q_sb + h * p.q_sh + (int64_t)my_i * p.q_ss;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * g;
        u32x2 v;
        v[0] = pack2<T>(acc[db][4 * rr + 0] * inv, acc[db][4 * rr + 1] * inv);
        v[1] = pack2<T>(acc[db][4 * rr + 2] * inv, acc[db][4 * rr + 3] * inv);
        *(u32x2 *)(Og + d0) = v;
      }
    }
    if (g == 0)
      p.lse[((int64_t)b * p.H + h) * p.Sq + my_i] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D, int NW>
hipError_t launch_t(const Params &p, hipStream_t s) {
  using C = FwdCfg<T, D, NW>;
  const int n_qtiles = (p.Sq + C::BM - 1) / C::BM;
  const int64_t blocks = (int64_t)n_qtiles * p.B * p.H;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_mfma_kernel<T, D, NW>), dim3((unsigned)blocks), dim3(C::NT), 0, s, p,
                     n_qtiles);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const Params &p, hipStream_t s) {
  const bool small_q = p.Sq <= 32;
  if (p.D == 64) return small_q ? launch_t<T, 64, 1>(p, s) : launch_t<T, 64, 4>(p, s);
  if (p.D == 128) return small_q ? launch_t<T, 128, 1>(p, s) : launch_t<T, 128, 4>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_mfma(const Params &p, int dtype, hipStream_t s) {
  if (dtype == FA_BF16) return launch_dtype<__bf16>(p, s);
  if (dtype == FA_F16) return launch_dtype<_Float16>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
