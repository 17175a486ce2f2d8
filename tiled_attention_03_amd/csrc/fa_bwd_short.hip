// Backward for short query blocks (S_q <= 32), bf16/f16, gfx950: dQ, dK and
// dV of one (batch, head) in one pass over its keys.
//
// The gradient of the FlashAttentionScore replacement guide, section 2
// (P recomputed from the saved row LSE, dP = dO V^T, dS = P * (dP - delta),
// dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K), for the late-interaction
// retrieval page's shape ("Layer 1 / Layer 2": a few dozen query tokens
// against hundreds of padded document tokens, many samples and heads).  The
// general backward splits the keys over workgroups of 128 and computes dQ in
// a second pass; with 32 query rows every one of those workgroups walks a
// single query block, and their fixed costs, not the bytes, set the time.
// Here one wave owns a (batch, head) and all of its 32 query rows, so it can
// finish every gradient itself, with no atomics:
//
//   * the Q and dO tiles and the rows' LSE and delta are loaded once into LDS;
//   * per 32-key tile: S = Q K^T and dP = dO V^T with the lane owning a key
//     (A = Q / dO rows from LDS, B = the tile's K rows from LDS and V rows
//     straight from HBM into operand registers), then P and dS per element;
//     dV^T += dO^T P and dK^T += Q^T dS (A = dO / Q read transposed from LDS,
//     B = P / dS from the accumulators), stored for the tile's keys at once;
//     dQ^T += K^T dS^T (A = K read transposed, B = dS passed through a 2 KB
//     LDS exchange so that the lane owns a query), kept for the whole pass;
//   * K tiles in three LDS slots and V tiles in three register sets, two in
//     flight ahead of the one computed; tiles without a valid key are not
//     loaded, their dK and dV rows are written as zeros.
//
// Handles what the short-query forward handles: S_q <= 32, S_k <= 2048,
// masks causal and padding, ALiBi or no bias, keep_prob = 1, and gradients
// in the input dtype; fa_bwd sends every other problem to the key and query
// passes.
#include <stdio.h>

#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int kBwdShortMaxTiles = 64;   // 32-key tiles the key-flag pass covers (one per lane)
constexpr int kXS = 40;                 // dS exchange: row stride (16-bit units) of a query's 32 keys

template <int D>
struct BwdShortCfg {
  static constexpr int NS = 3;          // K slots = V register sets: two tiles ahead
  static constexpr int KS = D / 16;     // k-steps over d
  static constexpr int DB = D / 32;     // 32-row blocks of d
  static constexpr int OCC = D == 64 ? 2 : 1;
  using G = TileGeom<D, 32, 1>;
  static constexpr int LPT = KS + G::NI;   // global load instructions per tile (V, then K)
};

template <typename T, int D>
__global__ __launch_bounds__(64, BwdShortCfg<D>::OCC) void bwd_short_kernel(Params p) {
  using C = BwdShortCfg<D>;
  constexpr int KS = C::KS, DB = C::DB, NS = C::NS;
  constexpr int ES = (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) uint16_t Qs[32 * D], Gs[32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t K0[32 * D], K1[32 * D], K2[32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t X[32 * kXS];
  __shared__ __attribute__((aligned(16))) float Ls[32], Ds[32];

  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh % p.H;
  const int l = threadIdx.x, g = l >> 5, lr = l & 31;
  const uint32_t flags = p.mask_flags;
  const bool causal = flags & FA_MASK_CAUSAL;
  const bool alibi = p.pse_kind == FA_PSE_ALIBI;

  const int64_t qoff = b * p.q_sb + h * p.q_sh, koff = b * p.k_sb + h * p.k_sh;
  const int64_t rbase = ((int64_t)b * p.H + h) * p.Sq;
  const auto Qr = make_rsrc((const T *)p.q + qoff, span_bytes(p.Sq, p.q_ss, D, ES));
  const auto Gr = make_rsrc((const T *)p.dout + qoff, span_bytes(p.Sq, p.q_ss, D, ES));
  const auto Kr = make_rsrc((const T *)p.k + koff, span_bytes(p.Sk, p.k_ss, D, ES));
  const auto Vr = make_rsrc((const T *)p.v + koff, span_bytes(p.Sk, p.k_ss, D, ES));
  const uint32_t krow_b = (uint32_t)(p.k_ss * ES), qrow_b = (uint32_t)(p.q_ss * ES);

  // Q and dO tiles (rows past S_q read as zeros), the rows' LSE (base 2) and delta
  {
    uint32_t vq[C::G::PER_WAVE];
    tile_offsets<D, 32, 1>(vq, qrow_b, 0, l);
    tile_load<D, 32, 1>(Qs, Qr, vq, 0u, 0);
    tile_load<D, 32, 1>(Gs, Gr, vq, 0u, 0);
  }
  if (l < 32) {
    const bool in = l < p.Sq;
    Ls[l] = in ? p.lse[rbase + l] * kLog2e : 0.f;
    Ds[l] = in ? p.delta[rbase + l] : 0.f;
  }

  const float c_log2 = p.scale_log2;
  const float sl2 = alibi ? p.alibi_slopes[h] * kLog2e : 0.f;

  uint32_t voff[C::G::PER_WAVE];
  tile_offsets<D, 32, 1>(voff, krow_b, 0, l);
  uint32_t ro[KS], to[2 * DB];
#pragma unroll
  for (int t = 0; t < KS; ++t) ro[t] = row_off<D>(lr, 2 * t + g);
#pragma unroll
  for (int db = 0; db < DB; ++db) tr_off<D>(&to[2 * db], 32 * db, l);

  // Issues the loads of tile t: V rows into register set S in the operand
  // layout (lane l: key l%32, eight consecutive d), K rows into LDS slot S.
  // t < 0 issues the same loads at offsets past the buffers' ends (zeros, no
  // memory touched, into a slot no later step reads), so every step has the
  // same loads in flight and the wait counts below are exact.
  u32x4 vr[NS][KS];
  auto issue_tile = [&](auto slot, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    const int j = 32 * t + lr;
    const uint32_t off = t >= 0 && j < p.Sk ? (uint32_t)((int64_t)j * p.k_ss * ES) : 0x80000000u;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) vr[S][kk] = buf_load16(Vr, off + (16 * kk + 8 * g) * ES);
    uint32_t vo[C::G::PER_WAVE];
#pragma unroll
    for (int k = 0; k < C::G::PER_WAVE; ++k) vo[k] = t >= 0 ? voff[k] : 0x80000000u;
    tile_load<D, 32, 1>(S == 0 ? K0 : S == 1 ? K1 : K2, Kr, vo,
                        t >= 0 ? (uint32_t)t * 32u * krow_b : 0u, 0);
  };

  // key range (rows < S_q see keys <= row under the causal rule) and, per
  // lane t, the bits of tile t's keys that exist, lie in the range and are valid
  const int k_hi = causal ? min(p.Sk, p.Sq) : p.Sk;
  const int nt = (k_hi + 31) >> 5;
  int tq[NS];
  tq[0] = nt > 0 ? 0 : -1;
  tq[1] = nt > 1 ? 1 : -1;
  tq[2] = -1;
  issue_tile(BufIdx<0>{}, tq[0]);
  issue_tile(BufIdx<1>{}, tq[1]);
  uint32_t kbits = 0u;
  if (l < nt) {
    const int rest = k_hi - 32 * l;
    kbits = rest >= 32 ? 0xffffffffu : (1u << rest) - 1u;
  }
  if (flags & FA_MASK_PADDING) {
    // 16-byte loads where the tile's flags lie wholly within the row and are
    // aligned, else independent byte loads (range-checked: zeros past S_k)
    const uint8_t *kvb = p.key_valid + (int64_t)b * p.Sk;
    const auto Fr = make_rsrc(kvb, (uint32_t)p.Sk);
    const uint32_t fo = 32u * (uint32_t)min(l, nt);
    uint32_t v = 0u;
    if (((uintptr_t)kvb & 15u) == 0 && 32 * l + 32 <= p.Sk) {
      const u32x4 f0 = buf_load16(Fr, fo), f1 = buf_load16(Fr, fo + 16u);
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const uint32_t word = e < 16 ? f0[e >> 2] : f1[(e - 16) >> 2];
        v |= (uint32_t)(((word >> (8 * (e & 3))) & 0xffu) != 0u) << e;
      }
    } else {
      uint8_t fb[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) fb[e] = __builtin_amdgcn_raw_buffer_load_b8(Fr, fo + e, 0, 0);
#pragma unroll
      for (int e = 0; e < 32; ++e) v |= (uint32_t)(fb[e] != 0) << e;
    }
    kbits &= v;
  }
  const uint64_t visited = __ballot(kbits != 0u);   // tiles with a valid key
  uint64_t rem = visited & ~3ull;                   // still to be issued (0 and 1 are out)
  const int n_tiles = min(nt, 2) + __builtin_popcountll(rem);
  auto pop = [&]() __attribute__((always_inline)) -> int {
    if (rem == 0ull) return -1;
    const int t = __builtin_ctzll(rem);
    rem &= rem - 1ull;
    return t;
  };

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

  T *dKg = (T *)p.dk + koff, *dVg = (T *)p.dv + koff;
  // one tile of keys: the lane owns key 32 t + lr of every product below
  auto compute = [&](auto slot, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    const uint16_t *ks = S == 0 ? K0 : S == 1 ? K1 : K2;
    // S = Q K^T and dP = dO V^T (queries x keys): register r holds query
    // 8 (r / 4) + 4 g + r % 4
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      s = Mfma<T>::mac(read_row_at<D>(Qs, 0, ro[kk]), read_row_at<D>(ks, 0, ro[kk]), s);
      dp = Mfma<T>::mac(read_row_at<D>(Gs, 0, ro[kk]), vr[S][kk], dp);
    }
    const int j = 32 * t + lr;
    const bool key_ok =
        (((uint32_t)__builtin_amdgcn_readlane((int)kbits, t) >> lr) & 1u) != 0u;
    f32x16 pv, dsv;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 lsa = *(const f32x4 *)(Ls + 8 * a + 4 * g);
      const f32x4 dsa = *(const f32x4 *)(Ds + 8 * a + 4 * g);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 4 * a + c, i = 8 * a + 4 * g + c;
        float x = s[r] * c_log2 - lsa[c];
        if (alibi) x -= sl2 * fabsf((float)(i - j));
        bool ok = key_ok && i < p.Sq;
        if (causal) ok = ok && j <= i;
        const float pe = ok ? exp2_fast(x) : 0.f;
        pv[r] = pe;
        dsv[r] = pe * (dp[r] - dsa[c]);
      }
    }
    u32x4 pk[2], dk16[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      pk[c] = pack8<T>(pv, 8 * c);
      dk16[c] = pack8<T>(dsv, 8 * c);
    }
    // dS through LDS so that a lane owns a query: X[i][key]
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int r = 8 * c + 2 * w;
        const int i0 = 8 * (r >> 2) + 4 * g + (r & 3);
        X[i0 * kXS + lr] = (uint16_t)(dk16[c][w] & 0xffffu);
        X[(i0 + 1) * kXS + lr] = (uint16_t)(dk16[c][w] >> 16);
      }
    // dV^T = dO^T P, dK^T = Q^T dS (d x keys): register r holds d = 32 db + 8 (r / 4) + 4 g + r % 4
    f32x16 dvt[DB], dkt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dvt[db] = dkt[db] = f32x16{};
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dvt[db] = Mfma<T>::mac(read_tr_at<D>(Gs, c, &to[2 * db]), pk[c], dvt[db]);
        dkt[db] = Mfma<T>::mac(read_tr_at<D>(Qs, c, &to[2 * db]), dk16[c], dkt[db]);
      }
    // dQ^T += K^T dS^T (d x queries): B = dS^T, lane l holds query l%32 and the
    // keys 16 c + 8 (s / 4) + 4 g + s % 4 of slot s (a wave's LDS operations
    // complete in order, so these reads see the writes above)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint16_t *xr = X + lr * kXS + 16 * c + 4 * g;
      const u32x2 lo = *(const u32x2 *)xr, hi = *(const u32x2 *)(xr + 8);
      const u32x4 xs = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int db = 0; db < DB; ++db) dq[db] = Mfma<T>::mac(read_tr_at<D>(ks, c, &to[2 * db]), xs, dq[db]);
    }
    // this tile's dK and dV rows
    if (j < p.Sk) {
      T *dvr = dVg + (int64_t)j * p.k_ss, *dkr = dKg + (int64_t)j * p.k_ss;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d0 = 32 * db + 8 * rr + 4 * g;
          u32x2 v, k;
          v[0] = pack2<T>(dvt[db][4 * rr + 0], dvt[db][4 * rr + 1]);
          v[1] = pack2<T>(dvt[db][4 * rr + 2], dvt[db][4 * rr + 3]);
          k[0] = pack2<T>(dkt[db][4 * rr + 0] * p.scale, dkt[db][4 * rr + 1] * p.scale);
          k[1] = pack2<T>(dkt[db][4 * rr + 2] * p.scale, dkt[db][4 * rr + 3] * p.scale);
          *(u32x2 *)(dvr + d0) = v;
          *(u32x2 *)(dkr + d0) = k;
        }
    }
  };

  // vmcnt(n) alone (expcnt and lgkmcnt at their maxima)
  auto wait_vm = [&](auto n) __attribute__((always_inline)) {
    constexpr int N = decltype(n)::value;
    static_assert(N < 64, "vmcnt holds six bits");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    asm volatile("" ::: "memory");   // no LDS read moves above the wait
    __builtin_amdgcn_sched_barrier(0);
  };

  // Step on slot S: issue the tile two places ahead into slot (S + 2) % NS,
  // wait until the tile of slot S (and everything issued before it: the Q and
  // dO tiles) has landed, compute it.  The slot being refilled was last read
  // by the previous step, whose products have consumed those reads.  Whole
  // rounds of NS steps, no exit inside a round.
  auto step = [&](auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    constexpr int SN = (S + 2) % NS;
    tq[SN] = pop();
    issue_tile(BufIdx<SN>{}, tq[SN]);
    wait_vm(std::integral_constant<int, 2 * C::LPT>{});
    if (tq[S] >= 0) compute(BufIdx<S>{}, tq[S]);
  };
  static_assert(NS == 3, "the loop below names three slots");
  for (int n = 0; n < n_tiles; n += NS) {
    step(BufIdx<0>{});
    step(BufIdx<1>{});
    step(BufIdx<2>{});
  }
  wait_vm(std::integral_constant<int, 0>{});   // no load into LDS outlives the workgroup

  // dK = dV = 0 for the keys of tiles that were not visited (no valid key,
  // or past the causal range); lane l writes 16 bytes of row 32 t + l / (D/8)
  {
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;           // rows per wave store
    const int nt_all = (p.Sk + 31) >> 5;
    for (int t = 0; t < nt_all; ++t) {
      if ((visited >> t) & 1ull) continue;
#pragma unroll
      for (int r0 = 0; r0 < 32; r0 += RPI) {
        const int j = 32 * t + r0 + l / CPR;
        if (j < p.Sk) {
          const int64_t o = (int64_t)j * p.k_ss + 8 * (l % CPR);
          *(u32x4 *)(dKg + o) = u32x4{0u, 0u, 0u, 0u};
          *(u32x4 *)(dVg + o) = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  }

  // dQ = scale dS K: lane l owns query l%32, register r holds d = 32 db + 8 (r / 4) + 4 g + r % 4
  if (lr < p.Sq) {
    T *dqr = (T *)p.dq + qoff + (int64_t)lr * p.q_ss;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * g;
        u32x2 v;
        v[0] = pack2<T>(dq[db][4 * rr + 0] * p.scale, dq[db][4 * rr + 1] * p.scale);
        v[1] = pack2<T>(dq[db][4 * rr + 2] * p.scale, dq[db][4 * rr + 3] * p.scale);
        *(u32x2 *)(dqr + d0) = v;
      }
  }
}

template <typename T, int D>
hipError_t launch_t(const Params &p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.B * p.H;
  if (blocks == 0) return hipSuccess;
  if (log_enabled()) {
    char name[96];
    snprintf(name, sizeof(name), "bwd_short_kernel<%s, D=%d>",
             std::is_same<T, __bf16>::value ? "bf16" : "f16", D);
    log_launch("fa_bwd", name, (long long)blocks, 64, p);
  }
  hipLaunchKernelGGL((bwd_short_kernel<T, D>), dim3((unsigned)blocks), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool bwd_short_fits(const Params &p, int dtype) {
  const uint32_t other = p.mask_flags & ~(uint32_t)(FA_MASK_CAUSAL | FA_MASK_PADDING);
  return (dtype == FA_BF16 || dtype == FA_F16) && (p.D == 64 || p.D == 128) && p.Sq >= 1 &&
         p.Sq <= 32 && p.Sk <= 32 * kBwdShortMaxTiles && !p.dropout && !p.grad_f32 &&
         !p.dpse && other == 0u && (p.pse_kind == FA_PSE_NONE || p.pse_kind == FA_PSE_ALIBI) &&
         (tile_override() == kTileAuto || tile_override() == kTileShort);
}

hipError_t launch_bwd_short(const Params &p, int dtype, hipStream_t s) {
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
