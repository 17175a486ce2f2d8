// Forward attention for short query blocks (S_q <= 32), bf16/f16, gfx950.
//
// The same operator as fa_fwd_kernel.h (FlashAttentionScore replacement
// guide, section 2: O = Softmax(Q K^T * scale + mask + pse) V with an online
// softmax over key tiles, and the row log-sum-exp), for the shape of the
// late-interaction retrieval page's scoring layer ("Layer 1 / Layer 2": a
// few dozen query tokens against hundreds of padded document tokens, many
// samples and heads).  There every (batch, head) reads its K and V rows once
// and does 4·D flops per pair with them: 64 flops per byte at 32 queries,
// far below the MFMA/HBM ridge, so the time is set by how many bytes are in
// flight, not by the matrix core.
//
// One wave per (batch, head), no lists and no cross-wave exchange:
//
//   * K rows go from HBM straight into MFMA operand registers (the A operand
//     of S^T = K . Q^T holds key l%32, eight consecutive d per lane), so only
//     V, which the P V product reads transposed, is staged in LDS.  A
//     workgroup needs 3 * 32 * D * 2 bytes of LDS (12 KB at D = 64), and a CU
//     holds twelve of them, three waves per SIMD.
//   * Tiles of 32 keys, two in flight ahead of the one being computed (K in
//     three register sets, V in three LDS slots, each named statically).
//   * Under a padding mask the wave reads the key flags of the whole range
//     (32 bytes per lane, lane t for tile t) and keeps, per lane, the
//     valid-key bits of its tile; tiles without a valid key are never loaded.
//   * Every tile takes the per-element rules (key flags, the causal rule,
//     ALiBi) from those bits and its indices.  Without the causal rule and
//     ALiBi, tiles past the first that sets the rows' running max take no max
//     (the optimistic reference above); a wave where a lane's check fails
//     computes its tiles again with the max on each.
//
// Tiles are visited from the first one up (the rows are positions 0..31, so
// under ALiBi the nearest keys come first).  Handles
// S_q <= 32, S_k <= 32 * kShortMaxTiles, masks causal and padding, ALiBi or no
// bias, keep_prob = 1; the launcher sends every other problem to
// fa_fwd_kernel.h.
#pragma once

#include <stdio.h>

#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int kShortMaxTiles = 64;   // 32-key tiles the key-flag pass covers (one per lane)
// Optimistic softmax reference (both forward kernels): once a row's running
// max is set, later tiles may skip the max and keep the reference, as long as
// every exponential stays <= 2^32 (then O and l stay far inside the fp32
// range).  Each lane checks that its share of a tile's sum of exponentials is
// at most kOptMax (so no element exceeds it); where one does not, the tiles
// are computed again with the max taken on every tile.  The reference is an
// actual score of the row, so no element that matters can underflow.
constexpr float kOptMax = 4294967296.f;   // 2^32

template <int D>
struct ShortCfg {
  static constexpr int P = 2;           // tiles in flight ahead of the one computed
  static constexpr int NS = P + 1;      // K register sets = V LDS slots
  static constexpr int KS = D / 16;     // k-steps of K Q^T
  static constexpr int DB = D / 32;     // 32-row blocks of O^T
  static constexpr int OCC = D == 64 ? 3 : 2;   // waves per SIMD the registers allow
  using G = TileGeom<D, 32, 1>;
  static constexpr int LPT = KS + G::NI;   // global load instructions per tile
};

template <typename T, int D>
__global__ __launch_bounds__(64, ShortCfg<D>::OCC) void fwd_short_kernel(Params p) {
  using C = ShortCfg<D>;
  constexpr int KS = C::KS, DB = C::DB, P = C::P, NS = C::NS;
  constexpr int ES = (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) uint16_t V0[32 * D], V1[32 * D], V2[32 * D];

  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh % p.H;
  const int l = threadIdx.x, g = l >> 5, i = l & 31;   // i: this lane's query row
  const uint32_t flags = p.mask_flags;
  const bool causal = flags & FA_MASK_CAUSAL;
  const bool alibi = p.pse_kind == FA_PSE_ALIBI;

  const T *Qg = (const T *)p.q + b * p.q_sb + h * p.q_sh;
  const T *Kg = (const T *)p.k + b * p.k_sb + h * p.k_sh;
  const T *Vg = (const T *)p.v + b * p.k_sb + h * p.k_sh;
  const auto Qr = make_rsrc(Qg, span_bytes(p.Sq, p.q_ss, D, ES));
  const auto Kr = make_rsrc(Kg, span_bytes(p.Sk, p.k_ss, D, ES));
  const auto Vr = make_rsrc(Vg, span_bytes(p.Sk, p.k_ss, D, ES));
  const uint32_t krow_b = (uint32_t)(p.k_ss * ES);

  // Q^T fragments (B operand), rows past S_q read as zeros
  u32x4 qf[KS];
  {
    const uint32_t qoff = i < p.Sq ? (uint32_t)((int64_t)i * p.q_ss * ES) : 0x80000000u;
#pragma unroll
    for (int t = 0; t < KS; ++t) qf[t] = buf_load16(Qr, qoff + (16 * t + 8 * g) * ES);
  }

  const float c_log2 = p.scale_log2;
  const float sl2 = alibi ? p.alibi_slopes[h] * kLog2e : 0.f;

  uint32_t voff[C::G::PER_WAVE];
  tile_offsets<D, 32, 1>(voff, krow_b, 0, l);
  uint32_t to[2 * DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) tr_off<D>(&to[2 * db], 32 * db, l);

  // Issues the loads of tile t into K set / V slot S; t < 0 issues the same
  // number of loads at offsets past the buffers' ends (they read zeros
  // without touching memory, and land in a slot no later step reads).  Every
  // step thus issues the same loads, so the wait counts below are exact and
  // the compiler's own count for the K registers is the same on every path.
  u32x4 kf[NS][KS];
  auto issue_tile = [&](auto slot, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    const int j = 32 * t + i;
    const uint32_t off = t >= 0 && j < p.Sk ? (uint32_t)((int64_t)j * p.k_ss * ES) : 0x80000000u;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kf[S][kk] = buf_load16(Kr, off + (16 * kk + 8 * g) * ES);
    uint32_t vo[C::G::PER_WAVE];
#pragma unroll
    for (int k = 0; k < C::G::PER_WAVE; ++k) vo[k] = t >= 0 ? voff[k] : 0x80000000u;
    tile_load<D, 32, 1>(S == 0 ? V0 : S == 1 ? V1 : V2, Vr, vo,
                        t >= 0 ? (uint32_t)t * 32u * krow_b : 0u, 0);
  };

  // key range; lane t < nt holds the bits of tile t's keys that exist, lie in
  // the range and are valid
  const int k_hi = causal ? min(p.Sk, p.Sq) : p.Sk;   // rows < S_q see keys <= row
  const int nt = (k_hi + 31) >> 5;
  // Tiles are visited from the first one up: the rows are positions 0..31, so
  // under ALiBi the nearest keys, with the largest logits, come first and the
  // running max settles at once.  The first two tiles are issued before the
  // key flags are read (under a padding mask valid keys usually start at 0),
  // so their loads and the flags' share one round trip; a tile that turns out
  // to hold no valid key is computed fully masked and adds nothing.
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
    // the 32 flags of tile l: two 16-byte loads where they lie wholly within
    // the row and are aligned, else 32 independent byte loads (range-checked:
    // flags past S_k read as zeros; a wider load that crosses the end of the
    // range would read as zeros as a whole)
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
  // tiles still to be issued, lowest first (0 and 1 are out already)
  uint64_t rem = __ballot(kbits != 0u) & ~3ull;
  const int n_tiles = min(nt, 2) + __builtin_popcountll(rem);
  auto pop = [&]() __attribute__((always_inline)) -> int {
    if (rem == 0ull) return -1;
    const int t = __builtin_ctzll(rem);
    rem &= rem - 1ull;
    return t;
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // one tile: S^T = K Q^T from registers, the per-element rules, online
  // softmax, O^T += V^T P^T.  Safe form: the lazy rescale (the reference max
  // moves only when a row's max grows by more than kShortTau).  Optimistic
  // form (OPT, neither the causal rule nor ALiBi, once every row of the wave
  // has a reference): no max, the reference stays, the key flags mask the
  // exponentials, and bad flags a lane whose share of the tile's sum passes
  // kOptMax.
  constexpr float kShortTau = 8.f;
  bool bad = false;
  auto compute = [&](auto slot, int t, auto opt) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    // the optimistic form at D = 64 only: at D = 128 its registers do not fit
    // two waves per SIMD without spills
    constexpr bool OPT = decltype(opt)::value && D <= 64;
    const uint16_t *vs = S == 0 ? V0 : S == 1 ? V1 : V2;
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) s = Mfma<T>::mac(kf[S][kk], qf[kk], s);
    // element r holds key 32 t + c + 4 g, c = 8 (r / 4) + r % 4
    const uint32_t kb = (uint32_t)__builtin_amdgcn_readlane((int)kbits, t) >> (4 * g);
    const int dj = 32 * t + 4 * g - i;   // key - row of element c = 0
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    float alpha = 1.f;
    if (OPT && !causal && !alibi && __all(m_run != -INFINITY)) {
      // p = exp2(s c - m), kept where the key flag bit is set: the bit,
      // sign-extended to 0 or all ones, masks p's bits (2 instructions)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 8 * (r >> 2) + (r & 3);
        const float x = exp2_fast(fmaf(s[r], c_log2, -m_run));
        const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)kb, c, 1);
        s[r] = __uint_as_float(__float_as_uint(x) & keep);
        part[r & 3] += s[r];
      }
    } else {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 8 * (r >> 2) + (r & 3);
        float x = s[r] * c_log2;
        if (alibi) x -= sl2 * fabsf((float)(dj + c));
        bool ok = (kb >> c) & 1u;
        if (causal) ok = ok && dj + c <= 0;
        x = ok ? x : -INFINITY;
        s[r] = x;
        mx = fmaxf(mx, x);
      }
      mx = max_lane_pair(mx);
      const bool grow = mx > m_run + kShortTau;
      if (grow) {
        alpha = exp2_fast(m_run - mx);
        m_run = mx;
      }
      if (__any(grow)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      }
      const float off = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = exp2_fast(s[r] - off);
        s[r] = x;
        part[r & 3] += x;
      }
    }
    const float tsum = (part[0] + part[1]) + (part[2] + part[3]);
    l_run = l_run * alpha + tsum;
    if (OPT) bad |= tsum > kOptMax;
    u32x4 pk[2];
    pk[0] = pack8<T>(s, 0);
    pk[1] = pack8<T>(s, 8);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 va[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) va[db] = read_tr_at<D>(vs, c, &to[2 * db]);
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = Mfma<T>::mac(va[db], pk[c], acc[db]);
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

  // Step on slot S: issue the tile P places ahead into slot (S + P) % NS,
  // wait until the tile of slot S has landed (the loads of the P tiles after
  // it may still be in flight), then compute it.  The slot being refilled was
  // last read by the previous step's P V products, which have consumed those
  // reads.  The loop runs whole rounds of NS steps with no exit inside a
  // round (steps past the last tile only issue and wait), so every step sees
  // the same loads in flight.
  auto step = [&](auto slot, auto opt) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    constexpr int SN = (S + P) % NS;
    tq[SN] = pop();
    issue_tile(BufIdx<SN>{}, tq[SN]);
    wait_vm(std::integral_constant<int, P * C::LPT>{});
    if (tq[S] >= 0) compute(BufIdx<S>{}, tq[S], opt);
  };
  static_assert(NS == 3, "the loop below names three slots");
  const uint64_t rem0 = rem;
  for (int n = 0; n < n_tiles; n += NS) {
    step(BufIdx<0>{}, std::true_type{});
    step(BufIdx<1>{}, std::true_type{});
    step(BufIdx<2>{}, std::true_type{});
  }
  wait_vm(std::integral_constant<int, 0>{});   // no load into LDS outlives the workgroup
  if (__any(bad)) {
    // an exponential of the optimistic pass reached kOptMax: every tile
    // again, the row max taken on each
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;
    rem = rem0;
    tq[0] = nt > 0 ? 0 : -1;
    tq[1] = nt > 1 ? 1 : -1;
    tq[2] = -1;
    issue_tile(BufIdx<0>{}, tq[0]);
    issue_tile(BufIdx<1>{}, tq[1]);
    for (int n = 0; n < n_tiles; n += NS) {
      step(BufIdx<0>{}, std::false_type{});
      step(BufIdx<1>{}, std::false_type{});
      step(BufIdx<2>{}, std::false_type{});
    }
    wait_vm(std::integral_constant<int, 0>{});
  }

  // epilogue: O = acc / l, LSE
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (i < p.Sq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T *Og = (T *)p.o + b * p.q_sb + h * p.q_sh + (int64_t)i * p.q_ss;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
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
      p.lse[((int64_t)b * p.H + h) * p.Sq + i] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Whether the short-query kernel covers the problem.
inline bool short_fits(const Params &p) {
  const uint32_t other = p.mask_flags & ~(uint32_t)(FA_MASK_CAUSAL | FA_MASK_PADDING);
  return p.Sq <= 32 && p.Sk <= 32 * kShortMaxTiles && !p.dropout && other == 0u &&
         (p.pse_kind == FA_PSE_NONE || p.pse_kind == FA_PSE_ALIBI);
}

template <typename T, int D>
hipError_t launch_short(const Params &p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.B * p.H;
  if (blocks == 0 || p.Sq == 0) return hipSuccess;
  if (log_enabled()) {
    char name[96];
    snprintf(name, sizeof(name), "fwd_short_kernel<%s, D=%d>",
             std::is_same<T, __bf16>::value ? "bf16" : "f16", D);
    log_launch("fa_fwd", name, (long long)blocks, 64, p);
  }
  hipLaunchKernelGGL((fwd_short_kernel<T, D>), dim3((unsigned)blocks), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace fa
