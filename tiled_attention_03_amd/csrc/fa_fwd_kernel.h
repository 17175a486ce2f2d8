// Forward attention, bf16/f16 inputs, MFMA on gfx950 (CDNA4).
//
// What is computed: O = Softmax(Q K^T * scale + mask + pse) V and the row
// log-sum-exp, tile by tile with an online softmax so the S_q x S_k score
// matrix never leaves registers (FlashAttentionScore replacement guide,
// section 2; the tile loop and running statistics are the "tiling + online
// softmax" of its section 1 and of the NPU FlashAttention study's flow
// description).
//
// Workgroup = NW waves, each owning RB blocks of 32 query rows (the tile
// table at the end of this file: RB = 1, NW = 4 with 64-key tiles, two
// workgroups and so two waves per SIMD; S_q <= 32 takes one-wave workgroups,
// with 32-key tiles at D = 64 and three waves per SIMD).  The workgroup's
// BM = 32*RB*NW rows share one stream of K/V tiles of BN = 32*KBN keys.  The
// products are arranged so that a lane owns one query row of each block for
// the whole kernel:
//
//   S^T (keys x queries) = K . Q^T     v_mfma_f32_32x32x16, A = K from LDS,
//                                      B = Q^T kept in registers
//   O^T (d x queries)   += V^T . P^T   A = V^T from LDS, B = P^T straight
//                                      from the S^T accumulators
//
// With the 32x32 accumulator layout (lane l, register r holds row
// 8*(r/4) + 4*(l/32) + r%4, column l%32), lane l holds query l%32 and half of
// the tile's keys; the other half sits in lane l^32.  Row max and row sum
// need one cross-lane exchange per tile; the running statistics and the O
// rescale are per-lane scalars.  The P^T operand is the score accumulators
// rounded to 16 bits in place; the V^T operand comes from the row-major V
// tile through gfx950's transposing LDS read.
//
// Softmax runs in the base-2 domain: t = s * scale * log2(e) + bias * log2(e),
// p = exp2(t - m); LSE = ln(2) * (m + log2(l)).  The online softmax does not
// depend on the order in which key tiles are visited.
//
// Two phases.  The workgroup first sorts its key tiles: "fast" tiles need no
// per-element work for any of its rows (wholly visible under the causal rule,
// within S_k, ALiBi on one side of the diagonal, every key valid and of a
// modality all rows may attend, an explicit mask allowing every pair); the
// rest are "generic" (the causal diagonal band, the S_k tail, partly masked
// tiles, dense bias, ...).  Tiles no row can see are dropped.  The summaries
// behind this come from one pass of wave votes over the key flags (padding,
// modality) and a scan of the workgroup's explicit-mask rows.
//
//   generic phase: one tile per step; each wave classifies the tile for its
//     own rows (nothing visible: skip; no element work: fast; else per-element
//     mask and bias) and runs  S = K Q^T, softmax, O += P V  in sequence.
//   fast phase: a software pipeline with no branches on the tile class.  Step
//     n computes the scores of tile n+1 (MFMA) interleaved with the
//     exponentials of tile n (VALU), in an order fixed by scheduling fences,
//     then multiplies P_n by V_n; K tiles are fetched two steps ahead and V
//     tiles one step ahead.  Past its first two tiles the phase takes no row
//     max (the reference stays at an actual score of the row); each lane
//     checks its share of every tile's sum of exponentials against a bound
//     far inside the fp32 range, and a workgroup where one does not hold
//     runs both phases again with the max taken on every tile.
//
// Tiles go straight from global memory into LDS (no register staging).  Each
// of the four tile buffers is its own LDS variable and steps are unrolled in
// pairs, so every LDS read names its buffer statically and never waits for
// the loads in flight to the others.  Within each phase, tiles are visited
// from the last one down: under ALiBi the largest logits (keys nearest the
// diagonal) come first, so the running max settles early and the lazy
// rescale rarely fires.
#pragma once

#include <stdio.h>

#include "fa_fwd_short.h"
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

// Key tiles summarised and sorted in LDS lists: at most this many (S_k up to
// 64 * kMaxTiles); longer key ranges run the LONG instance, without lists.
constexpr int kMaxTiles = 1024;
constexpr int kMaxTilesSmall = 128;   // the one-wave (S_q <= 32) instance: less LDS per workgroup
constexpr float kTau = 8.f;     // rescale O only when a row max grows by more than this (log2)
// After its first two tiles the fast phase takes no row max (kOptMax, in
// fa_fwd_short.h, bounds what it may then meet); a workgroup where a lane's
// check fails runs its tiles again with the max taken on every tile.

template <typename T, int D, int NW, int RB_, int KBN_>
struct FwdCfg {
  static constexpr int NT = NW * 64;
  static constexpr int KBN = KBN_;         // 32-key blocks per tile
  static constexpr int BN = 32 * KBN;      // keys per tile
  static constexpr int RB = RB_;           // 32-row blocks per wave
  static constexpr int WR = 32 * RB;       // query rows per wave
  // waves per SIMD the registers allow: the one-wave instance at D = 64 (32-key
  // tiles, small lists) fits three workgroups' waves in a SIMD's registers
  static constexpr int OCC = RB == 1 ? (NW == 1 && D == 64 ? 3 : 2) : 1;
  static constexpr int LT = NW == 1 ? kMaxTilesSmall : kMaxTiles;   // tiles the LDS lists hold
  static constexpr int BM = WR * NW;       // query rows per workgroup
  static constexpr int KS = D / 16;        // k-steps of Q K^T
  static constexpr int DB = D / 32;        // 32-row blocks of O^T
};

// Tile class for one wave: what the wave does with the tile's scores.
enum : int { kFast = 0, kGeneral = 1, kDead = 2 };

// DROP: dropout compiled in (keep_prob < 1); without it the kernel carries no
// dropout code.
// FOLD: ALiBi without the causal rule (fast tiles of both directions fold the
// bias per element); the other problems run the FOLD = false instance, whose
// fast tiles take the bias as the score accumulators' start value.
// LONG: the key range may hold more tiles than the LDS lists (kMaxTiles); every
// tile then runs in the generic phase, from the top down, each wave taking the
// unmasked fast form where its class allows.
template <typename T, int D, int NW, int RB_, int KBN_, bool DROP, bool FOLD, bool LONG>
__global__ __launch_bounds__(NW * 64, (FwdCfg<T, D, NW, RB_, KBN_>::OCC))
void fwd_mfma_kernel(Params p, int n_qtiles) {
  using C = FwdCfg<T, D, NW, RB_, KBN_>;
  constexpr int KS = C::KS, DB = C::DB, RB = C::RB, WR = C::WR, KBN = C::KBN, BN = C::BN;
  constexpr int NC = BN / 16;   // 16-key chunks of a tile
  __shared__ __attribute__((aligned(16))) uint16_t K0[BN * D], K1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t V0[BN * D], V1[BN * D];
  __shared__ int kv_range[2];
  __shared__ uint32_t wg_any, wg_all;   // modalities some / every row of the workgroup may attend
  __shared__ int n_list[2];             // generic tiles, all visited tiles
  __shared__ uint32_t tsum[C::LT];  // per key tile: bits 0-7 modality set of valid keys,
                                        // bit 8 some key invalid or past S_k, bit 9 the
                                        // explicit mask allows some (row, key) of the
                                        // workgroup, bit 10 it hides some
  __shared__ int16_t tlist[C::LT];  // generic tiles, then fast tiles
  __shared__ uint32_t fpair[C::LT]; // fast tiles n and n+1 in one word (0 past the end)

  const int BH = p.B * p.H;
  const int lin = blockIdx.x;
  const int qt = n_qtiles - 1 - lin / BH;   // longest causal rows first
  const int bh = lin % BH;
  const int b = bh / p.H, h = bh % p.H;
  const int q0 = qt * C::BM;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int l = tid & 63, g = l >> 5, lr = l & 31;
  const int qw = q0 + WR * w;   // first row of this wave
  int my_i[RB];                 // this lane's row in each block
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) my_i[rb] = qw + 32 * rb + lr;
  const uint32_t flags = p.mask_flags;
  const bool causal = flags & FA_MASK_CAUSAL;

  const T *Qg = (const T *)p.q + b * p.q_sb + h * p.q_sh;
  const T *Kg = (const T *)p.k + b * p.k_sb + h * p.k_sh;
  const T *Vg = (const T *)p.v + b * p.k_sb + h * p.k_sh;

  // ---- key range of this workgroup: the causal rule here; under a padding
  // mask the tiles holding the first and last valid key narrow it further
  // (below, from the tile summaries; the LONG instance scans the keys)
  int k_lo = 0, k_hi = p.Sk;
  if (causal) k_hi = min(k_hi, q0 + C::BM);
  if ((flags & FA_MASK_PADDING) && LONG) {
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
  int kt_begin = k_lo / BN;
  int kt_end = k_hi > k_lo ? (k_hi + BN - 1) / BN : kt_begin;

  constexpr int ES = (int)sizeof(T);
  const auto Qr = make_rsrc(Qg, span_bytes(p.Sq, p.q_ss, D, ES));
  const auto Kr = make_rsrc(Kg, span_bytes(p.Sk, p.k_ss, D, ES));
  const auto Vr = make_rsrc(Vg, span_bytes(p.Sk, p.k_ss, D, ES));
  const uint32_t krow_b = (uint32_t)(p.k_ss * ES);   // bytes between K/V rows

  // ---- Q^T fragments (B operand), one row per lane, loaded once (rows past
  // S_q read as zeros)
  u32x4 qf[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = my_i[rb];
    const uint32_t qoff = i < p.Sq ? (uint32_t)((int64_t)i * p.q_ss * ES) : 0x80000000u;
#pragma unroll
    for (int t = 0; t < KS; ++t) qf[rb][t] = buf_load16(Qr, qoff + (16 * t + 8 * g) * ES);
  }

  const bool alibi = p.pse_kind == FA_PSE_ALIBI;
  const bool dense = p.pse_kind == FA_PSE_DENSE;
  const float c_log2 = p.scale_log2;
  const float sl2 = alibi ? p.alibi_slopes[h] * kLog2e : 0.f;   // slope in log2 units
  const float sl2c = alibi ? sl2 / c_log2 : 0.f;                 // slope in raw-score units
  const bool raw_ok = !alibi || c_log2 > kRawMinC;   // the fast forms fold sl2c into raw scores
  // fast tiles: the ALiBi column term enters as the start value of the score
  // accumulators (causal rule) or per element (fold_pe: ALiBi without it)
  static_assert(KBN <= 2, "the exponentials' block offsets cover two 32-key blocks");
  constexpr bool fold_pe = FOLD;   // the launcher sets FOLD = ALiBi without the causal rule
  const float ash = alibi && !FOLD ? sl2c : 0.f;
  const bool f_pad = flags & FA_MASK_PADDING, f_mod = flags & FA_MASK_MODALITY;
  const bool f_exp = flags & FA_MASK_EXPLICIT;

  // ---- per key tile summaries (padding / modality: one wave-wide vote per
  // tile; explicit mask: a scan of the workgroup's mask rows); modalities the
  // rows of this wave (and of the workgroup) may attend
  const bool use_summary = (f_pad || f_mod) && !LONG;
  uint32_t allow_any = 0, allow_all = 0xffu;
  if (tid == 0) { wg_any = 0u; wg_all = 0xffu; kv_range[0] = kt_end; kv_range[1] = kt_begin - 1; }
  int t_first = kt_end, t_last = kt_begin - 1;   // this wave's tiles holding a valid key
  if (use_summary) {
    // wave w votes on tiles w, w + NW, ...; the key loads of eight tiles are
    // issued before any vote, so the pass costs one load round trip per eight
    // of this wave's tiles
    constexpr int U = 8;
    for (int kt0 = kt_begin + w; kt0 < kt_end; kt0 += U * NW) {
      bool valid[U];
      int mk[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = (kt0 + u * NW) * BN + l;
        valid[u] = l < BN && kt0 + u * NW < kt_end && j < p.Sk;
        mk[u] = 0;
        if (valid[u] && f_pad) valid[u] = p.key_valid[(int64_t)b * p.Sk + j] != 0;
        if (valid[u] && f_mod) mk[u] = p.kmod[(int64_t)b * p.Sk + j];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kt = kt0 + u * NW;
        if (kt >= kt_end) break;
        const bool in_tile = l < BN;   // a tile may be narrower than the wave
        uint32_t bits = __ballot(in_tile && !valid[u]) ? 0x100u : 0u;
        if (f_mod) {
          for (int mm = 0; mm < p.num_modalities; ++mm)
            if (__ballot(valid[u] && mk[u] == mm)) bits |= 1u << mm;
        } else if (__ballot(valid[u])) {
          bits |= 1u;
        }
        if (__ballot(valid[u])) {
          t_first = min(t_first, kt);
          t_last = max(t_last, kt);
        }
        if (l == 0) tsum[kt] = bits;
      }
    }
  }
  if (use_summary && f_mod) {
    for (int rb = 0; rb < RB; ++rb) {
      const int i = my_i[rb];
      const int mq = i < p.Sq ? p.qmod[(int64_t)b * p.Sq + i] : -1;
      for (int mm = 0; mm < p.num_modalities; ++mm) {
        if (__ballot(mq == mm)) {
          const uint32_t row = (uint32_t)(p.allow_bits >> (8 * mm)) & 0xffu;
          allow_any |= row;
          allow_all &= row;
        }
      }
    }
  }
  __syncthreads();
  if (l == 0 && use_summary) {
    if (f_mod) {
      atomicOr(&wg_any, allow_any);
      atomicAnd(&wg_all, allow_all);
    }
    if (f_pad) {
      atomicMin(&kv_range[0], t_first);
      atomicMax(&kv_range[1], t_last);
    }
  }
  __syncthreads();
  if (use_summary && f_pad) {   // tiles past the last valid key, or before the first, are out
    const int t0 = __builtin_amdgcn_readfirstlane(kv_range[0]);
    const int t1 = __builtin_amdgcn_readfirstlane(kv_range[1]);
    kt_end = t1 >= t0 ? t1 + 1 : kt_begin;
    kt_begin = t1 >= t0 ? t0 : kt_begin;
  }
  if (f_exp && !LONG && kt_end > kt_begin) {
    // explicit mask over the workgroup's rows [q0, q_end) and each tile's keys
    // (< S_k): bit 9 if some pair is allowed, bit 10 if some pair is hidden.
    // 16-byte reads when the rows allow them (aligned, S_k a multiple of 16 so
    // that no read crosses the end of the range, and the workgroup's rows
    // within a 32-bit buffer range from row q0), else one byte per lane.
    const int q_end = min(q0 + C::BM, p.Sq);
    const uint8_t *emb = p.em + (int64_t)b * p.em_sb + (int64_t)h * p.em_sh;
    const int64_t em_sq = p.em_sq;
    const int64_t em_span = (int64_t)(q_end - 1 - q0) * em_sq + p.Sk;
    const bool em_vec = ((uintptr_t)emb & 15u) == 0 && (em_sq & 15) == 0 && (p.Sk & 15) == 0 &&
                        em_span < ((int64_t)1 << 31);
    const auto Er = make_rsrc(em_vec ? emb + (int64_t)q0 * em_sq : nullptr,
                              em_vec ? (uint32_t)em_span : 0u);
    if (!use_summary) {   // the padding / modality summary did not write tsum
      for (int kt = kt_begin + tid; kt < kt_end; kt += C::NT) tsum[kt] = 0u;
    }
    __syncthreads();
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      const int k0 = kt * BN;
      bool any = false, hid = false;
      if (em_vec) {
        constexpr int LPR = BN / 16, RPI = 64 / LPR;
        const int kk = k0 + 16 * (l % LPR);
        for (int i = q0 + w * RPI + l / LPR; i < q_end; i += NW * RPI) {
          const u32x4 wv = buf_load16(Er, (uint32_t)((int64_t)(i - q0) * em_sq + kk));
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            if (kk + e < p.Sk) {
              const bool a = (wv[e >> 2] >> (8 * (e & 3))) & 0xffu;
              any |= a;
              hid |= !a;
            }
          }
        }
      } else if (l < BN && k0 + l < p.Sk) {
        for (int i = q0 + w; i < q_end; i += NW) {
          const bool a = emb[(int64_t)i * em_sq + k0 + l] != 0;
          any |= a;
          hid |= !a;
        }
      }
      const uint32_t eb = (__ballot(any) ? 0x200u : 0u) | (__ballot(hid) ? 0x400u : 0u);
      if (l == 0 && eb) atomicOr(&tsum[kt], eb);
    }
    __syncthreads();
  }

  // ---- tile lists.  Workgroup-level class of tile kt: 0 not visited,
  // 1 generic, 2 fast (no per-element work for any wave of the workgroup, or
  // a causal-band tile whose only per-element work is the causal rule: the
  // fast phase masks those, and they come first in it).
  static_assert(C::BM <= 2 * BN, "the fast phase masks at most its first two tiles");
  const bool band_fast = causal && c_log2 > 0.f && !f_pad && !f_mod;
  auto wg_class = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * BN;
    const uint32_t ts = tsum[kt];
    bool fast = raw_ok && !dense && !DROP && k0 + BN <= p.Sk;
    if (causal && k0 + BN - 1 > q0) fast = fast && band_fast;
    else if (alibi && !(k0 + BN - 1 <= q0 || (!causal && k0 >= q0 + C::BM - 1))) fast = false;
    if (f_exp) {
      if (!(ts & 0x200u)) return 0;
      if (ts & 0x400u) fast = false;
    }
    if (f_pad || f_mod) {
      if (!use_summary) return 1;
      const uint32_t kset = ts & 0xffu;
      const bool diag = f_mod && p.allow_diag && k0 < q0 + C::BM && k0 + BN > q0;
      if (f_mod ? ((kset & wg_any) == 0 && !diag) : kset == 0) return 0;
      if (ts & 0x100u) fast = false;
      if (f_mod && ((kset & ~wg_all) != 0 || diag)) fast = false;
    }
    return fast ? 2 : 1;
  };
  if (w == 0 && !LONG) {
    int cnt = 0;
    for (int pass = 1; pass <= 2; ++pass) {   // generic tiles first, then fast ones
      for (int base = kt_end - 1; base >= kt_begin; base -= 64) {
        const int kt = base - l;
        const bool take = kt >= kt_begin && wg_class(kt) == pass;
        const uint64_t m = __ballot(take);
        const int pos = cnt + __builtin_popcountll(m & ((1ull << l) - 1ull));
        if (take) tlist[pos] = (int16_t)kt;
        cnt += __builtin_popcountll(m);
      }
      if (l == 0) n_list[pass - 1] = cnt;
    }
  }
  __syncthreads();
  // every lane reads the same entries; readfirstlane makes that visible to
  // the compiler (tile load offsets must be scalar)
  const int n_gen = LONG ? kt_end - kt_begin : __builtin_amdgcn_readfirstlane(n_list[0]);
  const int n_all = LONG ? n_gen : __builtin_amdgcn_readfirstlane(n_list[1]);
  auto tile_at = [&](int n) __attribute__((always_inline)) {
    return LONG ? kt_end - 1 - n : __builtin_amdgcn_readfirstlane((int)tlist[n]);
  };

  f32x16 acc[RB][DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[rb][db] = f32x16{};
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) { m_run[rb] = -INFINITY; l_run[rb] = 0.f; }

  // ---- tile loads straight into LDS; rows past S_k read as zeros
  uint32_t voff[TileGeom<D, BN, NW>::PER_WAVE];
  tile_offsets<D, BN, NW>(voff, krow_b, w, l);
  auto load_tile = [&](int kt, uint16_t *dst, __amdgpu_buffer_rsrc_t rs)
                       __attribute__((always_inline)) {
    tile_load<D, BN, NW>(dst, rs, voff, (uint32_t)kt * BN * krow_b, w);
  };

  // per-lane LDS byte offsets: K rows (A operand of S^T) and V^T reads
  uint32_t ro[KS], to[2 * DB];
#pragma unroll
  for (int t = 0; t < KS; ++t) ro[t] = row_off<D>(lr, 2 * t + g);
#pragma unroll
  for (int db = 0; db < DB; ++db) tr_off<D>(&to[2 * db], 32 * db, l);

  // S^T of one tile (two 32-key blocks) for every row block; operand reads
  // batched ahead of the MFMAs, each read feeding RB products
  auto scores = [&](const uint16_t *ks, f32x16 (&s)[RB][KBN], const f32x16 &init)
                    __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < KBN; ++kb) s[rb][kb] = init;
#pragma unroll
    for (int t0 = 0; t0 < KS; t0 += 4) {
      u32x4 ka[4][KBN];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) ka[t][kb] = read_row_at<D>(ks, 32 * kb, ro[t0 + t]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            s[rb][kb] = Mfma<T>::mac(ka[t][kb], qf[rb][t0 + t], s[rb][kb]);
    }
  };

  // O^T += V^T . P^T over the tile's four 16-key chunks
  auto pv = [&](const uint16_t *vs, const u32x4 (&pk)[RB][NC]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < BN / 16; ++c) {
      u32x4 va[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) va[db] = read_tr_at<D>(vs, c, &to[2 * db]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb][db] = Mfma<T>::mac(va[db], pk[rb][c], acc[rb][db]);
    }
  };

  // lazy rescale: the reference max of a row moves only when its max mx
  // (already combined over the lane pair) grows by more than kTau;
  // exp2(t - m_run) then stays <= 2^kTau and O, l share the same reference.
  // Leaves in alpha the factors that rescale l.
  auto update_max = [&](const float (&mx)[RB], float (&alpha)[RB]) __attribute__((always_inline)) {
    bool grow_any = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bool grow = mx[rb] > m_run[rb] + kTau;
      alpha[rb] = 1.f;
      if (grow) {
        alpha[rb] = exp2_fast(m_run[rb] - mx[rb]);
        m_run[rb] = mx[rb];
      }
      grow_any |= grow;
    }
    if (__any(grow_any)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[rb][db] *= alpha[rb];
    }
  };

  // ==== generic phase: one tile per step, per-wave class
  auto generic_step = [&](int n, auto buf) __attribute__((always_inline)) {
    constexpr int B = decltype(buf)::value;
    const uint16_t *ks = B ? K1 : K0;
    const uint16_t *vs = B ? V1 : V0;
    opaque(ro);
    opaque(to);
    if (n + 1 < n_gen) {
      const int kn = tile_at(n + 1);
      load_tile(kn, B ? K0 : K1, Kr);
      load_tile(kn, B ? V0 : V1, Vr);
    }
    const int kt = tile_at(n);
    const int k0 = kt * BN;

    int cls = qw < p.Sq ? kFast : kDead;
    if (dense || f_exp || k0 + BN > p.Sk || !raw_ok) cls = max(cls, (int)kGeneral);
    if (causal) {
      if (k0 > qw + WR - 1) cls = kDead;
      else if (k0 + BN - 1 > qw) cls = max(cls, (int)kGeneral);
    }
    int adir = 0;   // ALiBi on a tile wholly below (+1) or above (-1) the diagonal
    if (alibi && cls != kDead) {
      if (k0 + BN - 1 <= qw) adir = 1;
      else if (k0 >= qw + WR - 1) adir = -1;
      else cls = kGeneral;
    }
    if (use_summary && cls != kDead) {
      const uint32_t ts = __builtin_amdgcn_readfirstlane(tsum[kt]);
      const uint32_t kset = ts & 0xffu;
      if (f_mod) {
        const bool diag = p.allow_diag && k0 < qw + WR && k0 + BN > qw;
        if ((kset & allow_any) == 0 && !diag) cls = kDead;
        else if ((kset & ~allow_all) != 0 || diag) cls = max(cls, (int)kGeneral);
      } else if (kset == 0) {
        cls = kDead;
      }
      if (cls == kFast && (ts & 0x100u)) cls = kGeneral;
    } else if ((f_pad || f_mod) && cls != kDead) {
      cls = kGeneral;
    }

    if (cls != kDead) {
      f32x16 s[RB][KBN];
      scores(ks, s, f32x16{});
      // logit of element r of block (rb, kb):  t = cs * s + lane_off[rb]  (base-2 units)
      float cs = c_log2, lane_off[RB], mx[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) { lane_off[rb] = 0.f; mx[rb] = -INFINITY; }
      if (cls == kFast) {
        if (adir != 0) {
          const float a = adir * sl2c;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r)
                s[rb][kb][r] = fmaf(a, (float)(32 * kb + 8 * (r >> 2) + (r & 3)), s[rb][kb][r]);
            lane_off[rb] = adir * sl2 * (float)(k0 + 4 * g - my_i[rb]);
          }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
          for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx[rb] = fmaxf(mx[rb], s[rb][kb][r]);
          mx[rb] = fmaf(mx[rb], cs, lane_off[rb]);
        }
      } else {
        cs = 1.f;
        // padding and modality rules of the tile's keys for this lane's rows,
        // from wave votes (lane l votes for key k0 + l): bit jj of kmask[rb]
        // says key k0 + jj exists, is valid and its modality is allowed to the
        // row (or it is the row's own position under the diagonal rule)
        uint64_t kmask[RB];
        const bool vote = f_pad || f_mod;
        if (vote) {
          const int jl = k0 + l;
          const bool kin = l < BN && jl < p.Sk;
          bool kv = kin;
          if (f_pad && kin) kv = p.key_valid[(int64_t)b * p.Sk + jl] != 0;
          const uint64_t vmask = __ballot(kv);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) kmask[rb] = f_mod ? 0ull : vmask;
          if (f_mod) {
            // modalities this lane's rows may attend (read per tile rather than
            // held through the kernel, which has no register to spare)
            uint32_t row_allow[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              const int i = my_i[rb];
              const int mq = i < p.Sq ? p.qmod[(int64_t)b * p.Sq + i] : -1;
              row_allow[rb] = mq >= 0 ? (uint32_t)(p.allow_bits >> (8 * mq)) & 0xffu : 0u;
            }
            const int mk = kin ? p.kmod[(int64_t)b * p.Sk + jl] : -1;
            for (int a = 0; a < p.num_modalities; ++a) {
              const uint64_t km = __ballot(mk == a);
              if (km == 0ull) continue;
#pragma unroll
              for (int rb = 0; rb < RB; ++rb)
                if ((row_allow[rb] >> a) & 1u) kmask[rb] |= km;
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              const int d = my_i[rb] - k0;
              if (p.allow_diag && d >= 0 && d < BN) kmask[rb] |= 1ull << d;
              kmask[rb] &= vmask;
            }
          }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int i = my_i[rb];
          // the lane's keys of 32-key block kb sit at bits 8 (r / 4) + r % 4
          // of word kb once the mask is shifted by the lane half's 4 g
          const uint64_t kmg = vote ? kmask[rb] >> (4 * g) : 0ull;
#pragma unroll
          for (int kb = 0; kb < KBN; ++kb) {
            const uint32_t kw = (uint32_t)(kmg >> (32 * kb));
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = k0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
              float t = s[rb][kb][r] * c_log2;
              bool ok = j < p.Sk && i < p.Sq;
              if (vote) ok = ok && ((kw >> (8 * (r >> 2) + (r & 3))) & 1u);
              if (causal) ok = ok && j <= i;
              if (f_exp && ok)
                ok = p.em[(int64_t)b * p.em_sb + (int64_t)h * p.em_sh + (int64_t)i * p.em_sq + j] != 0;
              if (ok) {
                if (alibi) t -= sl2 * fabsf((float)(i - j));
                else if (dense) t += dense_bias(p, b, h, i, j) * kLog2e;
              } else {
                t = -INFINITY;
              }
              s[rb][kb][r] = t;
              mx[rb] = fmaxf(mx[rb], t);
            }
          }
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) mx[rb] = max_lane_pair(mx[rb]);
      float alpha[RB];
      update_max(mx, alpha);
      u32x4 pk[RB][NC];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float off = lane_off[rb] - (m_run[rb] == -INFINITY ? 0.f : m_run[rb]);
        float part[4];
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float x = exp2_fast(fmaf(s[rb][kb][r], cs, off));
            s[rb][kb][r] = x;
            if (kb == 0 && r < 4) part[r] = x;   // (0 + x is not folded away: -0)
            else part[r & 3] += x;
          }
        l_run[rb] = l_run[rb] * alpha[rb] + ((part[0] + part[1]) + (part[2] + part[3]));
        if (DROP) {
          // P o M / keep_prob enters P V; the row sum above is taken before dropout
#pragma unroll
          for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const uint32_t keep =
                  dropout_keep4(p, b, h, my_i[rb], k0 + 32 * kb + 8 * rr + 4 * g);
#pragma unroll
              for (int q = 0; q < 4; ++q)
                s[rb][kb][4 * rr + q] *= dropout_scale(p, (keep >> q) & 1u);
            }
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) pk[rb][c] = pack8<T>(s[rb][c >> 1], 8 * (c & 1));
      }
      pv(vs, pk);
    }
    vm_wait_barrier();
  };

  auto generic_phase = [&]() __attribute__((always_inline)) {
    if (n_gen > 0) {
      const int k0t = tile_at(0);
      load_tile(k0t, K0, Kr);
      load_tile(k0t, V0, Vr);
    }
    vm_wait_barrier();
    int n = 0;
    for (; n + 1 < n_gen; n += 2) {
      generic_step(n, BufIdx<0>{});
      generic_step(n + 1, BufIdx<1>{});
    }
    if (n < n_gen) generic_step(n, BufIdx<0>{});
  };

  if constexpr (LONG) {
    generic_phase();
  } else {
  // ==== fast phase: software pipeline over list entries n_gen .. n_all-1
  const int n_fast = n_all - n_gen;
  auto ftile = [&](int n) __attribute__((always_inline)) { return tile_at(n_gen + n); };
  // The fast tiles again, pairs of consecutive entries packed in one word, so a
  // step learns both tiles it loads from a single LDS read.  Written here and
  // read only after the barriers of the generic phase's and the fast phase's
  // set-up.
  for (int i = tid; i < n_fast; i += C::NT) {
    const uint32_t nxt = i + 1 < n_fast ? (uint32_t)(uint16_t)tlist[n_gen + i + 1] : 0u;
    fpair[i] = (uint32_t)(uint16_t)tlist[n_gen + i] | (nxt << 16);
  }
  // Logit of element r of block (rb, kb) of a fast tile: t = c_log2 * s + lane_off[rb]
  // (base-2 units), with the ALiBi term's per-register part folded into s.  The
  // tile lies wholly below (+1) or above (-1) the diagonal for every row of the
  // workgroup, or (causal rule) straddles it, where every visible key is at or
  // below the row, so the +1 form holds for them.  fold_max folds the tile
  // starting at key k0 into s (coefficient 0 without ALiBi: no branch, the
  // scores stay in place) and leaves lane_off and the row max (combined over
  // the lane pair) in mx; `part` selects one of NC equal shares of the
  // elements (0..NC-1, one per 16-key chunk of the P V products) or
  // all of them (-1), so the work can be spread over MFMA sections.  MASK
  // applies the causal rule per element (raw score -inf where key > row, which
  // needs c_log2 > 0); on a tile wholly below the diagonal it changes nothing.
  // Under the causal rule every fast tile has direction +1, and the score
  // accumulators start at the ALiBi term of the key's offset within its
  // 32-key block (s_init; zero without ALiBi): the fold then only masks and
  // takes the max, with the running max shifted by 32 ash at each 32-key
  // block boundary and the exponentials offset by kb * 32 ash * c_log2.
  // ALiBi without the causal rule folds the whole term per element.
  auto fold_max = [&](f32x16 (&sc)[RB][KBN], int k0, int part, float (&lane_off)[RB],
                      float (&mx)[RB], auto mask, auto opt) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask)::value;
    constexpr bool MX = MASK || !decltype(opt)::value;   // the row max is taken
    const int adir = (causal || k0 + BN - 1 <= q0) ? 1 : -1;
    const float a = fold_pe ? adir * sl2c : 0.f;
    constexpr int NE = 16 * KBN;
    const int e0 = part < 0 ? 0 : part * NE / NC, e1 = part < 0 ? NE : (part + 1) * NE / NC;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (part <= 0) {
        lane_off[rb] = alibi ? adir * sl2 * (float)(k0 + 4 * g - my_i[rb]) : 0.f;
        if (MX) mx[rb] = -INFINITY;
      }
      // element (kb, r) holds key k0 + 4g + c with c = 32kb + 8(r/4) + r%4
      const int lim = causal ? my_i[rb] - k0 - 4 * g : 0x7fffffff;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        if (e < e0 || e >= e1) continue;
        const int kb = e / 16, r = e % 16;
        const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
        if (MX && kb > 0 && r == 0) mx[rb] -= 32.f * ash;   // the block's values lack 32 kb ash
        float v = sc[rb][kb][r];
        if (fold_pe) v = fmaf(a, (float)c, v);
        sc[rb][kb][r] = (MASK && c > lim) ? -INFINITY : v;
        if (MX) mx[rb] = fmaxf(mx[rb], sc[rb][kb][r]);
      }
      if (MX && (part < 0 || part == NC - 1))
        mx[rb] = max_lane_pair(fmaf(mx[rb] + (32.f * (KBN - 1)) * ash, c_log2, lane_off[rb]));
    }
  };

  // One step: softmax of tile n (folded scores in s, row max in mx), scores of
  // tile n+1 (into sn) with their fold and max (into lon, mxn), O += P V of
  // tile n.  Buffer parity B: K_{n+1} in K[1-B], V_n in V[B].
  // OPT (opt): the optimistic form; steps past the first two neither take the
  // row max nor move the reference, and flag (bad) a lane whose tile sum
  // passes kOptMax.
  bool bad = false;
  auto fast_step = [&](int n, auto buf, f32x16 (&s)[RB][KBN], float (&lo)[RB], float (&mx)[RB],
                       f32x16 (&sn)[RB][KBN], float (&lon)[RB], float (&mxn)[RB], auto mask,
                       auto opt, const f32x16 &s_init) __attribute__((always_inline)) {
    constexpr int B = decltype(buf)::value;
    constexpr bool OPT = decltype(opt)::value;
    const uint16_t *kn = B ? K0 : K1;   // K of tile n+1
    const uint16_t *vs = B ? V1 : V0;   // V of tile n
    opaque(ro);
    opaque(to);
    const uint32_t pr = n + 1 < n_fast ? __builtin_amdgcn_readfirstlane(fpair[n + 1]) : 0u;
    const int kt1 = (int)(pr & 0xffffu);
    if (n + 2 < n_fast) load_tile((int)(pr >> 16), B ? K1 : K0, Kr);
    if (n + 1 < n_fast) load_tile(kt1, B ? V0 : V1, Vr);
    float alpha[RB], off[RB], offk[RB];
    if (!OPT || n <= 1) {   // mx holds the max of tile n (its fold took it)
      update_max(mx, alpha);
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) alpha[rb] = 1.f;
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      off[rb] = lo[rb] - (m_run[rb] == -INFINITY ? 0.f : m_run[rb]);
      offk[rb] = fmaf(32.f * ash, c_log2, off[rb]);   // second 32-key block (KBN = 2)
    }

    // Scores of tile n+1 interleaved with the exponentials of tile n, in an
    // order fixed by scheduling fences (only scalar work may cross them): the
    // K operand reads run two k-steps ahead of their products; per k-step the
    // score products are followed by a share of the exponentials (which do not
    // depend on them), so the matrix core and the VALU work side by side.  The
    // V^T reads of the first 16-key chunk go out three quarters in, those of
    // chunk c+1 ahead of the products of chunk c, and each chunk's P V
    // products are followed by a quarter of tile n+1's fold and max.  On the
    // last step the scores come from a stale buffer and are unused.  The
    // matrix-dense part runs at raised issue priority, so the wave sharing
    // this SIMD fills the gaps with its own VALU work.
    __builtin_amdgcn_s_setprio(1);
    constexpr int NE = 16 * KBN * RB;    // score elements per lane
    constexpr int EPS = NE / KS;         // exponentials per k-step
    constexpr int KPF = 2;               // K operand reads run this many k-steps ahead
    u32x4 ka[KS][KBN];
#pragma unroll
    for (int t = 0; t < KPF; ++t)
#pragma unroll
      for (int kb = 0; kb < KBN; ++kb) ka[t][kb] = read_row_at<D>(kn, 32 * kb, ro[t]);
    __builtin_amdgcn_sched_barrier(0x0004);
    float part[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int kb = 0; kb < KBN; ++kb) sn[rb][kb] = s_init;
    }
    u32x4 va[NC][DB];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      if (t + KPF < KS) {
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) ka[t + KPF][kb] = read_row_at<D>(kn, 32 * kb, ro[t + KPF]);
      }
      if (t == 3 * KS / 4) {
#pragma unroll
        for (int db = 0; db < DB; ++db) va[0][db] = read_tr_at<D>(vs, 0, &to[2 * db]);
      }
#pragma unroll
      for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sn[rb][kb] = Mfma<T>::mac(ka[t][kb], qf[rb][t], sn[rb][kb]);
#pragma unroll
      for (int e = t * EPS; e < (t + 1) * EPS; ++e) {
        const int rb = e / (16 * KBN), kb = (e / 16) % KBN, r = e % 16;
        const float x = exp2_fast(fmaf(s[rb][kb][r], c_log2, kb ? offk[rb] : off[rb]));
        s[rb][kb][r] = x;
        if (kb == 0 && r < 4) part[rb][r] = x;   // four short sum chains
        else part[rb][r & 3] += x;
      }
      __builtin_amdgcn_sched_barrier(0x0004);
    }
    u32x4 pk[RB][NC];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float tsum_l = (part[rb][0] + part[rb][1]) + (part[rb][2] + part[rb][3]);
      l_run[rb] = l_run[rb] * alpha[rb] + tsum_l;
      if (OPT) bad |= tsum_l > kOptMax;
      // pins the sum here: left free, the compiler sinks one step's sum into
      // the next step's head, a serial chain ahead of its first products
      asm volatile("" : "+v"(l_run[rb]));
#pragma unroll
      for (int c = 0; c < NC; ++c) pk[rb][c] = pack8<T>(s[rb][c >> 1], 8 * (c & 1));
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c + 1 < NC) {
#pragma unroll
        for (int db = 0; db < DB; ++db) va[c + 1][db] = read_tr_at<D>(vs, c + 1, &to[2 * db]);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb][db] = Mfma<T>::mac(va[c][db], pk[rb][c], acc[rb][db]);
      fold_max(sn, kt1 * BN, c, lon, mxn, mask, opt);
      __builtin_amdgcn_sched_barrier(0x0004);
    }
    __builtin_amdgcn_s_setprio(0);
    vm_wait_barrier();
  };
  auto fast_phase = [&](auto opt) __attribute__((always_inline)) {
    f32x16 sA[RB][KBN], sB[RB][KBN];
    float loA[RB], mxA[RB], loB[RB], mxB[RB];
    f32x16 s_init;   // formed here, after the generic phase, which does not use it
#pragma unroll
    for (int r = 0; r < 16; ++r) s_init[r] = ash * (float)(8 * (r >> 2) + (r & 3));
    const int f0 = ftile(0);
    load_tile(f0, K0, Kr);
    load_tile(f0, V0, Vr);
    if (n_fast > 1) load_tile(ftile(1), K1, Kr);
    vm_wait_barrier();
    scores(K0, sA, s_init);
    fold_max(sA, f0 * BN, -1, loA, mxA, std::bool_constant<true>{}, opt);
    lds_barrier();   // every wave is done with K0 before the first step refills it
    // causal-band tiles lead the list: tile 0 was folded with the mask above,
    // step 0 folds tile 1 with it, and the steps after it need none
    constexpr std::bool_constant<false> nomask{};
    fast_step(0, BufIdx<0>{}, sA, loA, mxA, sB, loB, mxB, std::bool_constant<true>{}, opt, s_init);
    int n = 1;
    for (; n + 1 < n_fast; n += 2) {
      fast_step(n, BufIdx<1>{}, sB, loB, mxB, sA, loA, mxA, nomask, opt, s_init);
      fast_step(n + 1, BufIdx<0>{}, sA, loA, mxA, sB, loB, mxB, nomask, opt, s_init);
    }
    if (n < n_fast) fast_step(n, BufIdx<1>{}, sB, loB, mxB, sA, loA, mxA, nomask, opt, s_init);
  };

  generic_phase();
  if (n_fast > 0) {
    fast_phase(std::true_type{});
    if (__syncthreads_or(bad)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[rb][db] = f32x16{};
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
      }
      generic_phase();
      fast_phase(std::false_type{});
    }
  }
  }

  // ---- epilogue: O = acc / l, LSE
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = my_i[rb];
    const float l_tot = l_run[rb] + __shfl_xor(l_run[rb], 32, 64);
    if (i < p.Sq) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      T *Og = (T *)p.o + b * p.q_sb + h * p.q_sh + (int64_t)i * p.q_ss;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d0 = 32 * db + 8 * rr + 4 * g;
          u32x2 v;
          v[0] = pack2<T>(acc[rb][db][4 * rr + 0] * inv, acc[rb][db][4 * rr + 1] * inv);
          v[1] = pack2<T>(acc[rb][db][4 * rr + 2] * inv, acc[rb][db][4 * rr + 3] * inv);
          *(u32x2 *)(Og + d0) = v;
        }
      }
      if (g == 0)
        p.lse[((int64_t)b * p.H + h) * p.Sq + i] =
            l_tot > 0.f ? (m_run[rb] + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <typename T, int D, int NW, int RB, int KBN, bool LONG>
hipError_t launch_t(const Params &p, hipStream_t s) {
  using C = FwdCfg<T, D, NW, RB, KBN>;
  const int n_qtiles = (p.Sq + C::BM - 1) / C::BM;
  const int64_t blocks = (int64_t)n_qtiles * p.B * p.H;
  if (blocks == 0) return hipSuccess;
  const bool fold = p.pse_kind == FA_PSE_ALIBI && !(p.mask_flags & FA_MASK_CAUSAL);
  const dim3 grid((unsigned)blocks), block(C::NT);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, s, p, n_qtiles); };
  if (log_enabled()) {
    char name[128];
    snprintf(name, sizeof(name), "fwd_mfma_kernel<%s, D=%d, NW=%d, RB=%d, KBN=%d%s%s%s>",
             std::is_same<T, __bf16>::value ? "bf16" : "f16", D, NW, RB, KBN,
             p.dropout ? ", DROP" : "", fold ? ", FOLD" : "", LONG ? ", LONG" : "");
    log_launch("fa_fwd", name, (long long)blocks, C::NT, p);
  }
  if (p.dropout) {
    if (fold) go(fwd_mfma_kernel<T, D, NW, RB, KBN, true, true, LONG>);
    else go(fwd_mfma_kernel<T, D, NW, RB, KBN, true, false, LONG>);
  } else {
    if (fold) go(fwd_mfma_kernel<T, D, NW, RB, KBN, false, true, LONG>);
    else go(fwd_mfma_kernel<T, D, NW, RB, KBN, false, false, LONG>);
  }
  return hipGetLastError();
}

constexpr int kRB = 1, kKBN = 2;   // tile shape: 32-row blocks per wave, 32-key blocks per tile
constexpr int kNW = 4;             // waves per workgroup

// One (dtype, head_dim): S_q <= 32 takes a one-wave workgroup (lists of
// kMaxTilesSmall tiles); otherwise a key range of more than kMaxTiles tiles
// takes the LONG instance.
template <typename T, int D>
hipError_t launch_d(const Params &p, hipStream_t s) {
  const int64_t n_kt = ((int64_t)p.Sk + 32 * kKBN - 1) / (32 * kKBN);
  // S_q <= 32: one-wave workgroups streaming 32-key tiles (D = 64) or 64-key
  // tiles (D = 128), so that more workgroups fit a CU's LDS
  constexpr int KBN_S = D == 64 ? 1 : kKBN;
  const int64_t n_kt_s = ((int64_t)p.Sk + 32 * KBN_S - 1) / (32 * KBN_S);
  const int ov = tile_override();
  if ((ov == kTileAuto || ov == kTileShort) && short_fits(p)) return launch_short<T, D>(p, s);
  const bool small = ov == kTileWg1 ? n_kt_s <= kMaxTilesSmall
                                    : ov != kTileWg4 && p.Sq <= 32 * kRB && n_kt_s <= kMaxTilesSmall;
  if (small) return launch_t<T, D, 1, kRB, KBN_S, false>(p, s);
  if (n_kt > kMaxTiles) return launch_t<T, D, kNW, kRB, kKBN, true>(p, s);
  return launch_t<T, D, kNW, kRB, kKBN, false>(p, s);
}

}  // namespace
}  // namespace fa
