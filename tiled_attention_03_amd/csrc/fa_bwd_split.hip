// Key pass of the backward (dK, dV) with producer and consumer waves.
//
// Same gradient as the key pass in fa_bwd.hip (FlashAttentionScore
// replacement guide, section 2: P recomputed from the saved row LSE,
// dS = P * (dP - delta), dV = P^T dO, dK = dS^T Q * scale), organised for two
// waves per SIMD.  A workgroup owns 128 keys of one (batch, head) in four
// slices of 32 and walks the 32-row query blocks that can see them.  Eight
// waves: wave w < 4 is the producer of slice w, wave w + 4 its consumer, and
// the two share a SIMD.
//
//   producer, step n: S = Q K^T and dP = dO V^T of block n (A = Q / dO rows
//     from LDS, B = the slice's K / V rows held in registers), then P and dS;
//     it hands P^T and dS^T to its consumer through LDS.  In the 32x32
//     accumulator layout a lane holds one key and 16 queries, which is the
//     A-operand layout of P^T and dS^T, so each lane stores its own rounded
//     values and the consumer's lane of the same index reads them back.
//   consumer, step n: dV += P^T dO and dK += dS^T Q of block n - 1 (B = the
//     block's dO / Q read transposed from LDS); the accumulators never leave
//     its registers.
//
// Each role holds only its own state (the producer K and V, the consumer the
// dK / dV accumulators), so each fits half a SIMD's register file, and the
// matrix core takes products from whichever wave is ready.  One barrier per
// step.  Q / dO tiles and the row statistics of a block go straight from
// global memory into a ring of six LDS buffers, three blocks ahead of the
// producer; the exchange ring has two.
//
// Handles the causal rule with or without ALiBi, and plain (maskless)
// problems, with or without dropout, without the bias gradient (float32
// gradient outputs included); the launcher sends everything else to the
// one-role key pass.  Under the causal rule every row
// sees key 0, so no row has an empty softmax here and the LSE is finite.
#include <climits>

#include <stdio.h>

#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int SKB = 128;   // keys per workgroup: four slices of 32
constexpr int SQB = 32;    // query rows per block
constexpr int NPW = 4;     // producer waves (and consumer waves)

// One LDS-direct dword load per lane (row statistics); lane l writes the
// 4 bytes at dst + 4 l.  A device function, not a lambda, so that the kernel
// keeps its host stub.
__device__ __forceinline__ void stats_load(float *dst, __amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                           uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)dst, 4,
                                           voff, (int)soff, 0, 0);
}

// DROP: dropout compiled in (keep_prob < 1); the producer regenerates the
// Philox keep mask of its elements, as the one-role pass does.
template <typename T, int D, bool DROP>
__global__ __launch_bounds__(2 * NPW * 64, 1) void bwd_kv_split_kernel(Params p, int n_ktiles) {
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int ES = (int)sizeof(T);
  using G = TileGeom<D, SQB, NPW>;
  constexpr int LPW = 2 * G::PER_WAVE + 1;   // global loads per producer wave per block
  // Ring of six block slots (block b in slot b % 6), each one variable
  // holding the Q tile, the dO tile, then LSE and delta of the block's rows;
  // and the P^T / dS^T exchange (ring of two).  Every access names its
  // buffer statically, and the slots are few enough for the compiler's
  // wait-count pass to track the direct-to-LDS loads into each of them apart,
  // so a read of one slot does not wait for loads into another.
  constexpr int NSL = 6;
  constexpr int SLOT = 2 * SQB * D + 4 * SQB;   // 16-bit units
  __shared__ __attribute__((aligned(16))) uint16_t T0[SLOT], T1[SLOT], T2[SLOT], T3[SLOT],
      T4[SLOT], T5[SLOT];
  __shared__ __attribute__((aligned(16))) u32x4 X0[NPW * 64 * 4], X1[NPW * 64 * 4];

  const int BH = p.B * p.H;
  const int lin = blockIdx.x;
  const int kt = lin / BH;   // key tile 0 sees the most causal rows: first
  const int bh = lin % BH;
  const int b = bh / p.H, h = bh % p.H;
  const int j0 = kt * SKB;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int w = wv & (NPW - 1);                              // key slice
  const bool producer = wv < NPW;
  const int l = tid & 63, g = l >> 5, lr = l & 31;
  const int jw = j0 + 32 * w;
  const int my_j = jw + lr;
  const bool causal = p.mask_flags & FA_MASK_CAUSAL;
  const bool alibi = p.pse_kind == FA_PSE_ALIBI;

  const int64_t qoff = b * p.q_sb + h * p.q_sh;
  const int64_t koff = b * p.k_sb + h * p.k_sh;
  const int64_t rbase = ((int64_t)b * p.H + h) * p.Sq;
  const uint32_t qrow_b = (uint32_t)(p.q_ss * ES);

  const int it_begin = causal ? j0 / SQB : 0;
  const int it_end = (p.Sq + SQB - 1) / SQB;
  const int nb = max(it_end - it_begin, 0);   // query blocks; steps 0 .. nb

  auto slot = [&](auto bi) -> uint16_t * {
    constexpr int B = decltype(bi)::value;
    return B == 0 ? T0 : B == 1 ? T1 : B == 2 ? T2 : B == 3 ? T3 : B == 4 ? T4 : T5;
  };
  auto qbuf = [&](auto bi) { return slot(bi); };
  auto gbuf = [&](auto bi) { return slot(bi) + SQB * D; };
  auto lbuf = [&](auto bi) { return (float *)(slot(bi) + 2 * SQB * D); };
  auto ebuf = [&](auto bi) { return (float *)(slot(bi) + 2 * SQB * D) + SQB; };
  // exchange slots of this slice: operand k of lane l at [64 k + l] (a wave
  // writes or reads 1 KB of consecutive 16-byte chunks per instruction)
  auto xbuf = [&](auto bi) -> u32x4 * {
    constexpr int B = decltype(bi)::value;
    return (B % 2 == 0 ? X0 : X1) + w * 64 * 4;
  };

  if (producer) {
    // ======================= producer =======================
    const auto Qr = make_rsrc((const T *)p.q + qoff, span_bytes(p.Sq, p.q_ss, D, ES));
    const auto Gr = make_rsrc((const T *)p.dout + qoff, span_bytes(p.Sq, p.q_ss, D, ES));
    const auto Sr = make_rsrc(w < 2 ? (const void *)(p.lse + rbase) : (const void *)(p.delta + rbase),
                              (uint32_t)p.Sq * 4u);
    // K and V rows of this lane's key (rows past S_k read as zeros)
    u32x4 kf[KS], vf[KS];
    {
      const auto Kr = make_rsrc((const T *)p.k + koff, span_bytes(p.Sk, p.k_ss, D, ES));
      const auto Vr = make_rsrc((const T *)p.v + koff, span_bytes(p.Sk, p.k_ss, D, ES));
      const uint32_t off = my_j < p.Sk ? (uint32_t)((int64_t)my_j * p.k_ss * ES) : 0x80000000u;
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        kf[t] = buf_load16(Kr, off + (16 * t + 8 * g) * ES);
        vf[t] = buf_load16(Vr, off + (16 * t + 8 * g) * ES);
      }
      // without dropout the dP accumulator starts at the row's delta and V
      // enters negated, so it ends at delta - dP = -(dP - delta)
      if constexpr (!DROP) {
#pragma unroll
        for (int t = 0; t < KS; ++t) vf[t] ^= 0x80008000u;
      }
    }
    uint32_t voff[G::PER_WAVE];
    tile_offsets<D, SQB, NPW>(voff, qrow_b, w, l);
    // block n's Q / dO tiles and statistics into ring slot bi (wave w loads
    // its share of the tiles and 16 rows of LSE (w < 2) or delta (w >= 2))
    auto load_tiles = [&](int n, auto bi) __attribute__((always_inline)) {
      const int i0 = (it_begin + n) * SQB;
      tile_load<D, SQB, NPW>(qbuf(bi), Qr, voff, (uint32_t)i0 * qrow_b, w);
      tile_load<D, SQB, NPW>(gbuf(bi), Gr, voff, (uint32_t)i0 * qrow_b, w);
    };
    // (rows past S_q read as zeros, so a block past the last one is harmless)
    auto load_stats = [&](int n, auto bi) __attribute__((always_inline)) {
      const int i0 = (it_begin + n) * SQB;
      float *sd = (w < 2 ? lbuf(bi) : ebuf(bi)) + 16 * (w & 1);
      if (l < 16) stats_load(sd, Sr, 4u * (uint32_t)l, 4u * (uint32_t)(i0 + 16 * (w & 1)));
    };

    uint32_t ro[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) ro[t] = row_off<D>(lr, 2 * t + g);
    const float c_log2 = p.scale_log2;
    const float sl2 = alibi ? p.alibi_slopes[h] * kLog2e : 0.f;
    // The S accumulator of row i (block start i0) starts at the row term
    // W_i = -(LSE_i log2e + slope log2e (i - i0)) / c_log2, which a consumer
    // wave writes over the block's LSE in LDS two steps ahead, so that
    // c_log2 (S + W_i) + slope log2e (my_j - i0) is the base-2 logit
    // c_log2 S + slope log2e (my_j - i) - LSE_i log2e: one fma per element.
    // start values of block bi's S and dP accumulators
    auto init_acc = [&](auto bi, f32x16 &s0, f32x16 &dp0) __attribute__((always_inline)) {
      const float *ls = lbuf(bi), *ds = ebuf(bi);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const f32x4 wv4 = *(const f32x4 *)&ls[8 * rr + 4 * g];
#pragma unroll
        for (int q = 0; q < 4; ++q) s0[4 * rr + q] = wv4[q];
      }
      if constexpr (DROP) {
        dp0 = f32x16{};
      } else {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const f32x4 dv = *(const f32x4 *)&ds[8 * rr + 4 * g];
#pragma unroll
          for (int q = 0; q < 4; ++q) dp0[4 * rr + q] = dv[q];
        }
      }
    };

    // S and dP of the block in slot bi, not interleaved (the first block)
    auto scores = [&](auto bi, f32x16 &s, f32x16 &dp) __attribute__((always_inline)) {
      const uint16_t *qs = qbuf(bi), *gs = gbuf(bi);
      init_acc(bi, s, dp);
#pragma unroll
      for (int t0 = 0; t0 < KS; t0 += 4) {
        u32x4 qa[4], ga[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          qa[t] = read_row_at<D>(qs, 0, ro[t0 + t]);
          ga[t] = read_row_at<D>(gs, 0, ro[t0 + t]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          s = Mfma<T>::mac(qa[t], kf[t0 + t], s);
          dp = Mfma<T>::mac(ga[t], vf[t0 + t], dp);
        }
      }
    };

    // end of a step: this wave's loads of the block after next have landed
    // (those issued in this step may still be in flight), its LDS writes are
    // done; then the workgroup barrier
    auto finish = [&](bool more) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      if (more) __builtin_amdgcn_s_waitcnt(0x0070 | LPW);   // vmcnt(LPW) lgkmcnt(0)
      else __builtin_amdgcn_s_waitcnt(0x0070);              // vmcnt(0) lgkmcnt(0)
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };

    // Step n (block n in slot n % 6, its S and dP in s / dp from the step
    // before): S and dP of block n+1 into sn / dpn, interleaved k-step by
    // k-step with block n's P and dS (which do not depend on them), in an
    // order fixed by scheduling fences; block n's P^T / dS^T go to exchange
    // slot n % 2; then block n+3 is loaded into slot (n+3) % 6, which held
    // block n-3 (last read in step n-2).  On the last step the scores come
    // from a stale slot and are unused.
    //   element r: query i0 + 4g + c, c = 8(r/4) + r%4; key my_j.  Base-2
    //   logit t = c_log2 s + slope (my_j - i) - LSE log2e (the ALiBi form
    //   holds for every visible key, which is at or below its row).  MASK
    //   (the four blocks of the causal band, which lead the range) zeroes
    //   keys past their query.  Rows past S_q have zero Q and dO rows, so
    //   their P cannot reach dV or dK; keys past S_k are never stored; and
    //   outside the band every key is at or below every row, so P stays
    //   finite there without a mask.
    constexpr int KPF = 2;                 // operand reads run this many k-steps ahead
    constexpr int PRE = 4;                 // elements of P / dS before the first product
    auto pstep = [&](int n, auto bi, auto mask, f32x16 &s, f32x16 &dp, f32x16 &sn, f32x16 &dpn)
                     __attribute__((always_inline)) {
      constexpr int B = decltype(bi)::value;
      constexpr bool MASK = decltype(mask)::value;
      opaque(ro);
      const uint16_t *qn = qbuf(BufIdx<(B + 1) % NSL>{}), *gn = gbuf(BufIdx<(B + 1) % NSL>{});
      const float *ds = ebuf(bi);
      const int i0 = (it_begin + n) * SQB;
      const float L = sl2 * (float)(my_j - i0);
      const int lim = causal ? my_j - i0 - 4 * g : INT_MIN;   // c < lim is hidden
      // dropout: the four lanes of a quad hold four consecutive keys and the
      // same 16 queries, so lane q of the quad draws the Philox words of the
      // queries with r % 4 == q (one call covers the quad's four keys), packs
      // the keep bits, and the quad exchanges them; bit 4 rr of kq[q] is then
      // the keep bit of element 4 rr + q for this lane's key
      // LDS reads first, all in flight together: block n+1's row terms (the S
      // start values) and delta (the dP start values), its first KPF operand
      // k-steps, and under dropout block n's delta
      f32x4 dl[4];
      {
        const float *ln = lbuf(BufIdx<(B + 1) % NSL>{}), *dn = ebuf(BufIdx<(B + 1) % NSL>{});
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const f32x4 wv4 = *(const f32x4 *)&ln[8 * rr + 4 * g];
#pragma unroll
          for (int q = 0; q < 4; ++q) sn[4 * rr + q] = wv4[q];
        }
        if constexpr (DROP) {
          dpn = f32x16{};
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) dl[rr] = *(const f32x4 *)&ds[8 * rr + 4 * g];
        } else {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const f32x4 dv = *(const f32x4 *)&dn[8 * rr + 4 * g];
#pragma unroll
            for (int q = 0; q < 4; ++q) dpn[4 * rr + q] = dv[q];
          }
        }
      }
      u32x4 qa[KS], ga[KS];
#pragma unroll
      for (int t = 0; t < KPF; ++t) {
        qa[t] = read_row_at<D>(qn, 0, ro[t]);
        ga[t] = read_row_at<D>(gn, 0, ro[t]);
      }
      __builtin_amdgcn_sched_barrier(0x0004);
      // dropout: the four lanes of a quad hold four consecutive keys and the
      // same 16 queries, so lane q of the quad draws the Philox words of the
      // queries with r % 4 == q (one call covers the quad's four keys), packs
      // the keep bits, and the quad exchanges them; bit 4 rr of kq[q] is then
      // the keep bit of element 4 rr + q for this lane's key
      uint32_t kq[4] = {0u, 0u, 0u, 0u};
      if (DROP) {
        uint32_t mine = 0u;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          mine |= dropout_keep4(p, b, h, i0 + 8 * rr + 4 * g + (l & 3), my_j) << (4 * rr);
        kq[0] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0x00, 0xF, 0xF, false);
        kq[1] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0x55, 0xF, 0xF, false);
        kq[2] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0xAA, 0xF, 0xF, false);
        kq[3] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0xFF, 0xF, 0xF, false);
#pragma unroll
        for (int q = 0; q < 4; ++q) kq[q] >>= (l & 3);
      }
      // element r of block n: P, then dS (negated without dropout)
      auto elem = [&](int r) __attribute__((always_inline)) {
        const int rr = r >> 2, q = r & 3, c = 8 * rr + q;
        float pr = exp2_fast(fmaf(s[r], c_log2, L));
        if (MASK) pr = c < lim ? 0.f : pr;
        if constexpr (DROP) {
          // P o M / keep_prob feeds dV, and dP is masked the same way
          const float m = dropout_scale(p, (kq[q] >> (4 * rr)) & 1u);
          s[r] = pr * m;
          dp[r] = pr * (dp[r] * m - dl[rr][q]);
        } else {
          s[r] = pr;
          dp[r] = pr * dp[r];   // -dS: the accumulator holds delta - dP
        }
      };
      // the first PRE elements (registers only) cover the reads' latency
#pragma unroll
      for (int r = 0; r < PRE; ++r) elem(r);
      __builtin_amdgcn_sched_barrier(0x0004);
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        if (t + KPF < KS) {
          qa[t + KPF] = read_row_at<D>(qn, 0, ro[t + KPF]);
          ga[t + KPF] = read_row_at<D>(gn, 0, ro[t + KPF]);
        }
        sn = Mfma<T>::mac(qa[t], kf[t], sn);
        dpn = Mfma<T>::mac(ga[t], vf[t], dpn);
#pragma unroll
        for (int r = PRE + t * (16 - PRE) / KS; r < PRE + (t + 1) * (16 - PRE) / KS; ++r) elem(r);
        // the first half of P^T and dS^T goes to the exchange slot as soon as
        // its elements are done, so the step's tail only writes the second
        if (PRE + t * (16 - PRE) / KS < 8 && PRE + (t + 1) * (16 - PRE) / KS >= 8) {
          u32x4 *x = xbuf(bi) + l;
          x[0] = pack8<T>(s, 0);
          x[128] = pack8<T>(dp, 0);
        }
        __builtin_amdgcn_sched_barrier(0x0004);
      }
      u32x4 *x = xbuf(bi) + l;
      x[64] = pack8<T>(s, 8);
      x[192] = pack8<T>(dp, 8);
      __builtin_amdgcn_sched_barrier(0);
      const bool more = n + 3 < nb;
      if (more) {
        load_tiles(n + 3, BufIdx<(B + 3) % NSL>{});
        load_stats(n + 4, BufIdx<(B + 4) % NSL>{});
      }
      finish(more);
    };
    if (nb > 0) load_tiles(0, BufIdx<0>{});
    if (nb > 1) load_tiles(1, BufIdx<1>{});
    if (nb > 2) load_tiles(2, BufIdx<2>{});
    load_stats(0, BufIdx<0>{});
    load_stats(1, BufIdx<1>{});
    load_stats(2, BufIdx<2>{});
    load_stats(3, BufIdx<3>{});
    finish(false);   // everything has landed; the consumers turn the LSE of
    finish(false);   // blocks 0 and 1 into row terms between these barriers
    f32x16 sA, dpA, sB, dpB;
    scores(BufIdx<0>{}, sA, dpA);   // stale when nb == 0, and unused
    const std::true_type band;
    const std::false_type plain;
    if (0 <= nb) pstep(0, BufIdx<0>{}, band, sA, dpA, sB, dpB);
    if (1 <= nb) pstep(1, BufIdx<1>{}, band, sB, dpB, sA, dpA);
    if (2 <= nb) pstep(2, BufIdx<2>{}, band, sA, dpA, sB, dpB);
    if (3 <= nb) pstep(3, BufIdx<3>{}, band, sB, dpB, sA, dpA);
    for (int n = 4; n <= nb; n += 6) {
      pstep(n, BufIdx<4>{}, plain, sA, dpA, sB, dpB);
      if (n + 1 <= nb) pstep(n + 1, BufIdx<5>{}, plain, sB, dpB, sA, dpA);
      if (n + 2 <= nb) pstep(n + 2, BufIdx<0>{}, plain, sA, dpA, sB, dpB);
      if (n + 3 <= nb) pstep(n + 3, BufIdx<1>{}, plain, sB, dpB, sA, dpA);
      if (n + 4 <= nb) pstep(n + 4, BufIdx<2>{}, plain, sA, dpA, sB, dpB);
      if (n + 5 <= nb) pstep(n + 5, BufIdx<3>{}, plain, sB, dpB, sA, dpA);
    }
  } else {
    // ======================= consumer =======================
    f32x16 dv[DB], dk[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dv[db] = dk[db] = f32x16{};
    uint32_t to[2 * DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) tr_off<D>(&to[2 * db], 32 * db, l);

    // The transposed dO / Q operands of a block are read one step ahead:
    // block n's tiles have been in LDS since the barrier that ended step n-2,
    // so step n reads them after issuing its products, and step n+1 only
    // waits for the exchange reads before its first product.
    u32x4 gt[2][DB], qt[2][DB];
    auto prefetch = [&](auto bi) __attribute__((always_inline)) {
      const uint16_t *qs = qbuf(bi), *gs = gbuf(bi);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          gt[c][db] = read_tr_at<D>(gs, c, &to[2 * db]);
          qt[c][db] = read_tr_at<D>(qs, c, &to[2 * db]);
        }
    };
    auto consume = [&](auto xi) __attribute__((always_inline)) {
      const u32x4 *x = xbuf(xi) + l;
      const u32x4 pp[2] = {x[0], x[64]}, pd[2] = {x[128], x[192]};
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[db] = Mfma<T>::mac(pp[c], gt[c][db], dv[db]);
          dk[db] = Mfma<T>::mac(pd[c], qt[c][db], dk[db]);
        }
    };
    auto finish = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS reads are done
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    // step n: consume block n-1 (exchange slot (n-1)%2, operands already in
    // registers), then read block n's operands from ring slot n % 6
    // the producers' S start values: block bi's LSE (landed) becomes the row
    // term W_i = -(LSE_i log2e + slope log2e (i - i0)) / c_log2 in place
    const float inv_c = 1.f / p.scale_log2;
    const float sl2 = alibi ? p.alibi_slopes[h] * kLog2e : 0.f;
    auto row_terms = [&](auto bi) __attribute__((always_inline)) {
      if (l < SQB) {
        float *ls = lbuf(bi);
        ls[l] = -fmaf(ls[l], kLog2e, sl2 * (float)l) * inv_c;
      }
    };
    // step n: besides, the first consumer wave writes the row terms of block
    // n+2 (its statistics landed by the end of step n-1; the producers read
    // them in step n+1)
    auto cstep = [&](int n, auto bi) __attribute__((always_inline)) {
      constexpr int B = decltype(bi)::value;
      opaque(to);
      if (n >= 1 && n - 1 < nb) consume(BufIdx<(B + NSL - 1) % NSL>{});
      __builtin_amdgcn_sched_barrier(0);
      if (n < nb) prefetch(bi);
      if (wv == NPW) row_terms(BufIdx<(B + 2) % NSL>{});
      finish();
    };
    finish();   // the producers' loads of the first blocks have landed
    if (wv == NPW) row_terms(BufIdx<0>{});
    if (wv == NPW + 1) row_terms(BufIdx<1>{});
    finish();
    for (int n = 0; n <= nb; n += NSL) {
      cstep(n, BufIdx<0>{});
      if (n + 1 <= nb) cstep(n + 1, BufIdx<1>{});
      if (n + 2 <= nb) cstep(n + 2, BufIdx<2>{});
      if (n + 3 <= nb) cstep(n + 3, BufIdx<3>{});
      if (n + 4 <= nb) cstep(n + 4, BufIdx<4>{});
      if (n + 5 <= nb) cstep(n + 5, BufIdx<5>{});
    }

    // dK (scaled) and dV; element r: key jw + 8(r/4) + 4g + r%4, column 32db + lr.
    // Without dropout the exchanged dS is negated, and so is the scale.
    const float dks = DROP ? p.scale : -p.scale;
    if (p.grad_f32) {
      float *DKf = (float *)p.dk + koff;
      float *DVf = (float *)p.dv + koff;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jw + 8 * (r >> 2) + 4 * g + (r & 3);
          if (j < p.Sk) {
            DKf[(int64_t)j * p.k_ss + 32 * db + lr] = dk[db][r] * dks;
            DVf[(int64_t)j * p.k_ss + 32 * db + lr] = dv[db][r];
          }
        }
      }
      return;
    }
    T *DKg = (T *)p.dk + koff;
    T *DVg = (T *)p.dv + koff;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jw + 8 * (r >> 2) + 4 * g + (r & 3);
        if (j < p.Sk) {
          DKg[(int64_t)j * p.k_ss + 32 * db + lr] = from_f32<T>(dk[db][r] * dks);
          DVg[(int64_t)j * p.k_ss + 32 * db + lr] = from_f32<T>(dv[db][r]);
        }
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_t(const Params &p, hipStream_t s) {
  const int n_ktiles = (p.Sk + SKB - 1) / SKB;
  const int64_t blocks = (int64_t)n_ktiles * p.B * p.H;
  if (blocks == 0) return hipSuccess;
  if (log_enabled()) {
    char name[96];
    snprintf(name, sizeof(name), "bwd_kv_split_kernel<D=%d%s> (producer/consumer key pass)", D,
             p.dropout ? ", DROP" : "");
    log_launch("fa_bwd_main", name, (long long)blocks, 2 * NPW * 64, p);
  }
  if (p.dropout)
    hipLaunchKernelGGL((bwd_kv_split_kernel<T, D, true>), dim3((unsigned)blocks),
                       dim3(2 * NPW * 64), 0, s, p, n_ktiles);
  else
    hipLaunchKernelGGL((bwd_kv_split_kernel<T, D, false>), dim3((unsigned)blocks),
                       dim3(2 * NPW * 64), 0, s, p, n_ktiles);
  return hipGetLastError();
}

}  // namespace

bool bwd_kv_split_eligible(const Params &p) {
  const uint32_t other = FA_MASK_PADDING | FA_MASK_MODALITY | FA_MASK_EXPLICIT;
  if (p.mask_flags & other) return false;
  if (p.pse_kind == FA_PSE_DENSE) return false;
  if (p.pse_kind == FA_PSE_ALIBI && !(p.mask_flags & FA_MASK_CAUSAL)) return false;
  if (p.dpse) return false;
  // the S accumulator's start value divides by scale * log2(e)
  const float c = fabsf(p.scale_log2);
  if (!(c > kRawMinC && c < 1e20f)) return false;
  return p.D == 64 || p.D == 128;
}

hipError_t launch_bwd_kv_split(const Params &p, int dtype, hipStream_t s) {
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
