// Backward attention, bf16/f16 inputs, MFMA on gfx950.
//
// Recompute-based gradient (FlashAttentionScore replacement guide, section
// 2: gradients come without the N x N matrix, from O(N) saved statistics).
// Only O and the row LSE come from the forward; every P tile is recomputed
// as P = exp2(S * scale * log2 e + bias * log2 e - LSE * log2 e), and
// dS = P * (dP - delta) with delta_i = sum_d dO_id O_id (the prep pass).
//
// Two passes, no atomics, bitwise repeatable:
//
// * key pass (dK, dV): a workgroup of 4 waves owns 128 keys of one
//   (batch, head), 32 per wave, and walks the 32-row query blocks that can
//   see them (causal: from the diagonal down).  Per block and wave:
//     S  = Q . K^T,  dP = dO . V^T  (A = Q / dO rows from LDS, B = the wave's
//                                    K / V rows held in VGPRs)
//     dV += P^T . dO, dK += dS^T . Q (A = P^T / dS^T straight from the S / dP
//                                    accumulators, B = transposed LDS reads)
//   In the 32x32 accumulator layout a lane holds one key and 16 queries,
//   which is exactly the A layout of P^T and dS^T with queries as the
//   contraction index, so those never move.
//
// * query pass (dQ): a workgroup of 4 waves owns 128 query rows (32 per wave)
//   and walks the 64-key tiles they can see, like the forward:
//     S^T = K . Q^T, dP^T = V . dO^T (A = K / V rows from LDS, B = Q / dO rows
//                                    of the lane's query, in VGPRs)
//     dQ^T += K^T . dS^T             (A = transposed K reads, B = dS^T from
//                                    the accumulators)
//   A lane owns one query row, so LSE and delta are per-lane scalars.
//
// Both passes double-buffer their streamed tiles in LDS: the tiles of step
// n+1 are loaded from global memory straight into LDS (no register staging)
// while step n is multiplied, with one barrier per step; blocks the mask hides
// entirely are skipped.
#include <algorithm>
#include <climits>

#include <stdio.h>

#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int NWB = 4;      // waves per workgroup (both passes)
constexpr int KB = 128;     // keys per workgroup, key pass
constexpr int QB = 32;      // queries per step, key pass
constexpr int QBQ = 128;    // queries per workgroup, query pass
constexpr int KBQ = 64;     // keys per step, query pass

// ===========================================================================
// key pass: dK, dV
// DROP: dropout compiled in (keep_prob < 1); the kernel without it carries no
// dropout code at all.  EXTRA: the optional outputs (float32 gradients, the
// bias gradient) compiled in; likewise absent from the plain instance.
template <typename T, int D, bool DROP, bool EXTRA>
__global__ __launch_bounds__(256, 1) void bwd_kv_kernel(Params p, int n_ktiles) {
  constexpr int KS = D / 16, DB = D / 32, CH = D / 8;
  constexpr int ES = (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) uint16_t Q0[QB * D], Q1[QB * D], Q2[QB * D];
  __shared__ __attribute__((aligned(16))) uint16_t G0[QB * D], G1[QB * D], G2[QB * D];
  __shared__ __attribute__((aligned(16))) float lam_s[3][QB];   // LSE*log2e (+ALiBi row term)
  __shared__ __attribute__((aligned(16))) float lse_s[3][QB];   // LSE*log2e
  __shared__ __attribute__((aligned(16))) float dlt_s[3][QB];

  const int BH = p.B * p.H;
  const int lin = blockIdx.x;
  const int kt = lin / BH;            // key tile 0 sees the most causal rows: first
  const int bh = lin % BH;
  const int b = bh / p.H, h = bh % p.H;
  const int j0 = kt * KB;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int l = tid & 63, g = l >> 5, lr = l & 31;
  const int jw = j0 + 32 * w;
  const int my_j = jw + lr;
  const uint32_t flags = p.mask_flags;
  const bool causal = flags & FA_MASK_CAUSAL;
  const bool alibi = p.pse_kind == FA_PSE_ALIBI, dense = p.pse_kind == FA_PSE_DENSE;
  const bool f_elem = flags & (FA_MASK_PADDING | FA_MASK_MODALITY | FA_MASK_EXPLICIT);

  const int64_t qoff = b * p.q_sb + h * p.q_sh;
  const int64_t koff = b * p.k_sb + h * p.k_sh;
  const auto Qr = make_rsrc((const T *)p.q + qoff, span_bytes(p.Sq, p.q_ss, D, ES));
  const auto Gr = make_rsrc((const T *)p.dout + qoff, span_bytes(p.Sq, p.q_ss, D, ES));
  const auto Kr = make_rsrc((const T *)p.k + koff, span_bytes(p.Sk, p.k_ss, D, ES));
  const auto Vr = make_rsrc((const T *)p.v + koff, span_bytes(p.Sk, p.k_ss, D, ES));
  const uint32_t qrow_b = (uint32_t)(p.q_ss * ES);
  const int64_t rbase = ((int64_t)b * p.H + h) * p.Sq;

  // K and V rows of this lane's key: B operands of Q K^T and dO V^T
  u32x4 kf[KS], vf[KS];
  {
    const uint32_t off = my_j < p.Sk ? (uint32_t)((int64_t)my_j * p.k_ss * ES) : 0x80000000u;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      kf[t] = buf_load16(Kr, off + (16 * t + 8 * g) * ES);
      vf[t] = buf_load16(Vr, off + (16 * t + 8 * g) * ES);
    }
  }
  f32x16 dv[DB], dk[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dv[db] = dk[db] = f32x16{};

  const float c_log2 = p.scale_log2;
  const float sl2 = alibi ? p.alibi_slopes[h] * kLog2e : 0.f;

  const int it_begin = causal ? (j0 / QB) : 0;
  const int it_end = (p.Sq + QB - 1) / QB;

  // staging: Q and dO tiles go straight to LDS (rows past S_q read as zeros);
  // LSE and delta of the block pass through 32 lanes' registers.  The loaded
  // values are first used when they are stored to LDS at the end of the step
  // (nothing reads them earlier), so the step never waits for the global
  // loads it has just issued.
  float st_lse = 0.f, st_dlt = 0.f;
  uint32_t voff[TileGeom<D, QB, NWB>::PER_WAVE];
  tile_offsets<D, QB, NWB>(voff, qrow_b, w, l);
  auto gload = [&](int it, uint16_t *qdst, uint16_t *gdst) {
    const uint32_t base = (uint32_t)it * QB * qrow_b;
    tile_load<D, QB, NWB>(qdst, Qr, voff, base, w);
    tile_load<D, QB, NWB>(gdst, Gr, voff, base, w);
    if (tid < QB) {
      const int i = it * QB + tid;
      st_lse = i < p.Sq ? p.lse[rbase + i] : -INFINITY;
      st_dlt = i < p.Sq ? p.delta[rbase + i] : 0.f;
    }
  };
  auto sstore = [&](int buf) {
    if (tid < QB) {
      const float ls = st_lse == -INFINITY ? INFINITY : st_lse * kLog2e;   // dead rows give P = 0
      lse_s[buf][tid] = ls;
      lam_s[buf][tid] = ls + sl2 * (float)tid;
      dlt_s[buf][tid] = st_dlt;
    }
  };

  // Query blocks come in two groups.  Fast blocks need no per-element work
  // for any key of the workgroup (full blocks, no mask tensors or dense bias,
  // and under ALiBi every row at or below every key), or, under the causal
  // rule, only the causal rule itself: the band of blocks on the diagonal,
  // which lead the range and whose steps mask per element.  They form the
  // range [f0, f1) and run software-pipelined.  The other blocks (the S_q
  // tail, masked problems, ALiBi without the causal rule near the diagonal)
  // run one block per step with per-wave classification.  The sums over
  // blocks do not depend on the order.
  static_assert(KB / QB == 4, "the masked steps cover a band of four blocks");
  int f0 = it_end, f1 = it_end;
  if (!f_elem && !dense && !DROP && j0 + KB <= p.Sk) {
    const int first = (alibi && !causal) ? max(it_begin, (j0 + KB - 1 + QB - 1) / QB) : it_begin;
    const int last = p.Sq / QB;   // full blocks only
    if (first < last) { f0 = first; f1 = last; }
  }
  const int n_lead = f0 - it_begin;            // generic blocks before the fast range
  const int n_gen = n_lead + (it_end - f1);    // and after it
  auto gen_at = [&](int n) { return n < n_lead ? it_begin + n : f1 + (n - n_lead); };

  // per-lane LDS byte offsets: Q/dO rows (A operands) and their transposed reads
  uint32_t ro[KS], to[2 * DB];
#pragma unroll
  for (int t = 0; t < KS; ++t) ro[t] = row_off<D>(lr, 2 * t + g);
#pragma unroll
  for (int db = 0; db < DB; ++db) tr_off<D>(&to[2 * db], 32 * db, l);

  // ==== generic blocks: one block per step (buffers 0 and 1)
  auto gen_step = [&](int n, auto buf) __attribute__((always_inline)) {
    constexpr int cur = decltype(buf)::value;
    const uint16_t *qs = cur ? Q1 : Q0;
    const uint16_t *gs = cur ? G1 : G0;
    const bool has_next = n + 1 < n_gen;
    if (has_next) gload(gen_at(n + 1), cur ? Q0 : Q1, cur ? G0 : G1);
    opaque(ro);
    opaque(to);
    const int i0 = gen_at(n) * QB;
    // wave-level class of the (32 queries x 32 keys) block: fast (no
    // per-element work) or general.  Blocks the mask hides wholly take the
    // general path, which yields P = dS = 0; keeping the accumulation
    // unconditional lets the dK/dV accumulators stay in place.
    bool general = dense || DROP || (jw + 32 > p.Sk) || (i0 + QB > p.Sq);
    if (causal && jw + 31 > i0) general = true;
    if (alibi && !(i0 >= jw + 31)) general = true;   // fast ALiBi form needs i >= j
    // padding, modality and explicit rules of the block's 32 queries for the
    // lane's key (bit c: query i0 + c may attend key my_j), from wave votes.  A
    // block they hide from every key of the wave is skipped (it adds nothing);
    // one they show wholly to every key needs no per-element work.
    uint32_t qm;
    bool skip = false;
    if (!f_elem) {   // the bounds alone
      const uint32_t rows = (uint32_t)__ballot(i0 + (l & 31) < p.Sq);
      qm = my_j < p.Sk ? rows : 0u;
    } else {
      bool key_ok = my_j < p.Sk;
      if (key_ok && (flags & FA_MASK_PADDING)) key_ok = p.key_valid[(int64_t)b * p.Sk + my_j] != 0;
      uint32_t col_allow = 0u;
      if ((flags & FA_MASK_MODALITY) && my_j < p.Sk) {
        const int mk = p.kmod[(int64_t)b * p.Sk + my_j];
        for (int mm = 0; mm < p.num_modalities; ++mm)
          col_allow |= (uint32_t)((p.allow_bits >> (8 * mm + mk)) & 1u) << mm;
      }
      qm = col_querymask(p, b, h, my_j, i0, key_ok, col_allow, l);
      const uint32_t own = 0x0F0F0F0Fu << (4 * g);   // this lane's queries' bits
      skip = __ballot((qm & own) != 0) == 0;
      if (__ballot((qm & own) != own) != 0) general = true;
    }
    if (!skip) {
      f32x16 s = f32x16{}, dp = f32x16{};
      // operand reads are issued in batches ahead of their MFMAs
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
      // element r: query i0 + il, il = 8(r/4) + 4g + r%4; key my_j
      if (!general) {
        const float L = sl2 * (float)(my_j - i0);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const f32x4 lam = *(const f32x4 *)&lam_s[cur][8 * rr + 4 * g];
          const f32x4 dl = *(const f32x4 *)&dlt_s[cur][8 * rr + 4 * g];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 4 * rr + q;
            const float pr = exp2_fast(fmaf(s[r], c_log2, L - lam[q]));
            s[r] = pr;
            dp[r] = pr * (dp[r] - dl[q]);
          }
        }
      } else {
        // dropout: the four lanes of a quad hold four consecutive keys and the
        // same 16 queries, so lane q of the quad draws the Philox words of the
        // queries with r % 4 == q (one call covers the quad's four keys), packs
        // the keep bits, and the quad exchanges them
        uint32_t kq[4] = {0u, 0u, 0u, 0u};
        if (DROP) {
          uint32_t mine = 0u;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            mine |= dropout_keep4(p, b, h, i0 + 8 * rr + 4 * g + (l & 3), my_j) << (4 * rr);
          // quad_perm broadcasts of lane 0, 1, 2, 3
          kq[0] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0x00, 0xF, 0xF, false);
          kq[1] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0x55, 0xF, 0xF, false);
          kq[2] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0xAA, 0xF, 0xF, false);
          kq[3] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0xFF, 0xF, 0xF, false);
#pragma unroll
          for (int q = 0; q < 4; ++q) kq[q] >>= (l & 3);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const f32x4 ls = *(const f32x4 *)&lse_s[cur][8 * rr + 4 * g];
          const f32x4 dl = *(const f32x4 *)&dlt_s[cur][8 * rr + 4 * g];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 4 * rr + q;
            const int i = i0 + 8 * rr + 4 * g + q;
            const bool ok = ((qm >> (8 * rr + 4 * g + q)) & 1u) && (!causal || my_j <= i);
            float pr = 0.f;
            if (ok) {
              float t = s[r] * c_log2;
              if (alibi) t -= sl2 * fabsf((float)(i - my_j));
              else if (dense) t += dense_bias(p, b, h, i, my_j) * kLog2e;
              pr = exp2_fast(t - ls[q]);
            }
            // dropout: P o M / keep_prob feeds dV, and dP is masked the same way
            const float m = DROP ? dropout_scale(p, (kq[q] >> (4 * rr)) & 1u) : 1.f;
            s[r] = pr * m;
            dp[r] = pr * (dp[r] * m - dl[q]);
          }
        }
        if (EXTRA && p.dpse) {
          // bias gradient: dS itself, before it is rounded for the products
          float *dst = p.dpse + ((int64_t)(b * p.H + h) * p.Sq) * p.Sk + my_j;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = i0 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (i < p.Sq && my_j < p.Sk) dst[(int64_t)i * p.Sk] = dp[r];
          }
        }
      }
      // dV += P^T dO, dK += dS^T Q, contraction over the 32 queries
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x4 pp = pack8<T>(s, 8 * c);
        const u32x4 pd = pack8<T>(dp, 8 * c);
        u32x4 gt[DB], qt[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          gt[db] = read_tr_at<D>(gs, c, &to[2 * db]);
          qt[db] = read_tr_at<D>(qs, c, &to[2 * db]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[db] = Mfma<T>::mac(pp, gt[db], dv[db]);
          dk[db] = Mfma<T>::mac(pd, qt[db], dk[db]);
        }
      }
    }
    if (has_next) sstore(cur ^ 1);
    vm_wait_barrier();
  };

  if (n_gen > 0) {
    gload(gen_at(0), Q0, G0);
    sstore(0);
  }
  vm_wait_barrier();
  {
    int n = 0;
    for (; n + 1 < n_gen; n += 2) {
      gen_step(n, BufIdx<0>{});
      gen_step(n + 1, BufIdx<1>{});
    }
    if (n < n_gen) gen_step(n, BufIdx<0>{});
  }

  // ==== fast blocks: software pipeline over [f0, f1).  Block n sits in
  // buffer n % 3; step n computes S and dP of block n+1 (A = its Q / dO rows)
  // interleaved with P and dS of block n (whose scores came from the
  // previous step), then dV += P^T dO and dK += dS^T Q of block n (transposed
  // reads of its tiles), while block n+2 loads into the third buffer.
  const int n_fast = f1 - f0;
  f32x16 sA = f32x16{}, dpA = f32x16{}, sB = f32x16{}, dpB = f32x16{};
  // S and dP of the block in buffers (qs, gs), operand reads batched ahead
  auto scores = [&](const uint16_t *qs, const uint16_t *gs, f32x16 &s, f32x16 &dp)
                    __attribute__((always_inline)) {
    s = dp = f32x16{};
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
  if (n_fast > 0) {
    gload(f0, Q0, G0);
    sstore(0);
    if (n_fast > 1) {
      gload(f0 + 1, Q1, G1);
      sstore(1);
    }
  }
  vm_wait_barrier();
  // row statistics (LSE term, delta) of the block in flight, in registers
  f32x4 lmA[4], dlA[4], lmB[4], dlB[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    lmA[rr] = *(const f32x4 *)&lam_s[0][8 * rr + 4 * g];
    dlA[rr] = *(const f32x4 *)&dlt_s[0][8 * rr + 4 * g];
  }
  if (n_fast > 0) scores(Q0, G0, sA, dpA);

  // MASK: the causal rule per element (P = 0 for a key past its query);
  // on a block wholly below the diagonal it changes nothing.
  auto fast_step = [&](int n, auto buf, f32x16 &s, f32x16 &dp, f32x16 &sn, f32x16 &dpn,
                       f32x4 (&lam)[4], f32x4 (&dl)[4], f32x4 (&lamn)[4], f32x4 (&dln)[4],
                       auto mask) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask)::value;
    constexpr int B = decltype(buf)::value, N1 = (B + 1) % 3, N2 = (B + 2) % 3;
    const uint16_t *qs = B == 0 ? Q0 : B == 1 ? Q1 : Q2;      // block n
    const uint16_t *gs = B == 0 ? G0 : B == 1 ? G1 : G2;
    const uint16_t *qn = N1 == 0 ? Q0 : N1 == 1 ? Q1 : Q2;    // block n+1
    const uint16_t *gn = N1 == 0 ? G0 : N1 == 1 ? G1 : G2;
    const bool has_next2 = n + 2 < n_fast;
    if (has_next2) gload(f0 + n + 2, N2 == 0 ? Q0 : N2 == 1 ? Q1 : Q2, N2 == 0 ? G0 : N2 == 1 ? G1 : G2);
    opaque(ro);
    opaque(to);
    const int i0 = (f0 + n) * QB;
    const float L = sl2 * (float)(my_j - i0);
    // element r holds query i0 + 4g + c, c = 8(r/4) + r%4: masked when c < lim
    const int lim = causal ? my_j - i0 - 4 * g : INT_MIN;
    // Order fixed by scheduling fences (only scalar work may cross them): the
    // first half of the next block's operand reads up front, the rest one
    // k-step before they are needed; per k-step its two score products, then
    // two elements of this block's P and dS (which do not depend on them);
    // the transposed reads of this block's two 16-query chunks go out at the
    // second k-step and half way, and the next block's row statistics during
    // this block's last dV / dK products.  On the last step the next block's
    // scores and statistics come from stale buffers and are unused.
    u32x4 qa[KS], ga[KS];
#pragma unroll
    for (int t = 0; t < KS / 2; ++t) {
      qa[t] = read_row_at<D>(qn, 0, ro[t]);
      ga[t] = read_row_at<D>(gn, 0, ro[t]);
    }
    __builtin_amdgcn_sched_barrier(0x0004);
    sn = dpn = f32x16{};
    u32x4 gt[2][DB], qt[2][DB];
    constexpr int EPS = 16 / KS;   // elements of P / dS per k-step
    constexpr int DBS = 2 * DB / KS;   // chunk-0 d-blocks of dV / dK per late k-step
    u32x4 pp0, pd0;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      if (t == KS / 2 - 1) {
#pragma unroll
        for (int u = KS / 2; u < KS; ++u) {
          qa[u] = read_row_at<D>(qn, 0, ro[u]);
          ga[u] = read_row_at<D>(gn, 0, ro[u]);
        }
      }
      if (t == 1 || t == KS / 2) {
        const int c = t == 1 ? 0 : 1;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          gt[c][db] = read_tr_at<D>(gs, c, &to[2 * db]);
          qt[c][db] = read_tr_at<D>(qs, c, &to[2 * db]);
        }
      }
      sn = Mfma<T>::mac(qa[t], kf[t], sn);
      dpn = Mfma<T>::mac(ga[t], vf[t], dpn);
      if (t >= KS / 2) {
        // chunk 0 (elements 0..7) is complete: its dV / dK products fill the
        // second half of the k-steps
        if (t == KS / 2) {
          pp0 = pack8<T>(s, 0);
          pd0 = pack8<T>(dp, 0);
        }
#pragma unroll
        for (int db = (t - KS / 2) * DBS; db < (t - KS / 2 + 1) * DBS; ++db) {
          dv[db] = Mfma<T>::mac(pp0, gt[0][db], dv[db]);
          dk[db] = Mfma<T>::mac(pd0, qt[0][db], dk[db]);
        }
      }
#pragma unroll
      for (int r = t * EPS; r < (t + 1) * EPS; ++r) {
        float pr = exp2_fast(fmaf(s[r], c_log2, L - lam[r >> 2][r & 3]));
        if (MASK) pr = 8 * (r >> 2) + (r & 3) < lim ? 0.f : pr;
        s[r] = pr;
        dp[r] = pr * (dp[r] - dl[r >> 2][r & 3]);
      }
      __builtin_amdgcn_sched_barrier(0x0004);
    }
    // the next block's row statistics, then chunk 1's dV / dK products
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      lamn[rr] = *(const f32x4 *)&lam_s[N1][8 * rr + 4 * g];
      dln[rr] = *(const f32x4 *)&dlt_s[N1][8 * rr + 4 * g];
    }
    {
      const u32x4 pp = pack8<T>(s, 8);
      const u32x4 pd = pack8<T>(dp, 8);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dv[db] = Mfma<T>::mac(pp, gt[1][db], dv[db]);
        dk[db] = Mfma<T>::mac(pd, qt[1][db], dk[db]);
      }
      __builtin_amdgcn_sched_barrier(0x0004);
    }
    if (has_next2) sstore(N2);
    vm_wait_barrier();
  };
  // the first four steps (the causal band, when the range starts there) mask
  // per element; then six steps per trip: three buffers times two register sets
  const std::bool_constant<true> masked;
  const std::bool_constant<false> plain;
  if (n_fast > 0) fast_step(0, BufIdx<0>{}, sA, dpA, sB, dpB, lmA, dlA, lmB, dlB, masked);
  if (n_fast > 1) fast_step(1, BufIdx<1>{}, sB, dpB, sA, dpA, lmB, dlB, lmA, dlA, masked);
  if (n_fast > 2) fast_step(2, BufIdx<2>{}, sA, dpA, sB, dpB, lmA, dlA, lmB, dlB, masked);
  if (n_fast > 3) fast_step(3, BufIdx<0>{}, sB, dpB, sA, dpA, lmB, dlB, lmA, dlA, masked);
  for (int n = 4; n < n_fast; n += 6) {
    fast_step(n, BufIdx<1>{}, sA, dpA, sB, dpB, lmA, dlA, lmB, dlB, plain);
    if (n + 1 < n_fast) fast_step(n + 1, BufIdx<2>{}, sB, dpB, sA, dpA, lmB, dlB, lmA, dlA, plain);
    if (n + 2 < n_fast) fast_step(n + 2, BufIdx<0>{}, sA, dpA, sB, dpB, lmA, dlA, lmB, dlB, plain);
    if (n + 3 < n_fast) fast_step(n + 3, BufIdx<1>{}, sB, dpB, sA, dpA, lmB, dlB, lmA, dlA, plain);
    if (n + 4 < n_fast) fast_step(n + 4, BufIdx<2>{}, sA, dpA, sB, dpB, lmA, dlA, lmB, dlB, plain);
    if (n + 5 < n_fast) fast_step(n + 5, BufIdx<0>{}, sB, dpB, sA, dpA, lmB, dlB, lmA, dlA, plain);
  }

  // dK (scaled) and dV; element r: key jw + 8(r/4) + 4g + r%4, column 32db + lr
  if (EXTRA && p.grad_f32) {
    float *DKg = (float *)p.dk + koff;
    float *DVg = (float *)p.dv + koff;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jw + 8 * (r >> 2) + 4 * g + (r & 3);
        if (j < p.Sk) {
          DKg[(int64_t)j * p.k_ss + 32 * db + lr] = dk[db][r] * p.scale;
          DVg[(int64_t)j * p.k_ss + 32 * db + lr] = dv[db][r];
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
        DKg[(int64_t)j * p.k_ss + 32 * db + lr] = from_f32<T>(dk[db][r] * p.scale);
        DVg[(int64_t)j * p.k_ss + 32 * db + lr] = from_f32<T>(dv[db][r]);
      }
    }
  }
}

// ===========================================================================
// query pass: dQ
template <typename T, int D, bool DROP, bool EXTRA>
__global__ __launch_bounds__(256, 2) void bwd_q_kernel(Params p, int n_qtiles) {
  constexpr int KS = D / 16, DB = D / 32, CH = D / 8;
  constexpr int QRB = 2;   // k-steps of K / V row operands read ahead of their MFMAs
  constexpr int ES = (int)sizeof(T);
  // each buffer its own LDS variable, named statically by every access: the
  // compiler's wait-count pass can then tell a read of the current tile from
  // the next tile's loads in flight
  __shared__ __attribute__((aligned(16))) uint16_t K0[KBQ * D], K1[KBQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t V0[KBQ * D], V1[KBQ * D];

  const int BH = p.B * p.H;
  const int lin = blockIdx.x;
  const int qt = n_qtiles - 1 - lin / BH;   // longest causal rows first
  const int bh = lin % BH;
  const int b = bh / p.H, h = bh % p.H;
  const int q0 = qt * QBQ;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int l = tid & 63, g = l >> 5, lr = l & 31;
  const int qw = q0 + 32 * w;
  const int my_i = qw + lr;
  const uint32_t flags = p.mask_flags;
  const bool causal = flags & FA_MASK_CAUSAL;
  const bool alibi = p.pse_kind == FA_PSE_ALIBI, dense = p.pse_kind == FA_PSE_DENSE;
  const bool f_elem = flags & (FA_MASK_PADDING | FA_MASK_MODALITY | FA_MASK_EXPLICIT);

  const int64_t qoff = b * p.q_sb + h * p.q_sh;
  const int64_t koff = b * p.k_sb + h * p.k_sh;
  const auto Qr = make_rsrc((const T *)p.q + qoff, span_bytes(p.Sq, p.q_ss, D, ES));
  const auto Gr = make_rsrc((const T *)p.dout + qoff, span_bytes(p.Sq, p.q_ss, D, ES));
  const auto Kr = make_rsrc((const T *)p.k + koff, span_bytes(p.Sk, p.k_ss, D, ES));
  const auto Vr = make_rsrc((const T *)p.v + koff, span_bytes(p.Sk, p.k_ss, D, ES));
  const uint32_t krow_b = (uint32_t)(p.k_ss * ES);
  const int64_t rbase = ((int64_t)b * p.H + h) * p.Sq;

  // this lane's query row: Q and dO as B operands, LSE and delta
  u32x4 qf[KS], gf[KS];
  {
    const uint32_t off = my_i < p.Sq ? (uint32_t)((int64_t)my_i * p.q_ss * ES) : 0x80000000u;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      qf[t] = buf_load16(Qr, off + (16 * t + 8 * g) * ES);
      gf[t] = buf_load16(Gr, off + (16 * t + 8 * g) * ES);
    }
  }
  float lse2 = INFINITY, dlt = 0.f;
  if (my_i < p.Sq) {
    const float v = p.lse[rbase + my_i];
    lse2 = (v == -INFINITY) ? INFINITY : v * kLog2e;
    dlt = p.delta[rbase + my_i];
  }

  const float c_log2 = p.scale_log2;
  const float sl2 = alibi ? p.alibi_slopes[h] * kLog2e : 0.f;
  const float sl2c = alibi ? sl2 / c_log2 : 0.f;
  // Start values of the fast modes' accumulators (the lane's query is fixed):
  // S starts at the ALiBi term of the element's key offset within its 32-key
  // block in raw units (the block's own offset goes into the logit's offset),
  // dP at -delta, so P is one fma and an exponential and dS one multiply.
  f32x16 s_init, dp_init;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s_init[r] = sl2c * (float)(8 * (r >> 2) + (r & 3));
    dp_init[r] = -dlt;
  }

  int k_hi = p.Sk;
  if (causal) k_hi = min(k_hi, q0 + QBQ);
  const int kt_end = (k_hi + KBQ - 1) / KBQ;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  // K and V tiles go straight to LDS; rows past S_k read as zeros
  uint32_t voff[TileGeom<D, KBQ, NWB>::PER_WAVE];
  tile_offsets<D, KBQ, NWB>(voff, krow_b, w, l);
  auto gload = [&](int kt, uint16_t *kdst, uint16_t *vdst) {
    const uint32_t base = (uint32_t)kt * KBQ * krow_b;
    tile_load<D, KBQ, NWB>(kdst, Kr, voff, base, w);
    tile_load<D, KBQ, NWB>(vdst, Vr, voff, base, w);
  };

  // per-lane LDS byte offsets: K/V rows (A operands) and K^T reads
  uint32_t ro[KS], to[2 * DB];
#pragma unroll
  for (int t = 0; t < KS; ++t) ro[t] = row_off<D>(lr, 2 * t + g);
#pragma unroll
  for (int db = 0; db < DB; ++db) tr_off<D>(&to[2 * db], 32 * db, l);

  // One key tile per step.  Mode 2 (GEN): the per-element (general) code is
  // compiled in; the fast modes carry none of it, which keeps their register
  // footprint within two waves per SIMD.  Mode 1 (BAND): a fast tile on the
  // causal diagonal, where the causal rule zeroes P for keys above each row
  // (every visible key is at or below the row, so the fast ALiBi form holds).
  // The LDS offsets pass through an empty asm statement each step, so one set
  // of offset registers serves both buffers.
  auto body = [&](int kt, const uint16_t *ks, const uint16_t *vs, auto mode)
                  __attribute__((always_inline)) {
    constexpr bool GEN = decltype(mode)::value == 2;
    constexpr bool BAND = decltype(mode)::value == 1;
    const int k0 = kt * KBQ;
    // fast or general tile; tiles hidden from this wave (at most one per
    // workgroup on the causal diagonal) take the general path (dS = 0) so the
    // accumulation stays unconditional
    // (the fast ALiBi form folds slope / c_log2 into raw scores: c_log2 > kRawMinC)
    // (in the general phase dropout keeps every tile on the per-element code,
    // whose fast-tile branch draws no keep mask)
    bool general = dense || (GEN && DROP) || (k0 + KBQ > p.Sk) || (qw + 32 > p.Sq) ||
                   (alibi && !(c_log2 > kRawMinC));
    if (causal && k0 + KBQ - 1 > qw) general = true;
    if (alibi && !(k0 + KBQ - 1 <= qw)) general = true;
    // padding and modality rules over the wave's 32 rows and the tile's 64 keys,
    // from wave votes: a tile they hide wholly is skipped, one they show wholly
    // needs no per-element work (an explicit mask always takes the per-element
    // code)
    bool skip = false;
    // padding and modality rules for this lane's row against the tile's keys,
    // from the same votes (lane l votes for key k0 + l): bit jj says key
    // k0 + jj exists, is valid and its modality is allowed to the row (or it
    // is the row's own position under the diagonal rule)
    uint64_t kmask = ~0ull;
    if (GEN && f_elem) {
      static_assert(KBQ == 64, "one key per lane");
      const int j = k0 + l;
      const bool in = j < p.Sk;
      bool kv = in;
      if (in && (flags & FA_MASK_PADDING)) kv = p.key_valid[(int64_t)b * p.Sk + j] != 0;
      const uint64_t kvm = __ballot(kv);
      kmask = kvm;
      bool any = kvm != 0;
      bool full = !(flags & FA_MASK_EXPLICIT) && kvm == __ballot(in);
      if (flags & FA_MASK_MODALITY) {
        const int mk = kv ? p.kmod[(int64_t)b * p.Sk + j] : -1;
        const int mq = my_i < p.Sq ? p.qmod[(int64_t)b * p.Sq + my_i] : -1;
        const uint32_t my_row = mq >= 0 ? (uint32_t)(p.allow_bits >> (8 * mq)) & 0xffu : 0u;
        uint64_t mm = 0ull;
        for (int c = 0; c < p.num_modalities; ++c) {
          const uint64_t kc = __ballot(mk == c);
          if (kc != 0ull && ((my_row >> c) & 1u)) mm |= kc;
        }
        const int d = my_i - k0;
        if (p.allow_diag && d >= 0 && d < KBQ) mm |= 1ull << d;
        kmask = kvm & mm;
        bool some = false, all = true;
        for (int a = 0; a < p.num_modalities; ++a) {
          if (!__ballot(mq == a)) continue;
          const uint32_t row = (uint32_t)(p.allow_bits >> (8 * a)) & 0xffu;
          for (int c = 0; c < p.num_modalities; ++c) {
            if (!__ballot(mk == c)) continue;
            if ((row >> c) & 1u) some = true;
            else all = false;
          }
        }
        const bool diag = p.allow_diag && k0 < qw + 32 && k0 + KBQ > qw;
        if (!some && !diag) any = false;
        if (!all || diag) full = false;
      }
      skip = !any;
      if (!full) general = true;
    } else if (f_elem) {
      general = true;
    }
    if (!GEN) general = false;   // the fast phase only visits tiles fast for every wave
    if (qw >= p.Sq) skip = true;   // a wave past the last query row has nothing to add
    if (!skip) {
      const float off = (alibi ? sl2 * (float)(k0 + 4 * g - my_i) : 0.f) - lse2;
      // one 32-key block at a time (LSE is known: no row max to wait for)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        f32x16 s, dp;
        if constexpr (GEN) {
          s = dp = f32x16{};
        } else {
          s = s_init;
          if constexpr (DROP) dp = f32x16{};   // the keep mask scales dP before delta
          else dp = dp_init;
        }
        // fast steps: MFMA runs at raised issue priority, so the other wave on
        // the SIMD fills their gaps with its VALU work
        if (!GEN) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t0 = 0; t0 < KS; t0 += QRB) {
          u32x4 ka[QRB], va[QRB];
#pragma unroll
          for (int t = 0; t < QRB; ++t) {
            ka[t] = read_row_at<D>(ks, 32 * jb, ro[t0 + t]);
            va[t] = read_row_at<D>(vs, 32 * jb, ro[t0 + t]);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int t = 0; t < QRB; ++t) {
            s = Mfma<T>::mac(ka[t], qf[t0 + t], s);
            dp = Mfma<T>::mac(va[t], gf[t0 + t], dp);
          }
        }
        if (!GEN) __builtin_amdgcn_s_setprio(0);
        // element r: key k0 + 32jb + 8(r/4) + 4g + r%4, query my_i
        if (!general) {
          const int lim = my_i - k0 - 4 * g;   // BAND: keys past the row have c > lim
          const float offj = jb ? fmaf(32.f, sl2, off) : off;
          // dropout: keys 4t .. 4t + 3 of a register group share one Philox call
          uint32_t keep[4] = {0u, 0u, 0u, 0u};
          if constexpr (DROP && !GEN) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              keep[rr] = dropout_keep4(p, b, h, my_i, k0 + 32 * jb + 8 * rr + 4 * g);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 32 * jb + 8 * (r >> 2) + (r & 3);
            float pr;
            if constexpr (GEN) {
              float u = s[r];
              if (alibi) u = fmaf(sl2c, (float)c, u);
              pr = exp2_fast(fmaf(u, c_log2, off));
              dp[r] = dp[r] - dlt;
            } else {
              pr = exp2_fast(fmaf(s[r], c_log2, offj));   // S carries its start value
              if constexpr (DROP) {
                const float m = dropout_scale(p, (keep[r >> 2] >> (r & 3)) & 1u);
                dp[r] = dp[r] * m - dlt;   // dropout masks dP like P
              }
            }
            if (BAND) pr = c > lim ? 0.f : pr;
            dp[r] = pr * dp[r];
          }
        } else if constexpr (GEN) {
          // keys 4t .. 4t + 3 of a register group share one Philox call
          uint32_t keep[4] = {0u, 0u, 0u, 0u};
          if (DROP) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              keep[rr] = dropout_keep4(p, b, h, my_i, k0 + 32 * jb + 8 * rr + 4 * g);
          }
          // the lane's keys of this block sit at bits 8 (r / 4) + r % 4 of kw
          const uint32_t kw = (uint32_t)((kmask >> (4 * g)) >> (32 * jb));
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = k0 + 32 * jb + 8 * (r >> 2) + 4 * g + (r & 3);
            bool ok = j < p.Sk && my_i < p.Sq && ((kw >> (8 * (r >> 2) + (r & 3))) & 1u);
            if (causal) ok = ok && j <= my_i;
            if (ok && (flags & FA_MASK_EXPLICIT))
              ok = p.em[(int64_t)b * p.em_sb + (int64_t)h * p.em_sh + (int64_t)my_i * p.em_sq + j] != 0;
            float pr = 0.f;
            if (ok) {
              float t = s[r] * c_log2;
              if (alibi) t -= sl2 * fabsf((float)(my_i - j));
              else if (dense) t += dense_bias(p, b, h, my_i, j) * kLog2e;
              pr = exp2_fast(t - lse2);
            }
            const float m = DROP ? dropout_scale(p, (keep[r >> 2] >> (r & 3)) & 1u) : 1.f;
            dp[r] = pr * (dp[r] * m - dlt);   // dropout masks dP like P
          }
        }
        // dQ^T += K^T . dS^T over this block's two 16-key chunks
        if (!GEN) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const u32x4 pd = pack8<T>(dp, 8 * hh);
          u32x4 kop[DB];
#pragma unroll
          for (int db = 0; db < DB; ++db) kop[db] = read_tr_at<D>(ks, 2 * jb + hh, &to[2 * db]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db] = Mfma<T>::mac(kop[db], pd, acc[db]);
        }
        if (!GEN) __builtin_amdgcn_s_setprio(0);
      }
    }
    vm_wait_barrier();
  };

  // fast range [0, f_end): full tiles every row of the workgroup sees whole
  // (below the causal diagonal; ALiBi direction +1), without mask tensors or
  // dense bias.  Under the causal rule alone the full tiles on the
  // diagonal, [f_end, b_end), run the fast code with the causal mask (it needs
  // c_log2 > 0); the rest, [b_end, kt_end), take the general code.  Those two
  // groups go first, one per step.
  int f_end = 0, b_end = 0;
  if (!f_elem && !dense && q0 + QBQ <= p.Sq && (!alibi || c_log2 > kRawMinC)) {
    f_end = min(kt_end, p.Sk / KBQ);
    b_end = f_end;
    if (causal || alibi) f_end = min(f_end, (q0 + 1) / KBQ);
    if (!causal || !(c_log2 > 0.f)) b_end = f_end;
  }
  f_end = __builtin_amdgcn_readfirstlane(f_end);
  b_end = __builtin_amdgcn_readfirstlane(b_end);
  if (f_end < kt_end) gload(f_end, K0, V0);
  vm_wait_barrier();
  int cur = 0;
  for (int kt = f_end; kt < b_end; ++kt, cur ^= 1) {
    opaque(ro);
    opaque(to);
    if (kt + 1 < kt_end) gload(kt + 1, cur ? K0 : K1, cur ? V0 : V1);
    body(kt, cur ? K1 : K0, cur ? V1 : V0, std::integral_constant<int, 1>{});
  }
  for (int kt = b_end; kt < kt_end; ++kt, cur ^= 1) {
    opaque(ro);
    opaque(to);
    if (kt + 1 < kt_end) gload(kt + 1, cur ? K0 : K1, cur ? V0 : V1);
    body(kt, cur ? K1 : K0, cur ? V1 : V0, std::integral_constant<int, 2>{});
  }
  if (f_end > 0) {
    gload(0, K0, V0);
    vm_wait_barrier();
  }
  auto fstep = [&](int kt, auto buf) __attribute__((always_inline)) {
    constexpr int B = decltype(buf)::value;
    opaque(ro);
    opaque(to);
    if (kt + 1 < f_end) gload(kt + 1, B ? K0 : K1, B ? V0 : V1);
    body(kt, B ? K1 : K0, B ? V1 : V0, std::integral_constant<int, 0>{});
  };
  {
    int kt = 0;
    for (; kt + 1 < f_end; kt += 2) {
      fstep(kt, BufIdx<0>{});
      fstep(kt + 1, BufIdx<1>{});
    }
    if (kt < f_end) fstep(kt, BufIdx<0>{});
  }

  // dQ = scale * acc; element (db, r): column 32db + 8(r/4) + 4g + r%4
  if (EXTRA && my_i < p.Sq && p.grad_f32) {
    float *Dg = (float *)p.dq + qoff + (int64_t)my_i * p.q_ss;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * g;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[db][4 * rr + e] * p.scale;
        *(f32x4 *)(Dg + d0) = v;
      }
    }
  } else if (my_i < p.Sq) {
    T *Dg = (T *)p.dq + qoff + (int64_t)my_i * p.q_ss;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * g;
        u32x2 v;
        v[0] = pack2<T>(acc[db][4 * rr + 0] * p.scale, acc[db][4 * rr + 1] * p.scale);
        v[1] = pack2<T>(acc[db][4 * rr + 2] * p.scale, acc[db][4 * rr + 3] * p.scale);
        *(u32x2 *)(Dg + d0) = v;
      }
    }
  }
}

// Zeros n floats (16-byte aligned): the bias gradient of pairs the key pass
// never visits.  A kernel rather than a memset, so the call stays safe to
// capture in a graph.
__global__ __launch_bounds__(256) void zero_f32_kernel(float *dst, int64_t n) {
  const int64_t n4 = n >> 2;
  for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < n4; k += (int64_t)gridDim.x * 256)
    ((f32x4 *)dst)[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) dst[4 * n4 + threadIdx.x] = 0.f;
}

template <typename T, int D>
hipError_t launch_kv(const Params &p, hipStream_t s) {
  const int n_ktiles = (p.Sk + KB - 1) / KB;
  const int64_t blocks = (int64_t)n_ktiles * p.B * p.H;
  if (p.dpse) {
    const int64_t n = (int64_t)p.B * p.H * p.Sq * p.Sk;
    if (n > 0) {
      const int64_t grid = std::min<int64_t>((n / 4 + 255) / 256 + 1, 4096);
      hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)grid), dim3(256), 0, s, p.dpse, n);
    }
  }
  if (blocks == 0) return hipGetLastError();
  const bool extra = p.grad_f32 || p.dpse;
  const dim3 grid((unsigned)blocks), block(NWB * 64);
  if (log_enabled()) {
    char name[96];
    snprintf(name, sizeof(name), "bwd_kv_kernel<D=%d%s%s> (one-role key pass)", D,
             p.dropout ? ", DROP" : "", extra ? ", EXTRA" : "");
    log_launch("fa_bwd_main", name, (long long)blocks, NWB * 64, p);
  }
  if (p.dropout) {
    if (extra) hipLaunchKernelGGL((bwd_kv_kernel<T, D, true, true>), grid, block, 0, s, p, n_ktiles);
    else hipLaunchKernelGGL((bwd_kv_kernel<T, D, true, false>), grid, block, 0, s, p, n_ktiles);
  } else {
    if (extra) hipLaunchKernelGGL((bwd_kv_kernel<T, D, false, true>), grid, block, 0, s, p, n_ktiles);
    else hipLaunchKernelGGL((bwd_kv_kernel<T, D, false, false>), grid, block, 0, s, p, n_ktiles);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_q(const Params &p, hipStream_t s) {
  const int n_qtiles = (p.Sq + QBQ - 1) / QBQ;
  const int64_t blocks = (int64_t)n_qtiles * p.B * p.H;
  if (blocks == 0) return hipSuccess;
  const bool extra = p.grad_f32 != 0;
  const dim3 grid((unsigned)blocks), block(NWB * 64);
  if (log_enabled()) {
    char name[96];
    snprintf(name, sizeof(name), "bwd_q_kernel<D=%d%s%s> (query pass)", D,
             p.dropout ? ", DROP" : "", extra ? ", EXTRA" : "");
    log_launch("fa_bwd_post", name, (long long)blocks, NWB * 64, p);
  }
  if (p.dropout) {
    if (extra) hipLaunchKernelGGL((bwd_q_kernel<T, D, true, true>), grid, block, 0, s, p, n_qtiles);
    else hipLaunchKernelGGL((bwd_q_kernel<T, D, true, false>), grid, block, 0, s, p, n_qtiles);
  } else {
    if (extra) hipLaunchKernelGGL((bwd_q_kernel<T, D, false, true>), grid, block, 0, s, p, n_qtiles);
    else hipLaunchKernelGGL((bwd_q_kernel<T, D, false, false>), grid, block, 0, s, p, n_qtiles);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_zero_words(void *dst, int64_t n_words, hipStream_t s) {
  if (n_words <= 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>((n_words / 4 + 255) / 256 + 1, 4096);
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)grid), dim3(256), 0, s, (float *)dst, n_words);
  return hipGetLastError();
}

hipError_t launch_bwd_kv_mfma(const Params &p, int dtype, hipStream_t s) {
  if (bwd_kv_split_eligible(p)) return launch_bwd_kv_split(p, dtype, s);
  if (dtype == FA_BF16) {
    if (p.D == 64) return launch_kv<__bf16, 64>(p, s);
    if (p.D == 128) return launch_kv<__bf16, 128>(p, s);
  } else if (dtype == FA_F16) {
    if (p.D == 64) return launch_kv<_Float16, 64>(p, s);
    if (p.D == 128) return launch_kv<_Float16, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_q_mfma(const Params &p, int dtype, hipStream_t s) {
  if (dtype == FA_BF16) {
    if (p.D == 64) return launch_q<__bf16, 64>(p, s);
    if (p.D == 128) return launch_q<__bf16, 128>(p, s);
  } else if (dtype == FA_F16) {
    if (p.D == 64) return launch_q<_Float16, 64>(p, s);
    if (p.D == 128) return launch_q<_Float16, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
