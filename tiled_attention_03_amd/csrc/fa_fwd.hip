// Forward attention, bf16/f16 inputs, MFMA on gfx950 (CDNA4).
//
// What is computed: O = Softmax(Q K^T * scale + mask + pse) V and the row
// log-sum-exp, tile by tile with an online softmax so the S_q x S_k score
// matrix never leaves registers (FlashAttentionScore replacement guide,
// section 2; the tile loop and running statistics are the "tiling + online
// softmax" of its section 1 and of the NPU FlashAttention study's flow
// description).
//
// Workgroup = NW waves, two workgroups per CU (two waves per SIMD).  Each
// wave owns 32 query rows; the workgroup's BM = 32*NW rows share one stream
// of K/V tiles of BN = 64 keys.  The products are arranged so that a lane
// owns ONE query row for the whole kernel:
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
// modality all rows may attend); the rest are "generic" (the causal diagonal
// band, the S_k tail, explicit masks, dense bias, ...).  Tiles no row can see
// are dropped.
//
//   generic phase: one tile per step; each wave classifies the tile for its
//     own rows (nothing visible: skip; no element work: fast; else per-element
//     mask and bias) and runs  S = K Q^T, softmax, O += P V  in sequence.
//   fast phase: a software pipeline with no branches on the tile class.  Step
//     n computes the scores of tile n+1 (MFMA) interleaved with the
//     exponentials of tile n (VALU), in an order fixed by scheduling fences,
//     then multiplies P_n by V_n; K tiles are fetched two steps ahead and V
//     tiles one step ahead.
//
// Tiles go straight from global memory into LDS (no register staging).  Each
// of the four tile buffers is its own LDS variable and steps are unrolled in
// pairs, so every LDS read names its buffer statically and never waits for
// the loads in flight to the others.  Within each phase, tiles are visited
// from the last one down: under ALiBi the largest logits (keys nearest the
// diagonal) come first, so the running max settles early and the lazy
// rescale rarely fires.
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int BN = 64;          // keys per tile
constexpr int kMaxTiles = 512;  // key tiles summarised in LDS (S_k <= 32768)
constexpr float kTau = 8.f;     // rescale O only when a row max grows by more than this (log2)

template <typename T, int D, int NW>
struct FwdCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = 32 * NW;       // query rows per workgroup
  static constexpr int KS = D / 16;        // k-steps of Q K^T
  static constexpr int DB = D / 32;        // 32-row blocks of O^T
};

// Tile class for one wave: what the wave does with the tile's scores.
enum : int { kFast = 0, kGeneral = 1, kDead = 2 };

template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void fwd_mfma_kernel(Params p, int n_qtiles) {
  using C = FwdCfg<T, D, NW>;
  constexpr int KS = C::KS, DB = C::DB;
  __shared__ __attribute__((aligned(16))) uint16_t K0[BN * D], K1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t V0[BN * D], V1[BN * D];
  __shared__ int kv_range[2];
  __shared__ uint32_t wg_any, wg_all;   // modalities some / every row of the workgroup may attend
  __shared__ int n_list[2];             // generic tiles, all visited tiles
  __shared__ uint32_t tsum[kMaxTiles];  // per key tile: bits 0-7 modality set of valid keys,
                                        // bit 8 some key invalid or past S_k
  __shared__ int16_t tlist[kMaxTiles];  // generic tiles, then fast tiles

  const int BH = p.B * p.H;
  const int lin = blockIdx.x;
  const int qt = n_qtiles - 1 - lin / BH;   // longest causal rows first
  const int bh = lin % BH;
  const int b = bh / p.H, h = bh % p.H;
  const int q0 = qt * C::BM;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int l = tid & 63, g = l >> 5, lr = l & 31;
  const int qw = q0 + 32 * w;   // first row of this wave
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
  u32x4 qf[KS];
  {
    const uint32_t qoff = my_i < p.Sq ? (uint32_t)((int64_t)my_i * p.q_ss * ES) : 0x80000000u;
#pragma unroll
    for (int t = 0; t < KS; ++t) qf[t] = buf_load16(Qr, qoff + (16 * t + 8 * g) * ES);
  }

  const bool alibi = p.pse_kind == FA_PSE_ALIBI;
  const bool dense = p.pse_kind == FA_PSE_DENSE;
  const float c_log2 = p.scale_log2;
  const float sl2 = alibi ? p.alibi_slopes[h] * kLog2e : 0.f;   // slope in log2 units
  const float sl2c = alibi ? sl2 / c_log2 : 0.f;                 // slope in raw-score units
  const bool f_pad = flags & FA_MASK_PADDING, f_mod = flags & FA_MASK_MODALITY;
  const bool f_exp = flags & FA_MASK_EXPLICIT;

  // ---- per key tile summaries (padding / modality), one wave-wide vote per
  // tile; modalities the rows of this wave (and of the workgroup) may attend
  const int n_kt_all = (p.Sk + BN - 1) / BN;
  const bool use_summary = (f_pad || f_mod) && n_kt_all <= kMaxTiles;
  uint32_t allow_any = 0, allow_all = 0xffu;
  if (tid == 0) { wg_any = 0u; wg_all = 0xffu; }
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
  }
  __syncthreads();
  if (l == 0 && use_summary && f_mod) {
    atomicOr(&wg_any, allow_any);
    atomicAnd(&wg_all, allow_all);
  }
  __syncthreads();

  // ---- tile lists.  Workgroup-level class of tile kt: 0 not visited,
  // 1 generic, 2 fast (no per-element work for any wave of the workgroup).
  auto wg_class = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * BN;
    bool fast = !dense && !f_exp && k0 + BN <= p.Sk;
    if (causal && k0 + BN - 1 > q0) fast = false;
    if (alibi && !(k0 + BN - 1 <= q0 || (!causal && k0 >= q0 + C::BM - 1))) fast = false;
    if (f_pad || f_mod) {
      if (!use_summary) return 1;
      const uint32_t ts = tsum[kt], kset = ts & 0xffu;
      const bool diag = f_mod && p.allow_diag && k0 < q0 + C::BM && k0 + BN > q0;
      if (f_mod ? ((kset & wg_any) == 0 && !diag) : kset == 0) return 0;
      if (ts & 0x100u) fast = false;
      if (f_mod && ((kset & ~wg_all) != 0 || diag)) fast = false;
    }
    return fast ? 2 : 1;
  };
  if (w == 0) {
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
  const int n_gen = __builtin_amdgcn_readfirstlane(n_list[0]);
  const int n_all = __builtin_amdgcn_readfirstlane(n_list[1]);
  auto tile_at = [&](int n) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane((int)tlist[n]);
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

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

  // S^T of one tile (two 32-key blocks), operand reads batched ahead of the MFMAs
  auto scores = [&](const uint16_t *ks, f32x16 (&s)[2]) __attribute__((always_inline)) {
    s[0] = s[1] = f32x16{};
#pragma unroll
    for (int t0 = 0; t0 < KS; t0 += 4) {
      u32x4 ka[4][2];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) ka[t][kb] = read_row_at<D>(ks, 32 * kb, ro[t0 + t]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = Mfma<T>::mac(ka[t][kb], qf[t0 + t], s[kb]);
    }
  };

  // O^T += V^T . P^T over the tile's four 16-key chunks
  auto pv = [&](const uint16_t *vs, const u32x4 (&pk)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < BN / 16; ++c) {
      u32x4 va[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) va[db] = read_tr_at<D>(vs, c, &to[2 * db]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = Mfma<T>::mac(va[db], pk[c], acc[db]);
    }
  };

  // lazy rescale: the reference max moves only when the row max mx (already
  // combined over the lane pair) grows by more than kTau; exp2(t - m_run)
  // then stays <= 2^kTau and O, l share the same reference.  Returns the
  // factor that rescales l.
  auto update_max = [&](float mx) __attribute__((always_inline)) {
    const bool grow = mx > m_run + kTau;
    float alpha = 1.f;
    if (grow) {
      alpha = exp2_fast(m_run - mx);
      m_run = mx;
    }
    if (__any(grow)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    return alpha;
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
    if (dense || f_exp || k0 + BN > p.Sk) cls = max(cls, (int)kGeneral);
    if (causal) {
      if (k0 > qw + 31) cls = kDead;
      else if (k0 + BN - 1 > qw) cls = max(cls, (int)kGeneral);
    }
    int adir = 0;   // ALiBi on a tile wholly below (+1) or above (-1) the diagonal
    if (alibi && cls != kDead) {
      if (k0 + BN - 1 <= qw) adir = 1;
      else if (k0 >= qw + 31) adir = -1;
      else cls = kGeneral;
    }
    if (use_summary && cls != kDead) {
      const uint32_t ts = __builtin_amdgcn_readfirstlane(tsum[kt]);
      const uint32_t kset = ts & 0xffu;
      if (f_mod) {
        const bool diag = p.allow_diag && k0 < qw + 32 && k0 + BN > qw;
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
      f32x16 s[2];
      scores(ks, s);
      // logit of element r of block kb:  t = cs * s + lane_off  (base-2 units)
      float cs = c_log2, lane_off = 0.f, mx = -INFINITY;
      if (cls == kFast) {
        if (adir != 0) {
          const float a = adir * sl2c;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              s[kb][r] = fmaf(a, (float)(32 * kb + 8 * (r >> 2) + (r & 3)), s[kb][r]);
          lane_off = adir * sl2 * (float)(k0 + 4 * g - my_i);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = fmaf(mx, cs, lane_off);
      } else {
        cs = 1.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = k0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
            float t = s[kb][r] * c_log2;
            bool ok = j < p.Sk && my_i < p.Sq;
            if (ok) ok = allowed_elem(p, b, h, my_i, j);
            if (ok) {
              if (alibi) t -= sl2 * fabsf((float)(my_i - j));
              else if (dense) t += dense_bias(p, b, h, my_i, j) * kLog2e;
            } else {
              t = -INFINITY;
            }
            s[kb][r] = t;
            mx = fmaxf(mx, t);
          }
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float alpha = update_max(mx);
      const float off = lane_off - (m_run == -INFINITY ? 0.f : m_run);
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = exp2_fast(fmaf(s[kb][r], cs, off));
          s[kb][r] = x;
          part[r & 3] += x;
        }
      l_run = l_run * alpha + ((part[0] + part[1]) + (part[2] + part[3]));
      u32x4 pk[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) pk[c] = pack8<T>(s[c >> 1], 8 * (c & 1));
      pv(vs, pk);
    }
    vm_wait_barrier();
  };

  if (n_gen > 0) {
    const int k0t = tile_at(0);
    load_tile(k0t, K0, Kr);
    load_tile(k0t, V0, Vr);
  }
  vm_wait_barrier();
  {
    int n = 0;
    for (; n + 1 < n_gen; n += 2) {
      generic_step(n, BufIdx<0>{});
      generic_step(n + 1, BufIdx<1>{});
    }
    if (n < n_gen) generic_step(n, BufIdx<0>{});
  }

  // ==== fast phase: software pipeline over list entries n_gen .. n_all-1
  const int n_fast = n_all - n_gen;
  auto ftile = [&](int n) __attribute__((always_inline)) { return tile_at(n_gen + n); };
  f32x16 sA[2], sB[2];
  if (n_fast > 0) {
    const int f0 = ftile(0);
    load_tile(f0, K0, Kr);
    load_tile(f0, V0, Vr);
    if (n_fast > 1) load_tile(ftile(1), K1, Kr);
  }
  vm_wait_barrier();
  if (n_fast > 0) scores(K0, sA);
  lds_barrier();   // every wave is done with K0 before the first step refills it

  // one step: softmax of tile n (scores in s), scores of tile n+1 (into sn),
  // O += P V of tile n.  Buffer parity B: K_{n+1} in K[1-B], V_n in V[B].
  auto fast_step = [&](int n, auto buf, f32x16 (&s)[2], f32x16 (&sn)[2])
                       __attribute__((always_inline)) {
    constexpr int B = decltype(buf)::value;
    const uint16_t *kn = B ? K0 : K1;   // K of tile n+1
    const uint16_t *vs = B ? V1 : V0;   // V of tile n
    opaque(ro);
    opaque(to);
    if (n + 2 < n_fast) load_tile(ftile(n + 2), B ? K1 : K0, Kr);
    if (n + 1 < n_fast) load_tile(ftile(n + 1), B ? V0 : V1, Vr);
    const int k0 = ftile(n) * BN;

    // ALiBi: the tile lies wholly below (+1) or above (-1) the diagonal for
    // every row of the workgroup; the per-register part of the term is folded
    // into s (coefficient 0 without ALiBi: no branch, the scores stay in place)
    const int adir = k0 + BN - 1 <= q0 ? 1 : -1;
    const float a = alibi ? adir * sl2c : 0.f;
    const float lane_off = alibi ? adir * sl2 * (float)(k0 + 4 * g - my_i) : 0.f;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kb][r] = fmaf(a, (float)(32 * kb + 8 * (r >> 2) + (r & 3)), s[kb][r]);
        mx = fmaxf(mx, s[kb][r]);
      }
    mx = fmaf(mx, c_log2, lane_off);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float alpha = update_max(mx);
    const float off = lane_off - (m_run == -INFINITY ? 0.f : m_run);

    // Scores of tile n+1 interleaved with the exponentials of tile n, in an
    // order fixed by scheduling fences (only scalar work may cross them): the
    // first half of the K operand reads up front and the rest one k-step
    // before they are needed,
    // then per k-step the two score products followed by a share of the
    // exponentials (which do not depend on them), so the matrix core and the
    // VALU work side by side.  The V^T reads of the first 16-key chunk go out
    // three quarters in, those of chunk c+1 ahead of the products of chunk c.
    // On the last step the scores come from a stale buffer and are unused.
    constexpr int NE = 32;               // score elements per lane
    constexpr int EPS = NE / KS;         // exponentials per k-step
    u32x4 ka[KS][2];
#pragma unroll
    for (int t = 0; t < KS / 2; ++t)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) ka[t][kb] = read_row_at<D>(kn, 32 * kb, ro[t]);
    __builtin_amdgcn_sched_barrier(0x0004);
    sn[0] = sn[1] = f32x16{};
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    u32x4 va[4][DB];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      if (t == KS / 2 - 1) {
#pragma unroll
        for (int u = KS / 2; u < KS; ++u)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) ka[u][kb] = read_row_at<D>(kn, 32 * kb, ro[u]);
      }
      if (t == 3 * KS / 4) {
#pragma unroll
        for (int db = 0; db < DB; ++db) va[0][db] = read_tr_at<D>(vs, 0, &to[2 * db]);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sn[kb] = Mfma<T>::mac(ka[t][kb], qf[t], sn[kb]);
#pragma unroll
      for (int e = t * EPS; e < (t + 1) * EPS; ++e) {
        const int kb = e / 16, r = e % 16;
        const float x = exp2_fast(fmaf(s[kb][r], c_log2, off));
        s[kb][r] = x;
        part[r & 3] += x;   // four short sum chains instead of one long one
      }
      __builtin_amdgcn_sched_barrier(0x0004);
    }
    l_run = l_run * alpha + ((part[0] + part[1]) + (part[2] + part[3]));
    u32x4 pk[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) pk[c] = pack8<T>(s[c >> 1], 8 * (c & 1));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c + 1 < 4) {
#pragma unroll
        for (int db = 0; db < DB; ++db) va[c + 1][db] = read_tr_at<D>(vs, c + 1, &to[2 * db]);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = Mfma<T>::mac(va[c][db], pk[c], acc[db]);
      __builtin_amdgcn_sched_barrier(0x0004);
    }
    vm_wait_barrier();
  };
  {
    int n = 0;
    for (; n + 1 < n_fast; n += 2) {
      fast_step(n, BufIdx<0>{}, sA, sB);
      fast_step(n + 1, BufIdx<1>{}, sB, sA);
    }
    if (n < n_fast) fast_step(n, BufIdx<0>{}, sA, sB);
  }

  // ---- epilogue: O = acc / l, LSE
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (my_i < p.Sq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T *Og = (T *)p.o + b * p.q_sb + h * p.q_sh + (int64_t)my_i * p.q_ss;
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
