// fp64 reference of the fused attention operator, in plain C++ (test
// infrastructure: only the tests, the smoke check and the benchmark's CPU
// baseline load it; the HIP library never does, and the two share no code).
//
// What it computes is the definition, term by term, one (batch, head) at a
// time with the whole S_q x S_k probability matrix held in memory:
//
//   * scores s_ij = scale * q_i . k_j + bias_ij, where the bias is added after
//     scaling and is not scaled itself (FlashAttentionScore replacement guide,
//     section 4 step 1: scale, then add the mask, then softmax, then times V;
//     section 3.2: pse may be ALiBi, materialised here as -slope_h |i - j|);
//   * a pair the masks hide gets s_ij = -inf: causal keeps j <= i (the CogVLM
//     guide's tril mask), the explicit mask keeps nonzero entries, the
//     modality rule keeps allow[m_q(i)][m_k(j)] (or i == j when the diagonal
//     flag is set: the multimodal page's default keeps it), the padding rule
//     keeps valid keys (the retrieval page's document mask);
//   * P = row softmax (guide section 2); a row with no visible key gives O = 0,
//     LSE = -inf and no gradient;
//   * O_i = sum_j P_ij Z_ij v_j, LSE_i = m_i + ln sum_j exp(s_ij - m_i), with Z
//     the dropout factors: 1/keep_prob where the keep mask holds, 0 elsewhere
//     (keep_prob < 1; guide section 3.2 names only the keep ratio);
//   * the backward is the exact gradient of L = sum(O * dO):
//     dV_j = sum_i P_ij Z_ij dO_i, dP_ij = Z_ij dO_i . v_j,
//     D_i = sum_j P_ij dP_ij, dS_ij = P_ij (dP_ij - D_i),
//     dQ_i = scale sum_j dS_ij k_j, dK_j = scale sum_i dS_ij q_i.
//
// The keep mask is Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011), written here from
// the paper: counter (j div 4, i, h, b), key = the 64-bit seed (low word
// first); key j takes output word j mod 4 and is kept iff that word is below
// floor(keep_prob * 2^32).
//
// Arrays are BNSD (q [B][H][S_q][D], k and v [B][H][S_k][D]); the Python side
// converts other layouts and upcasts the inputs exactly.  OpenMP runs one
// (batch, head) per thread.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include <omp.h>

extern "C" {

typedef struct fa_ref_problem {
  int32_t B, H, Sq, Sk, D;
  double scale;
  int32_t causal;
  // explicit mask, nonzero = may attend; element b*em_sb + h*em_sh + i*em_sq + j
  const uint8_t *em;
  int64_t em_sb, em_sh, em_sq;
  // modality: ids [B][S_q], [B][S_k]; allow[mq * M + mk]
  const int8_t *qmod, *kmod;
  int32_t M;
  const uint8_t *allow;
  int32_t allow_diag;
  // padding: key_valid [B][S_k]
  const uint8_t *key_valid;
  // bias: alibi slopes [H] or a dense bias element b*pse_sb + h*pse_sh + i*pse_sq + j
  const double *alibi;
  const double *pse;
  int64_t pse_sb, pse_sh, pse_sq;
  // dropout
  double keep_prob;
  uint64_t seed;
} fa_ref_problem;

}  // extern "C"

namespace {

const double kNegInf = -std::numeric_limits<double>::infinity();

// One Philox4x32-10 block: ctr (4 words) under key (2 words).
void philox(uint32_t ctr[4], uint32_t k0, uint32_t k1) {
  const uint64_t M0 = 0xD2511F53ull, M1 = 0xCD9E8D57ull;
  for (int round = 0; round < 10; ++round) {
    const uint64_t a = M0 * ctr[0], c = M1 * ctr[2];
    const uint32_t n0 = (uint32_t)(c >> 32) ^ ctr[1] ^ k0;
    const uint32_t n1 = (uint32_t)c;
    const uint32_t n2 = (uint32_t)(a >> 32) ^ ctr[3] ^ k1;
    const uint32_t n3 = (uint32_t)a;
    ctr[0] = n0; ctr[1] = n1; ctr[2] = n2; ctr[3] = n3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

bool allowed(const fa_ref_problem &p, int b, int h, int i, int j) {
  if (p.causal && j > i) return false;
  if (p.em && !p.em[b * p.em_sb + h * p.em_sh + (int64_t)i * p.em_sq + j]) return false;
  if (p.qmod) {
    const int mq = p.qmod[(int64_t)b * p.Sq + i], mk = p.kmod[(int64_t)b * p.Sk + j];
    if (!p.allow[mq * p.M + mk] && !(p.allow_diag && i == j)) return false;
  }
  if (p.key_valid && !p.key_valid[(int64_t)b * p.Sk + j]) return false;
  return true;
}

double bias(const fa_ref_problem &p, int b, int h, int i, int j) {
  double x = 0.0;
  if (p.pse) x += p.pse[b * p.pse_sb + h * p.pse_sh + (int64_t)i * p.pse_sq + j];
  if (p.alibi) x -= p.alibi[h] * std::fabs((double)i - (double)j);
  return x;
}

// Dropout factor matrix of head (b, h): Z[i][j] = 1/keep_prob (kept) or 0.
void dropout_factors(const fa_ref_problem &p, int b, int h, std::vector<double> &Z) {
  const float kpf = (float)p.keep_prob;
  const uint32_t thr = (uint32_t)std::floor((double)kpf * 4294967296.0);
  const double inv = 1.0 / (double)kpf;
  for (int i = 0; i < p.Sq; ++i)
    for (int j4 = 0; j4 < p.Sk; j4 += 4) {
      uint32_t w[4] = {(uint32_t)(j4 / 4), (uint32_t)i, (uint32_t)h, (uint32_t)b};
      philox(w, (uint32_t)(p.seed & 0xffffffffu), (uint32_t)(p.seed >> 32));
      for (int t = 0; t < 4 && j4 + t < p.Sk; ++t)
        Z[(size_t)i * p.Sk + j4 + t] = w[t] < thr ? inv : 0.0;
    }
}

bool has_dropout(const fa_ref_problem &p) { return (float)p.keep_prob < 1.0f; }

// P (the undropped probabilities) of head (b, h), [S_q][S_k], and the row LSE.
void probabilities(const fa_ref_problem &p, int b, int h, const double *q, const double *k,
                   std::vector<double> &P, double *lse) {
  const int Sq = p.Sq, Sk = p.Sk, D = p.D;
  for (int i = 0; i < Sq; ++i) {
    const double *qi = q + (size_t)i * D;
    double *row = &P[(size_t)i * Sk];
    double m = kNegInf;
    for (int j = 0; j < Sk; ++j) {
      if (!allowed(p, b, h, i, j)) {
        row[j] = kNegInf;
        continue;
      }
      const double *kj = k + (size_t)j * D;
      double dot = 0.0;
      for (int d = 0; d < D; ++d) dot += qi[d] * kj[d];
      row[j] = p.scale * dot + bias(p, b, h, i, j);
      if (row[j] > m) m = row[j];
    }
    if (m == kNegInf) {   // no visible key
      for (int j = 0; j < Sk; ++j) row[j] = 0.0;
      lse[i] = kNegInf;
      continue;
    }
    double l = 0.0;
    for (int j = 0; j < Sk; ++j) {
      row[j] = row[j] == kNegInf ? 0.0 : std::exp(row[j] - m);
      l += row[j];
    }
    for (int j = 0; j < Sk; ++j) row[j] /= l;
    lse[i] = m + std::log(l);
  }
}

}  // namespace

extern "C" {

int fa_ref_abi_version(void) { return 1; }

// Threads of the (batch, head) loops (OpenMP); returns the previous count.
int fa_ref_set_threads(int n) {
  const int old = omp_get_max_threads();
  if (n > 0) omp_set_num_threads(n);
  return old;
}

// Forward: o [B][H][S_q][D], lse [B][H][S_q].  Returns 0, or -1 on bad sizes.
int fa_ref_fwd(const fa_ref_problem *pp, const double *q, const double *k, const double *v,
               double *o, double *lse) {
  if (!pp || pp->B < 0 || pp->H < 0 || pp->Sq < 0 || pp->Sk < 0 || pp->D <= 0) return -1;
  const fa_ref_problem p = *pp;
  const int BH = p.B * p.H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < BH; ++bh) {
    const int b = bh / p.H, h = bh % p.H;
    const size_t qo = (size_t)bh * p.Sq * p.D, ko = (size_t)bh * p.Sk * p.D;
    std::vector<double> P((size_t)p.Sq * p.Sk), Z;
    probabilities(p, b, h, q + qo, k + ko, P, lse + (size_t)bh * p.Sq);
    if (has_dropout(p)) {
      Z.assign((size_t)p.Sq * p.Sk, 0.0);
      dropout_factors(p, b, h, Z);
    }
    for (int i = 0; i < p.Sq; ++i) {
      double *oi = o + qo + (size_t)i * p.D;
      for (int d = 0; d < p.D; ++d) oi[d] = 0.0;
      for (int j = 0; j < p.Sk; ++j) {
        double w = P[(size_t)i * p.Sk + j];
        if (w == 0.0) continue;
        if (!Z.empty()) w *= Z[(size_t)i * p.Sk + j];
        const double *vj = v + ko + (size_t)j * p.D;
        for (int d = 0; d < p.D; ++d) oi[d] += w * vj[d];
      }
    }
  }
  return 0;
}

// Backward: dq [B][H][S_q][D], dk and dv [B][H][S_k][D]; optional ds
// [B][H][S_q][S_k] (the gradient of the softmax's input, which is also the
// gradient of an additive bias element), may be null.
int fa_ref_bwd(const fa_ref_problem *pp, const double *q, const double *k, const double *v,
               const double *dout, double *dq, double *dk, double *dv, double *ds) {
  if (!pp || pp->B < 0 || pp->H < 0 || pp->Sq < 0 || pp->Sk < 0 || pp->D <= 0) return -1;
  const fa_ref_problem p = *pp;
  const int BH = p.B * p.H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < BH; ++bh) {
    const int b = bh / p.H, h = bh % p.H;
    const int Sq = p.Sq, Sk = p.Sk, D = p.D;
    const size_t qo = (size_t)bh * Sq * D, ko = (size_t)bh * Sk * D;
    std::vector<double> P((size_t)Sq * Sk), Z, lse(Sq), dS((size_t)Sq * Sk);
    probabilities(p, b, h, q + qo, k + ko, P, lse.data());
    if (has_dropout(p)) {
      Z.assign((size_t)Sq * Sk, 0.0);
      dropout_factors(p, b, h, Z);
    }
    for (size_t x = 0; x < (size_t)Sk * D; ++x) dk[ko + x] = dv[ko + x] = 0.0;
    for (int i = 0; i < Sq; ++i) {
      const double *doi = dout + qo + (size_t)i * D;
      double Di = 0.0;
      for (int j = 0; j < Sk; ++j) {
        const double Pij = P[(size_t)i * Sk + j];
        double dPij = 0.0;
        if (Pij != 0.0) {
          const double *vj = v + ko + (size_t)j * D;
          for (int d = 0; d < D; ++d) dPij += doi[d] * vj[d];
          if (!Z.empty()) dPij *= Z[(size_t)i * Sk + j];
        }
        dS[(size_t)i * Sk + j] = dPij;   // dP for now
        Di += Pij * dPij;
      }
      double *dqi = dq + qo + (size_t)i * D;
      for (int d = 0; d < D; ++d) dqi[d] = 0.0;
      const double *qi = q + qo + (size_t)i * D;
      for (int j = 0; j < Sk; ++j) {
        const double Pij = P[(size_t)i * Sk + j];
        const double dSij = Pij * (dS[(size_t)i * Sk + j] - Di);
        dS[(size_t)i * Sk + j] = dSij;
        if (Pij == 0.0) continue;
        const double pz = Z.empty() ? Pij : Pij * Z[(size_t)i * Sk + j];
        const double *kj = k + ko + (size_t)j * D;
        double *dkj = dk + ko + (size_t)j * D, *dvj = dv + ko + (size_t)j * D;
        for (int d = 0; d < D; ++d) {
          dqi[d] += p.scale * dSij * kj[d];
          dkj[d] += p.scale * dSij * qi[d];
          dvj[d] += pz * doi[d];
        }
      }
    }
    if (ds) std::memcpy(ds + (size_t)bh * Sq * Sk, dS.data(), sizeof(double) * (size_t)Sq * Sk);
  }
  return 0;
}

// Philox4x32-10 on one counter (for known-answer checks): out = block(ctr, key).
void fa_ref_philox(const uint32_t ctr[4], uint32_t k0, uint32_t k1, uint32_t out[4]) {
  uint32_t w[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  philox(w, k0, k1);
  for (int t = 0; t < 4; ++t) out[t] = w[t];
}

}  // extern "C"
