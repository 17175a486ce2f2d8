"""fp64 CPU oracle for the fused attention operator (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library
and its Python binding) never calls it and shares no code with it.

What it computes is the plain definition, written out with numpy float64,
one (batch, head) at a time, materialising the whole S_q x S_k score matrix:

* attention: Softmax(Q K^T * scale) V (FlashAttentionScore replacement
  guide, section 2 "operator math"), with the unfused order of operations
  of section 4 step 1: scores are scaled first, then the additive mask is
  added, then softmax, then the product with V;
* the additive position bias ``pse`` (section 3.2 parameter table) is added
  after scaling and is not scaled itself; ALiBi is materialised as
  ``-slope_h * |i - j|``;
* boolean masks use True = may attend (ops-transformer multimodal
  FlashAttention page, "Layer 2: cross-modal attention", mask docstring;
  CogVLM guide, "attention mask": ones then ``tril_``; retrieval page,
  "Layer 2: semantic modelling": invalid document tokens become -inf).
  Masked scores are exactly -inf;
* the per-row log-sum-exp is the natural log and includes scale and bias;
* a row with no allowed key returns O = 0, LSE = -inf and contributes
  nothing to any gradient (the pages leave this open: the multimodal page's
  blockwise code would produce NaN there);
* the backward is the exact gradient of O with respect to Q, K, V given
  dO (the guide's section 2 says the fused operator returns gradients
  without storing the N x N matrix; here that matrix is simply stored,
  since this is the definition, not the method);
* dropout (``keep_prob`` < 1, section 3.2 parameter table, "retention
  proportion", default 1.0 = none): the probabilities that multiply V are
  P_ij * M_ij / keep_prob with M a 0/1 keep mask; the LSE is that of the
  undropped softmax.  The pages name no generator, so the mask is drawn
  from Philox4x32-10 (Salmon et al., "Parallel random numbers: as easy as
  1, 2, 3", SC 2011), written here from that paper's definition: word
  j mod 4 of the output for counter (j div 4, i, h, b) under the 64-bit
  seed as key; kept iff that word < floor(keep_prob * 2^32) with keep_prob
  the float32 value.  The gradient is that of the same function with M
  fixed.

The MaxSim late-interaction score (retrieval page, "Layer 2: semantic
modelling") is :func:`maxsim`: plain dot products of query and document
token embeddings, invalid document tokens excluded, the best match of each
query token, summed over the query tokens and divided by L_q.  The page's
code sets a whole invalid query row to -inf and then sums every row, which
makes the score -inf as soon as one query token is padding; here that row's
max is reported as -inf but left out of the sum (the divisor stays L_q, as
printed).

Every function is pinned: the core by ``tests/test_oracle_pins.py`` (brute
force, closed forms, invariants, finite differences, a library attention
routine on sliced problems; the row-restricted :func:`attention_rows`, which
full-size GPU checks use on sampled rows, against the brute force and torch
autograd), the problem wrappers ``problem_masks``,
``problem_fwd`` and ``problem_bwd`` by ``tests/test_oracle_problem_pins.py``
(BSH against BNSD, each mask and bias field changing exactly the rows it
should, the dropout fields reaching the core, the bias gradient against
central differences).  Nothing here is "parity unpinned".  The plain C++
fp64 oracle in ``oracle/fa_ref.cpp`` (``oracle.cpp``) computes the same
definition independently and is pinned by ``tests/test_oracle_cpp.py``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bsh_to_bnsd", "bnsd_to_bsh", "allowed", "bias", "head_scores",
    "softmax_rows", "attention_fwd", "attention_bwd", "probabilities",
    "problem_masks", "problem_fwd", "problem_bwd", "philox4x32_10", "dropout_mask", "maxsim",
    "e4m3_decode",
]


def bsh_to_bnsd(x: np.ndarray, heads: int) -> np.ndarray:
    """[B, S, H*D] -> [B, H, S, D]: the head split ``view(B,N,H,D).transpose(1,2)``
    of the multimodal page's cross-modal attention module."""
    B, S, HD = x.shape
    return np.ascontiguousarray(x.reshape(B, S, heads, HD // heads).transpose(0, 2, 1, 3))


def bnsd_to_bsh(x: np.ndarray) -> np.ndarray:
    """[B, H, S, D] -> [B, S, H*D], the inverse of :func:`bsh_to_bnsd`."""
    B, H, S, D = x.shape
    return np.ascontiguousarray(x.transpose(0, 2, 1, 3).reshape(B, S, H * D))


def allowed(b, h, Sq, Sk, *, causal=False, explicit_mask=None, q_modality=None,
            k_modality=None, modality_allow=None, modality_allow_diag=False,
            key_valid=None, rows=None) -> np.ndarray:
    """Boolean [Sq, Sk]: may query i of head (b, h) attend to key j.  With
    ``rows`` (query indices) only those rows are formed, [len(rows), Sk].

    The mask kinds combine by AND:
    * causal: the lower triangle ``tril`` including the diagonal, j <= i
      (CogVLM guide, attention mask);
    * explicit: a user bool mask, True = may attend, broadcast over B and H
      (multimodal page, cross-modal mask [B,N,N] expanded to [B,H,N,N]);
    * modality: allowed iff allow[m_q(i)][m_k(j)], optionally OR'ed with
      i == j (the multimodal page's default rule keeps the diagonal);
    * padding: key j of sample b is a real token (retrieval page doc_mask).
    """
    r = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(Sk)
    ok = np.ones((len(r), Sk), dtype=bool)
    if causal:
        ok &= j[None, :] <= r[:, None]    # tril, the diagonal included
    if explicit_mask is not None:
        em = np.asarray(explicit_mask, dtype=bool)
        if em.ndim == 2:                  # [Sq, Sk]
            em = em[None, None]
        elif em.ndim == 3:                # [B, Sq, Sk], shared by every head
            em = em[:, None]
        ok &= em[b if em.shape[0] > 1 else 0, h if em.shape[1] > 1 else 0][r]
    if q_modality is not None:
        allow = np.asarray(modality_allow, dtype=bool)
        qm = np.asarray(q_modality)[b].astype(np.int64)[r]
        km = np.asarray(k_modality)[b].astype(np.int64)
        m = allow[qm[:, None], km[None, :]]
        if modality_allow_diag:
            m = m | (j[None, :] == r[:, None])
        ok &= m
    if key_valid is not None:
        ok &= np.asarray(key_valid, dtype=bool)[b][None, :]
    return ok


def bias(b, h, Sq, Sk, *, pse=None, alibi_slopes=None, rows=None) -> np.ndarray | None:
    """float64 [Sq, Sk] additive bias for head (b, h), or None (with ``rows``,
    only those query rows).

    ``pse`` is a dense tensor broadcastable to [B, H, Sq, Sk]; ALiBi uses
    -slope_h * |i - j| with the caller's slope values (upcast exactly)."""
    r = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = None
    if pse is not None:
        p = np.asarray(pse, dtype=np.float64)
        p = p[b if p.shape[0] > 1 else 0, h if p.shape[1] > 1 else 0]
        out = np.broadcast_to(p, (Sq, Sk))[r].astype(np.float64)
    if alibi_slopes is not None:
        slope = float(np.asarray(alibi_slopes, dtype=np.float64)[h])
        i = r.astype(np.float64)[:, None]
        j = np.arange(Sk, dtype=np.float64)[None, :]
        a = -slope * np.abs(i - j)
        out = a if out is None else out + a
    return out


def head_scores(q, k, scale, b, h, masks: dict, rows=None) -> np.ndarray:
    """Scaled scores plus bias for head (b, h), with disallowed entries set to
    exactly -inf.  ``q`` [B,H,Sq,D] and ``k`` [B,H,Sk,D] are float64.  With
    ``rows`` (query indices) only those rows of the score matrix."""
    Sq, Sk = q.shape[2], k.shape[2]
    qr = q[b, h] if rows is None else q[b, h][np.asarray(rows, dtype=np.int64)]
    s = scale * (qr @ k[b, h].T)
    bb = bias(b, h, Sq, Sk, pse=masks.get("pse"), alibi_slopes=masks.get("alibi_slopes"),
              rows=rows)
    if bb is not None:
        s = s + bb
    ok = allowed(b, h, Sq, Sk, rows=rows,
                 **{key: masks[key] for key in _MASK_KEYS if key in masks})
    return np.where(ok, s, -np.inf)


_MASK_KEYS = ("causal", "explicit_mask", "q_modality", "k_modality", "modality_allow",
              "modality_allow_diag", "key_valid")


def softmax_rows(s: np.ndarray):
    """Row softmax of a score matrix that may hold -inf.

    Returns (P, lse): P[i, j] = exp(s_ij - m_i) / sum_j exp(s_ij - m_i) with
    m_i the row max, and lse_i = m_i + ln(sum_j exp(s_ij - m_i)).  A row whose
    scores are all -inf gets P = 0 and lse = -inf."""
    m = s.max(axis=1)
    dead = ~np.isfinite(m)
    m_safe = np.where(dead, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    e[dead] = 0.0
    l = e.sum(axis=1)
    l_safe = np.where(dead, 1.0, l)
    P = e / l_safe[:, None]
    lse = np.where(dead, -np.inf, m_safe + np.log(l_safe))
    return P, lse


_U32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds (Salmon et al., SC 2011, section 5.2).

    Counter words ``c0..c3`` are integer arrays (broadcast together), the
    key is two 32-bit integers.  One round: the products M0*c0 and M1*c2
    are split into high and low halves; the new counter is
    (hi(M1*c2) ^ c1 ^ key0, lo(M1*c2), hi(M0*c0) ^ c3 ^ key1, lo(M0*c0)).
    Between rounds the key is advanced by the Weyl constants (the golden
    ratio and sqrt(3) - 1, scaled to 32 bits).  Returns four uint64 arrays
    holding 32-bit words."""
    M0, M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
    W0, W1 = 0x9E3779B9, 0xBB67AE85
    x = [np.asarray(c, dtype=np.uint64) & _U32 for c in (c0, c1, c2, c3)]
    x = list(np.broadcast_arrays(*x))
    key0, key1 = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    for _ in range(10):
        p0 = M0 * x[0]            # < 2^64: both factors are below 2^32
        p1 = M1 * x[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _U32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _U32
        x = [hi1 ^ x[1] ^ np.uint64(key0), lo1, hi0 ^ x[3] ^ np.uint64(key1), lo0]
        key0 = (key0 + W0) & 0xFFFFFFFF
        key1 = (key1 + W1) & 0xFFFFFFFF
    return x


def dropout_mask(b, h, Sq, Sk, keep_prob, seed) -> np.ndarray:
    """Boolean [Sq, Sk] keep mask of head (b, h); all True when keep_prob >= 1."""
    kp = float(np.float32(keep_prob))
    if kp >= 1.0:
        return np.ones((Sq, Sk), dtype=bool)
    thr = np.uint64(int(np.floor(kp * 4294967296.0)))
    i = np.arange(Sq, dtype=np.uint64)[:, None]
    j4 = np.arange((Sk + 3) // 4, dtype=np.uint64)[None, :]
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    w = philox4x32_10(j4, i, np.uint64(h), np.uint64(b), seed & 0xFFFFFFFF, seed >> 32)
    words = np.stack(w, axis=-1).reshape(Sq, -1)[:, :Sk]      # key j -> word j % 4
    return words < thr


def _as_f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):          # a torch tensor: exact upcast
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _as_np(x):
    if x is None or isinstance(x, (bool, int, float)):
        return x
    if hasattr(x, "detach"):
        return x.detach().cpu().numpy()
    return np.asarray(x)


def _masks(kw) -> dict:
    out = {}
    for key, val in kw.items():
        if val is None:
            continue
        if key in ("pse", "alibi_slopes"):
            out[key] = _as_f64(val)
        else:
            out[key] = _as_np(val)
    return out


def probabilities(q, k, scale, b=0, h=0, **masks) -> np.ndarray:
    """P for head (b, h): the softmax of the masked, biased, scaled scores."""
    q, k = _as_f64(q), _as_f64(k)
    P, _ = softmax_rows(head_scores(q, k, scale, b, h, _masks(masks)))
    return P


def _drop_scale(b, h, Sq, Sk, keep_prob, seed):
    """The dropout factor matrix M / keep_prob (float64), or None without dropout."""
    if float(np.float32(keep_prob)) >= 1.0:
        return None
    return dropout_mask(b, h, Sq, Sk, keep_prob, seed) / float(np.float32(keep_prob))


def attention_fwd(q, k, v, scale, keep_prob=1.0, dropout_seed=0, **masks):
    """O [B,H,Sq,D] and LSE [B,H,Sq], float64, for BNSD inputs.

    O_i = sum_j P_ij Z_ij v_j with P the row softmax of
    scale * q_i . k_j + bias_ij over the allowed keys and Z the dropout
    factors (1 without dropout)."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    mk = _masks(masks)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    O = np.zeros((B, H, Sq, v.shape[3]), dtype=np.float64)
    LSE = np.empty((B, H, Sq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            P, lse = softmax_rows(head_scores(q, k, scale, b, h, mk))
            Z = _drop_scale(b, h, Sq, Sk, keep_prob, dropout_seed)
            O[b, h] = (P if Z is None else P * Z) @ v[b, h]
            LSE[b, h] = lse
    return O, LSE


def attention_bwd(q, k, v, do, scale, keep_prob=1.0, dropout_seed=0, return_dbias=False,
                  **masks):
    """dQ, dK, dV (float64, BNSD) of L = sum(O * dO).

    With P the forward probabilities and Z the dropout factors (1 without
    dropout): dV_j = sum_i P_ij Z_ij dO_i;  dP_ij = Z_ij dO_i . v_j;
    D_i = sum_j P_ij dP_ij;  dS_ij = P_ij (dP_ij - D_i);
    dQ_i = scale sum_j dS_ij k_j;  dK_j = scale sum_i dS_ij q_i.
    dS is the gradient of L with respect to the softmax's input, hence also
    with respect to an additive bias element; ``return_dbias`` appends it as
    a fourth result, float64 [B, H, Sq, Sk] (one slice per (b, h), before
    any reduction over a broadcast bias)."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    mk = _masks(masks)
    B, H, Sq = q.shape[:3]
    Sk = k.shape[2]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dbias = np.zeros((B, H, Sq, Sk)) if return_dbias else None
    for b in range(B):
        for h in range(H):
            P, _ = softmax_rows(head_scores(q, k, scale, b, h, mk))
            Z = _drop_scale(b, h, Sq, Sk, keep_prob, dropout_seed)
            dv[b, h] = (P if Z is None else P * Z).T @ do[b, h]
            dP = do[b, h] @ v[b, h].T
            if Z is not None:
                dP = dP * Z
            Dl = (P * dP).sum(axis=1)
            dS = P * (dP - Dl[:, None])
            dq[b, h] = scale * (dS @ k[b, h])
            dk[b, h] = scale * (dS.T @ q[b, h])
            if dbias is not None:
                dbias[b, h] = dS
    return (dq, dk, dv) if dbias is None else (dq, dk, dv, dbias)


def attention_rows(q, k, v, do, scale, rows, b=0, h=0, **masks):
    """O, LSE and dQ of the query rows ``rows`` of head (b, h) only (float64,
    [len(rows), D], [len(rows)], [len(rows), D]), BNSD inputs, no dropout.

    Each of these is a function of its own row of scores: P_i is the softmax
    of row i, O_i = sum_j P_ij v_j, dP_ij = dO_i . v_j, D_i = sum_j P_ij dP_ij,
    dQ_i = scale sum_j P_ij (dP_ij - D_i) k_j -- the same quantities as
    :func:`attention_fwd` and :func:`attention_bwd` form for every row, here
    for a few rows of a problem too large to form whole."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    P, lse = softmax_rows(head_scores(q, k, scale, b, h, _masks(masks), rows=rows))
    r = np.asarray(rows, dtype=np.int64)
    O = P @ v[b, h]
    dP = do[b, h][r] @ v[b, h].T
    Dl = (P * dP).sum(axis=1)
    dQ = scale * ((P * (dP - Dl[:, None])) @ k[b, h])
    return O, lse, dQ


def problem_masks(p) -> dict:
    """The mask/bias keyword arguments of a problem description (an object
    with the attributes of ``tiled_attention_03_amd.inputs.Problem``)."""
    return dict(causal=p.causal, explicit_mask=p.explicit_mask, q_modality=p.q_modality,
                k_modality=p.k_modality, modality_allow=p.modality_allow,
                modality_allow_diag=p.modality_allow_diag, key_valid=p.key_valid,
                pse=p.pse, alibi_slopes=p.alibi_slopes)


def _bnsd(x, p):
    x = _as_f64(x)
    return bsh_to_bnsd(x, p.heads) if p.layout == "BSH" else x


def _problem_drop(p) -> dict:
    return dict(keep_prob=getattr(p, "keep_prob", 1.0), dropout_seed=getattr(p, "dropout_seed", 0))


def problem_fwd(p):
    """(O, LSE) for a problem, O in the problem's own layout (float64)."""
    O, LSE = attention_fwd(_bnsd(p.q, p), _bnsd(p.k, p), _bnsd(p.v, p), p.scale,
                           **_problem_drop(p), **problem_masks(p))
    return (bnsd_to_bsh(O) if p.layout == "BSH" else O), LSE


def problem_bwd(p, return_dbias=False):
    """(dQ, dK, dV) for a problem with upstream gradient ``p.do``, each in the
    problem's own layout (float64); with ``return_dbias`` also dS [B,H,Sq,Sk]."""
    g = attention_bwd(_bnsd(p.q, p), _bnsd(p.k, p), _bnsd(p.v, p), _bnsd(p.do, p), p.scale,
                      return_dbias=return_dbias, **_problem_drop(p), **problem_masks(p))
    out = tuple(bnsd_to_bsh(x) if p.layout == "BSH" else x for x in g[:3])
    return out + (g[3],) if return_dbias else out


def maxsim(q, d, q_valid=None, d_valid=None):
    """MaxSim of each sample: (rowmax [B, L_q], score [B]), float64.

    q [B, L_q, D] and d [B, L_d, D]; q_valid [B, L_q] and d_valid [B, L_d]
    are booleans (None = all valid).  sim_ij = q_i . d_j; invalid documents
    are -inf; rowmax_i = max_j sim_ij, -inf for an invalid query token or
    when no document token is valid; score = (sum of rowmax over valid
    query tokens) / L_q, and 0 when there is no valid query token."""
    q, d = _as_f64(q), _as_f64(d)
    B, Lq = q.shape[:2]
    Ld = d.shape[1]
    qv = np.ones((B, Lq), dtype=bool) if q_valid is None else np.asarray(_as_np(q_valid), dtype=bool)
    dv = np.ones((B, Ld), dtype=bool) if d_valid is None else np.asarray(_as_np(d_valid), dtype=bool)
    rowmax = np.full((B, Lq), -np.inf)
    score = np.zeros(B)
    for b in range(B):
        sim = q[b] @ d[b].T                                  # [L_q, L_d]
        sim = np.where(dv[b][None, :], sim, -np.inf)
        rm = sim.max(axis=1) if Ld > 0 else np.full(Lq, -np.inf)
        rm = np.where(qv[b], rm, -np.inf)
        rowmax[b] = rm
        if Lq > 0:
            score[b] = rm[qv[b]].sum() / Lq
    return rowmax, score


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of OCP FP8 E4M3 bytes (the "fn" variant): bit 7 sign,
    bits 6..3 exponent with bias 7, bits 2..0 mantissa; exponent 0 is
    subnormal (m / 8 * 2^-6); 0x7f and 0xff are NaN; there are no infinities,
    so exponent 15 with mantissa < 7 is a normal number (up to 448)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = sign * val
    return np.where((c & 0x7F) == 0x7F, np.nan, val)
