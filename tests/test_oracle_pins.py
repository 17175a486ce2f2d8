"""Pins for the fp64 oracle: it is checked against things other than itself.

* brute force in pure Python (its own mask rules, math.exp, math.fsum) on
  sequences of at most 8 tokens, for every mask kind and bias;
* closed forms: Q = 0 gives the mean of the allowed V rows and
  LSE = ln(#allowed); one allowed key returns that key's V row; ALiBi with
  causal and Q = 0 is a geometric series; S_k = 1 gives O = V and zero
  dQ/dK;
* invariants: rows of P sum to 1, a per-row constant shifts only LSE,
  permuting keys (with the mask columns) leaves O unchanged, causal equals
  the explicit lower-triangular mask, and the backward's sums vanish;
* a library routine: torch's scaled_dot_product_attention in float64 on the
  CPU (forward, and autograd for the backward) with an additive mask the test
  builds itself, and on sliced sub-problems for the modality and padding
  masks;
* central finite differences of L = sum(O * dO) for the backward;
* the pages' own mask examples (tests/golden), and a hand-derived worked
  example.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------
# an independent brute-force attention in pure Python

def naive_attention(q, k, v, scale, rule, bias_fn=None):
    """q [Sq][D], k/v [Sk][D] as nested lists; rule(i, j) -> bool; returns
    (O rows, LSE list) computed term by term."""
    Sq, Sk, Dv = len(q), len(k), len(v[0])
    O, L = [], []
    for i in range(Sq):
        s = []
        for j in range(Sk):
            if not rule(i, j):
                s.append(-math.inf)
                continue
            dot = math.fsum(q[i][d] * k[j][d] for d in range(len(q[i])))
            val = dot * scale
            if bias_fn is not None:
                val += bias_fn(i, j)
            s.append(val)
        finite = [x for x in s if x != -math.inf]
        if not finite:
            O.append([0.0] * Dv)
            L.append(-math.inf)
            continue
        m = max(finite)
        w = [math.exp(x - m) if x != -math.inf else 0.0 for x in s]
        tot = math.fsum(w)
        O.append([math.fsum(w[j] * v[j][d] for j in range(Sk)) / tot for d in range(Dv)])
        L.append(m + math.log(tot))
    return O, L


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def mask_cases():
    """(name, masks-for-oracle, rule(b,h,i,j), bias(b,h,i,j)) over B=2, H=2, Sq=7, Sk=8."""
    B, H, Sq, Sk = 2, 2, 7, 8
    rng = np.random.default_rng(7)
    em = rng.random((B, 1, Sq, Sk)) < 0.6
    qm = rng.integers(0, 3, (B, Sq))
    km = rng.integers(0, 3, (B, Sk))
    allow = np.array([[1, 1, 0], [0, 1, 1], [1, 0, 1]], dtype=bool)
    kv = rng.random((B, Sk)) < 0.7
    slopes = np.array([0.5, 0.125])
    pse = rng.standard_normal((1, H, Sq, Sk))
    cases = [
        ("none", {}, lambda b, h, i, j: True, None),
        ("causal", {"causal": True}, lambda b, h, i, j: j <= i, None),
        ("explicit", {"explicit_mask": em}, lambda b, h, i, j: bool(em[b, 0, i, j]), None),
        ("modality", {"q_modality": qm, "k_modality": km, "modality_allow": allow},
         lambda b, h, i, j: bool(allow[qm[b, i], km[b, j]]), None),
        ("modality_diag", {"q_modality": qm, "k_modality": km, "modality_allow": allow,
                           "modality_allow_diag": True},
         lambda b, h, i, j: bool(allow[qm[b, i], km[b, j]]) or i == j, None),
        ("padding", {"key_valid": kv}, lambda b, h, i, j: bool(kv[b, j]), None),
        ("alibi", {"alibi_slopes": slopes}, lambda b, h, i, j: True,
         lambda b, h, i, j: -slopes[h] * abs(i - j)),
        ("dense_pse_causal_padding", {"pse": pse, "causal": True, "key_valid": kv},
         lambda b, h, i, j: j <= i and bool(kv[b, j]), lambda b, h, i, j: pse[0, h, i, j]),
        ("everything", {"causal": True, "explicit_mask": em, "q_modality": qm, "k_modality": km,
                        "modality_allow": allow, "key_valid": kv, "alibi_slopes": slopes},
         lambda b, h, i, j: j <= i and bool(em[b, 0, i, j]) and bool(allow[qm[b, i], km[b, j]])
         and bool(kv[b, j]),
         lambda b, h, i, j: -slopes[h] * abs(i - j)),
    ]
    return (B, H, Sq, Sk), cases


SHAPE, CASES = mask_cases()


@pytest.mark.parametrize("name,masks,rule,bias_fn", CASES, ids=[c[0] for c in CASES])
def test_bruteforce_forward(name, masks, rule, bias_fn):
    B, H, Sq, Sk = SHAPE
    D = 5
    q, k, v = rnd((B, H, Sq, D), 1), rnd((B, H, Sk, D), 2), rnd((B, H, Sk, 3), 3)
    scale = 0.37
    O, L = oracle.attention_fwd(q, k, v, scale, **masks)
    for b in range(B):
        for h in range(H):
            bf = (lambda i, j: bias_fn(b, h, i, j)) if bias_fn else None
            On, Ln = naive_attention(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), scale,
                                     lambda i, j: rule(b, h, i, j), bf)
            np.testing.assert_allclose(O[b, h], np.array(On), rtol=0, atol=1e-12)
            Ln = np.array(Ln)
            assert np.array_equal(np.isinf(L[b, h]), np.isinf(Ln))
            fin = np.isfinite(Ln)
            np.testing.assert_allclose(L[b, h][fin], Ln[fin], rtol=0, atol=1e-12)


def test_rows_sum_to_one_and_masked_entries_zero():
    B, H, Sq, Sk = SHAPE
    for name, masks, rule, _ in CASES:
        q, k = rnd((B, H, Sq, 6), 11), rnd((B, H, Sk, 6), 12)
        for b in range(B):
            for h in range(H):
                P = oracle.probabilities(q, k, 0.9, b, h, **masks)
                rows = P.sum(axis=1)
                live = np.array([any(rule(b, h, i, j) for j in range(Sk)) for i in range(Sq)])
                assert np.all(np.abs(rows[live] - 1.0) <= 1e-12), name
                assert np.all(rows[~live] == 0.0), name
                for i in range(Sq):
                    for j in range(Sk):
                        if not rule(b, h, i, j):
                            assert P[i, j] == 0.0


def test_zero_query_gives_mean_of_allowed_values():
    B, H, S, D = 2, 3, 9, 4
    q = np.zeros((B, H, S, D))
    k, v = rnd((B, H, S, D), 21), rnd((B, H, S, D), 22)
    kv = np.ones((B, S), dtype=bool)
    kv[0, 3] = kv[1, 0] = kv[1, 5] = False
    O, L = oracle.attention_fwd(q, k, v, 0.5, causal=True, key_valid=kv)
    for b in range(B):
        for h in range(H):
            for i in range(S):
                idx = [j for j in range(i + 1) if kv[b, j]]
                if not idx:
                    assert np.all(O[b, h, i] == 0) and L[b, h, i] == -np.inf
                    continue
                np.testing.assert_allclose(O[b, h, i], v[b, h, idx].mean(axis=0), atol=1e-13)
                assert abs(L[b, h, i] - math.log(len(idx))) < 1e-13
    # causal only: LSE_i = ln(i + 1)
    O, L = oracle.attention_fwd(q, k, v, 0.5, causal=True)
    np.testing.assert_allclose(L[0, 0], np.log(np.arange(1, S + 1)), atol=1e-13)


def test_single_allowed_key_returns_its_value_row():
    B, H, Sq, Sk, D = 1, 2, 6, 9, 4
    q, k, v = rnd((B, H, Sq, D), 31), rnd((B, H, Sk, D), 32), rnd((B, H, Sk, D), 33)
    pick = np.random.default_rng(3).integers(0, Sk, Sq)
    em = np.zeros((1, 1, Sq, Sk), dtype=bool)
    em[0, 0, np.arange(Sq), pick] = True
    O, L = oracle.attention_fwd(q, k, v, 0.7, explicit_mask=em)
    for h in range(H):
        np.testing.assert_array_equal(O[0, h], v[0, h, pick])
        s = 0.7 * np.einsum("id,id->i", q[0, h], k[0, h, pick])
        np.testing.assert_allclose(L[0, h], s, atol=1e-14)


def test_single_key_sequence_forward_and_backward():
    B, H, Sq, D = 2, 2, 5, 3
    q, k, v = rnd((B, H, Sq, D), 41), rnd((B, H, 1, D), 42), rnd((B, H, 1, D), 43)
    do = rnd((B, H, Sq, D), 44)
    O, _ = oracle.attention_fwd(q, k, v, 0.3)
    np.testing.assert_allclose(O, np.broadcast_to(v, O.shape), atol=1e-15)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.3)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    np.testing.assert_allclose(dv[:, :, 0], do.sum(axis=2), atol=1e-13)


def test_row_constant_shifts_only_lse():
    B, H, Sq, Sk, D = 1, 2, 6, 7, 4
    q, k, v = rnd((B, H, Sq, D), 51), rnd((B, H, Sk, D), 52), rnd((B, H, Sk, D), 53)
    c = rnd((1, H, Sq, 1), 54) * 5
    pse = np.broadcast_to(c, (1, H, Sq, Sk)).copy()
    O0, L0 = oracle.attention_fwd(q, k, v, 0.5, causal=True)
    O1, L1 = oracle.attention_fwd(q, k, v, 0.5, causal=True, pse=pse)
    np.testing.assert_allclose(O1, O0, atol=1e-13)
    np.testing.assert_allclose(L1, L0 + c[..., 0], atol=1e-12)


def test_alibi_causal_zero_query_closed_form():
    S, H = 12, 3
    q = np.zeros((1, H, S, 4))
    k = rnd((1, H, S, 4), 61)
    v = np.broadcast_to(np.arange(S, dtype=np.float64)[None, None, :, None], (1, H, S, 4)).copy()
    slopes = np.array([0.75, 0.25, 2.0 ** -8])
    O, L = oracle.attention_fwd(q, k, v, 1.0, causal=True, alibi_slopes=slopes)
    for h, m in enumerate(slopes):
        for i in range(S):
            lse = math.log((1 - math.exp(-m * (i + 1))) / (1 - math.exp(-m)))
            assert abs(L[0, h, i] - lse) < 1e-12
            w = np.exp(-m * (i - np.arange(i + 1)))
            assert abs(O[0, h, i, 0] - (w * np.arange(i + 1)).sum() / w.sum()) < 1e-12


def test_causal_is_bit_identical_to_explicit_tril():
    B, H, S, D = 2, 2, 9, 5
    q, k, v, do = (rnd((B, H, S, D), s) for s in (71, 72, 73, 74))
    tril = np.tril(np.ones((S, S), dtype=bool))[None, None]
    a = oracle.attention_fwd(q, k, v, 0.4, causal=True)
    b = oracle.attention_fwd(q, k, v, 0.4, explicit_mask=tril)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    ga = oracle.attention_bwd(q, k, v, do, 0.4, causal=True)
    gb = oracle.attention_bwd(q, k, v, do, 0.4, explicit_mask=tril)
    for x, y in zip(ga, gb):
        assert np.array_equal(x, y)


def test_key_permutation_invariance():
    B, H, Sq, Sk, D = 1, 2, 6, 10, 4
    q, k, v = rnd((B, H, Sq, D), 81), rnd((B, H, Sk, D), 82), rnd((B, H, Sk, D), 83)
    em = np.random.default_rng(8).random((1, 1, Sq, Sk)) < 0.7
    perm = np.random.default_rng(9).permutation(Sk)
    O0, L0 = oracle.attention_fwd(q, k, v, 0.6, explicit_mask=em)
    O1, L1 = oracle.attention_fwd(q, k[:, :, perm], v[:, :, perm], 0.6,
                                  explicit_mask=em[..., perm])
    np.testing.assert_allclose(O1, O0, atol=1e-13)
    np.testing.assert_allclose(L1, L0, atol=1e-13)


# ----------------------------------------------------------------------------------
# library routine: torch SDPA in float64 on the CPU

def _sdpa(q, k, v, scale, add_mask):
    t = lambda x: torch.tensor(x, dtype=torch.float64)
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=t(add_mask), scale=scale)


def test_modality_and_padding_reduce_to_textbook_attention():
    """Multimodal workload rule (text attends to all valid keys, image to image
    only, text slots past the text length are padding) equals plain attention
    on the sliced key sets."""
    B, H, T, I, D = 3, 2, 6, 9, 4
    S = T + I
    q, k, v = rnd((B, H, S, D), 91), rnd((B, H, S, D), 92), rnd((B, H, S, D), 93)
    mod = np.zeros((B, S), dtype=np.int8)
    mod[:, T:] = 1
    tl = [2, 6, 4]
    kv = np.ones((B, S), dtype=bool)
    for b in range(B):
        kv[b, tl[b]:T] = False
    allow = np.array([[1, 1], [0, 1]], dtype=bool)
    O, L = oracle.attention_fwd(q, k, v, 0.5, q_modality=mod, k_modality=mod,
                                modality_allow=allow, key_valid=kv)
    for b in range(B):
        text_keys = [j for j in range(S) if kv[b, j]]
        img_keys = list(range(T, S))
        for rows, keys in ((range(0, T), text_keys), (range(T, S), img_keys)):
            rows = list(rows)
            zero = np.zeros((len(rows), len(keys)))
            ref = _sdpa(q[b][:, rows], k[b][:, keys], v[b][:, keys], 0.5, zero).numpy()
            np.testing.assert_allclose(O[b][:, rows], ref, atol=1e-13)
            s = 0.5 * q[b][:, rows] @ k[b][:, keys].transpose(0, 2, 1)
            lse = torch.logsumexp(torch.tensor(s), dim=-1).numpy()
            np.testing.assert_allclose(L[b][:, rows], lse, atol=1e-13)


def test_padding_equals_truncated_keys():
    B, H, Sq, Sk, D = 3, 2, 5, 11, 4
    q, k, v = rnd((B, H, Sq, D), 101), rnd((B, H, Sk, D), 102), rnd((B, H, Sk, D), 103)
    lens = [3, 11, 7]
    kv = np.arange(Sk)[None, :] < np.array(lens)[:, None]
    O, L = oracle.attention_fwd(q, k, v, 0.8, key_valid=kv)
    for b, n in enumerate(lens):
        Ot, Lt = oracle.attention_fwd(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.8)
        np.testing.assert_allclose(O[b], Ot[0], atol=1e-14)
        np.testing.assert_allclose(L[b], Lt[0], atol=1e-14)


@pytest.mark.parametrize("name,masks,rule,bias_fn", CASES, ids=[c[0] for c in CASES])
def test_against_torch_sdpa_forward_and_autograd(name, masks, rule, bias_fn):
    B, H, Sq, Sk = SHAPE
    D = 4
    q, k, v, do = rnd((B, H, Sq, D), 111), rnd((B, H, Sk, D), 112), rnd((B, H, Sk, D), 113), \
        rnd((B, H, Sq, D), 114)
    add = np.zeros((B, H, Sq, Sk))
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                for j in range(Sk):
                    if not rule(b, h, i, j):
                        add[b, h, i, j] = -np.inf
                    elif bias_fn is not None:
                        add[b, h, i, j] = bias_fn(b, h, i, j)
    live = np.isfinite(add).any(axis=-1)           # torch gives NaN on dead rows
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.tensor(add), scale=0.45)
    O, _ = oracle.attention_fwd(q, k, v, 0.45, **masks)
    ref = out.detach().numpy()
    np.testing.assert_allclose(O[live], ref[live], atol=1e-13)
    assert np.all(O[~live] == 0)
    # backward through torch autograd on the live rows only
    w = torch.tensor(live[..., None].astype(np.float64))
    (torch.nan_to_num(out) * torch.tensor(do) * w).sum().backward()
    do_live = do * live[..., None]
    dq, dk, dv = oracle.attention_bwd(q, k, v, do_live, 0.45, **masks)
    np.testing.assert_allclose(dq[live], tq.grad.numpy()[live], atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


# ----------------------------------------------------------------------------------
# backward: finite differences and invariants

@pytest.mark.parametrize("name,masks,rule,bias_fn", CASES, ids=[c[0] for c in CASES])
def test_backward_central_differences(name, masks, rule, bias_fn):
    B, H, Sq, Sk = SHAPE
    D = 3
    q, k, v, do = rnd((B, H, Sq, D), 121), rnd((B, H, Sk, D), 122), rnd((B, H, Sk, D), 123), \
        rnd((B, H, Sq, D), 124)
    scale = 0.55

    def loss(q_, k_, v_):
        O, _ = oracle.attention_fwd(q_, k_, v_, scale, **masks)
        return float((O * do).sum())

    grads = oracle.attention_bwd(q, k, v, do, scale, **masks)
    eps = 1e-6
    for which, g in zip(range(3), grads):
        base = [q, k, v]
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, which, idx, fd, g[idx])


def test_backward_invariants():
    B, H, Sq, Sk, D = 2, 2, 8, 8, 5
    q, k, v, do = rnd((B, H, Sq, D), 131), rnd((B, H, Sk, D), 132), rnd((B, H, Sk, D), 133), \
        rnd((B, H, Sq, D), 134)
    kv = np.ones((B, Sk), dtype=bool)
    kv[1, 2] = False
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.5, causal=True, key_valid=kv,
                                      alibi_slopes=np.array([0.3, 0.1]))
    live = np.ones((B, Sq), dtype=bool)
    for b in range(B):
        for i in range(Sq):
            live[b, i] = any(kv[b, j] for j in range(i + 1))
    np.testing.assert_allclose(dk.sum(axis=2), 0, atol=1e-12)
    for b in range(B):
        np.testing.assert_allclose(dv[b].sum(axis=1), do[b][:, live[b]].sum(axis=1), atol=1e-12)
    # dS rows sum to zero: sum_j dS_ij = 0 <=> dQ is orthogonal... check directly
    for b in range(B):
        for h in range(H):
            P = oracle.probabilities(q, k, 0.5, b, h, causal=True, key_valid=kv,
                                     alibi_slopes=np.array([0.3, 0.1]))
            dP = do[b, h] @ v[b, h].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            np.testing.assert_allclose(dS.sum(axis=1), 0, atol=1e-12)
            # dQ rows of dead queries are zero
            for i in range(Sq):
                if not live[b, i]:
                    assert np.all(dq[b, h, i] == 0)


# ----------------------------------------------------------------------------------
# layouts and the pages' own examples

def test_bsh_head_split_by_coordinates():
    B, S, H, D = 2, 5, 3, 4
    x = np.zeros((B, S, H * D))
    for b in range(B):
        for s in range(S):
            for h in range(H):
                for d in range(D):
                    x[b, s, h * D + d] = 1000 * b + 100 * s + 10 * h + d
    y = oracle.bsh_to_bnsd(x, H)
    for b in range(B):
        for h in range(H):
            for s in range(S):
                for d in range(D):
                    assert y[b, h, s, d] == 1000 * b + 100 * s + 10 * h + d
    assert np.array_equal(oracle.bnsd_to_bsh(y), x)


def _read_bits(name):
    rows = [ln.strip() for ln in open(os.path.join(GOLDEN, name)) if ln.strip() and
            not ln.startswith("#")]
    return np.array([[c == "1" for c in r] for r in rows])


def test_golden_cross_modal_mask_of_the_multimodal_page():
    want = _read_bits("cross_modal_mask_n24.txt")
    N = want.shape[0]
    mod = np.ones((2, N), dtype=np.int8)
    mod[:, :8] = 0
    allow = np.array([[0, 1], [1, 0]], dtype=bool)
    for b in range(2):
        got = oracle.allowed(b, 0, N, N, q_modality=mod, k_modality=mod, modality_allow=allow,
                             modality_allow_diag=True)
        assert np.array_equal(got, want)


def test_golden_causal_tril():
    want = _read_bits("causal_tril_s5.txt")
    assert np.array_equal(oracle.allowed(0, 0, 5, 5, causal=True), want)


def test_golden_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_two_keys.json")))
    O, L = oracle.attention_fwd(np.array(ex["q"]), np.array(ex["k"]), np.array(ex["v"]),
                                ex["scale"])
    np.testing.assert_allclose(O, np.array(ex["o"]), rtol=0, atol=ex["tolerance"])
    np.testing.assert_allclose(L, np.array(ex["lse"]), rtol=0, atol=ex["tolerance"])


def test_fully_masked_rows_are_zero_with_minus_inf_lse():
    q, k, v, do = rnd((1, 1, 4, 3), 141), rnd((1, 1, 5, 3), 142), rnd((1, 1, 5, 3), 143), \
        rnd((1, 1, 4, 3), 144)
    em = np.ones((1, 1, 4, 5), dtype=bool)
    em[0, 0, 2, :] = False
    O, L = oracle.attention_fwd(q, k, v, 1.0, explicit_mask=em)
    assert np.all(O[0, 0, 2] == 0) and L[0, 0, 2] == -np.inf
    assert np.all(np.isfinite(L[0, 0, [0, 1, 3]]))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 1.0, explicit_mask=em)
    assert np.all(dq[0, 0, 2] == 0)
    # the dead row's dO contributes nothing
    do2 = do.copy()
    do2[0, 0, 2] = 123.0
    g2 = oracle.attention_bwd(q, k, v, do2, 1.0, explicit_mask=em)
    for a, b in zip((dq, dk, dv), g2):
        np.testing.assert_array_equal(a, b)


# ----------------------------------------------------------------------------------
# dropout: the generator, the mask and the dropped attention

def test_philox_known_answer_vectors():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "philox4x32_10_kat.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        v = [int(x, 16) for x in r]
        got = oracle.philox4x32_10(*v[:6])
        assert [int(x) for x in got] == v[6:], r


def test_dropout_mask_element_rule():
    # element (i, j) of head (b, h) is word j % 4 of counter (j // 4, i, h, b), taken
    # here one scalar call at a time, against the vectorised mask
    b, h, Sq, Sk, seed = 1, 2, 5, 11, 0x0123456789ABCDEF
    for kp in (0.5, 0.8):
        m = oracle.dropout_mask(b, h, Sq, Sk, kp, seed)
        thr = math.floor(float(np.float32(kp)) * 2.0**32)
        for i in range(Sq):
            for j in range(Sk):
                w = oracle.philox4x32_10(j // 4, i, h, b, seed & 0xFFFFFFFF, seed >> 32)
                assert m[i, j] == (int(w[j % 4]) < thr)
    # keep_prob 0.5: the threshold is 2^31, so kept <=> the word's top bit is clear
    m = oracle.dropout_mask(0, 0, 3, 8, 0.5, 7)
    for i in range(3):
        for j in range(8):
            w = int(oracle.philox4x32_10(j // 4, i, 0, 0, 7, 0)[j % 4])
            assert m[i, j] == ((w >> 31) == 0)


@pytest.mark.parametrize("kp", [0.1, 0.5, 0.9])
def test_dropout_keep_fraction_and_independence(kp):
    n = 256
    m = oracle.dropout_mask(0, 0, n, n, kp, 1234)
    sd = math.sqrt(kp * (1 - kp) / n / n)
    assert abs(m.mean() - kp) < 6 * sd
    # another head, batch or seed gives an independent mask: agreement rate kp^2 + (1-kp)^2
    agree = kp * kp + (1 - kp) * (1 - kp)
    sd2 = math.sqrt(agree * (1 - agree) / n / n)
    for other in (oracle.dropout_mask(0, 1, n, n, kp, 1234), oracle.dropout_mask(1, 0, n, n, kp, 1234),
                  oracle.dropout_mask(0, 0, n, n, kp, 1235)):
        assert abs((m == other).mean() - agree) < 6 * sd2
    # the four words of one counter are not tied to each other
    c = np.array([m[:, j::4].mean() for j in range(4)])
    assert np.all(np.abs(c - kp) < 6 * math.sqrt(kp * (1 - kp) / (n * n / 4)))


def test_keep_prob_one_is_bit_identical_to_no_dropout():
    q, k, v, do = rnd((2, 2, 6, 3), 151), rnd((2, 2, 7, 3), 152), rnd((2, 2, 7, 3), 153), \
        rnd((2, 2, 6, 3), 154)
    a = oracle.attention_fwd(q, k, v, 0.7, causal=True)
    b = oracle.attention_fwd(q, k, v, 0.7, keep_prob=1.0, dropout_seed=99, causal=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    ga = oracle.attention_bwd(q, k, v, do, 0.7, causal=True)
    gb = oracle.attention_bwd(q, k, v, do, 0.7, keep_prob=1.0, dropout_seed=99, causal=True)
    for x, y in zip(ga, gb):
        np.testing.assert_array_equal(x, y)


def test_dropout_forward_bruteforce():
    # O_i = sum_j P_ij * keep_ij / kp * v_j term by term; LSE is the undropped one
    B, H, Sq, Sk, D, kp, seed = 1, 2, 5, 9, 3, 0.6, 42
    q, k, v = rnd((B, H, Sq, D), 161), rnd((B, H, Sk, D), 162), rnd((B, H, Sk, D), 163)
    O, L = oracle.attention_fwd(q, k, v, 0.8, keep_prob=kp, dropout_seed=seed, causal=True)
    _, L0 = oracle.attention_fwd(q, k, v, 0.8, causal=True)
    np.testing.assert_array_equal(L, L0)
    for h in range(H):
        P = oracle.probabilities(q, k, 0.8, 0, h, causal=True)
        M = oracle.dropout_mask(0, h, Sq, Sk, kp, seed)
        for i in range(Sq):
            for d in range(D):
                want = math.fsum(P[i, j] * (1.0 / float(np.float32(kp)) if M[i, j] else 0.0)
                                 * v[0, h, j, d] for j in range(Sk))
                assert abs(O[0, h, i, d] - want) < 1e-13


def test_dropout_is_unbiased_over_seeds():
    # E over seeds of the dropped output is the undropped output (the 1/kp scaling)
    B, H, Sq, Sk, D, kp = 1, 1, 3, 6, 2, 0.7
    q, k, v = rnd((B, H, Sq, D), 171), rnd((B, H, Sk, D), 172), rnd((B, H, Sk, D), 173)
    O0, _ = oracle.attention_fwd(q, k, v, 1.0)
    n = 3000
    acc = np.zeros_like(O0)
    for s in range(n):
        acc += oracle.attention_fwd(q, k, v, 1.0, keep_prob=kp, dropout_seed=s * 7919 + 1)[0]
    P = oracle.probabilities(q, k, 1.0)
    var = (P ** 2) @ (v[0, 0] ** 2) * (1.0 / kp - 1.0)          # per-element variance
    err = np.abs(acc / n - O0)[0, 0]
    assert np.all(err < 6 * np.sqrt(var / n) + 1e-12), (err, np.sqrt(var / n))


@pytest.mark.parametrize("masks", [dict(), dict(causal=True, alibi_slopes=np.array([0.4, 0.2]))],
                         ids=["plain", "causal_alibi"])
def test_dropout_backward_central_differences(masks):
    B, H, Sq, Sk, D, kp, seed = 1, 2, 4, 6, 3, 0.6, 2024
    q, k, v, do = rnd((B, H, Sq, D), 181), rnd((B, H, Sk, D), 182), rnd((B, H, Sk, D), 183), \
        rnd((B, H, Sq, D), 184)
    scale = 0.55

    def loss(q_, k_, v_):
        O, _ = oracle.attention_fwd(q_, k_, v_, scale, keep_prob=kp, dropout_seed=seed, **masks)
        return float((O * do).sum())

    grads = oracle.attention_bwd(q, k, v, do, scale, keep_prob=kp, dropout_seed=seed, **masks)
    # the mask really drops something here, and the gradient differs from the undropped one
    assert not oracle.dropout_mask(0, 0, Sq, Sk, kp, seed).all()
    g0 = oracle.attention_bwd(q, k, v, do, scale, **masks)
    assert not np.allclose(grads[2], g0[2])
    eps = 1e-6
    for which, g in zip(range(3), grads):
        base = [q, k, v]
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (which, idx, fd, g[idx])


# ----------------------------------------------------------------------------------
# MaxSim (retrieval page, "Layer 2: semantic modelling")

def _maxsim_bruteforce(q, d, qv, dv):
    """Term by term: math.fsum dot products, the mask rules written out."""
    B, Lq, D = q.shape
    Ld = d.shape[1]
    rows, scores = [], []
    for b in range(B):
        rm = []
        for i in range(Lq):
            best = -math.inf
            for j in range(Ld):
                if dv[b][j]:
                    best = max(best, math.fsum(float(q[b, i, k]) * float(d[b, j, k])
                                               for k in range(D)))
            rm.append(best if qv[b][i] else -math.inf)
        rows.append(rm)
        kept = [rm[i] for i in range(Lq) if qv[b][i]]
        scores.append(math.fsum(kept) / Lq if Lq else 0.0)
    return rows, scores


@pytest.mark.parametrize("Lq,Ld,D", [(1, 1, 1), (3, 5, 4), (6, 2, 3), (4, 7, 8)])
def test_maxsim_bruteforce(Lq, Ld, D):
    rng = np.random.default_rng(Lq * 100 + Ld * 10 + D)
    B = 3
    q, d = rng.standard_normal((B, Lq, D)), rng.standard_normal((B, Ld, D))
    qv, dv = rng.random((B, Lq)) < 0.8, rng.random((B, Ld)) < 0.7
    dv[0] = True                       # one sample with every document valid
    dv[2] = False                      # and one with none
    rows, scores = _maxsim_bruteforce(q, d, qv, dv)
    rm, sc = oracle.maxsim(q, d, qv, dv)
    for b in range(B):
        for i in range(Lq):
            if math.isinf(rows[b][i]):
                assert rm[b, i] == rows[b][i]
            else:
                assert abs(rm[b, i] - rows[b][i]) < 1e-12
        if math.isinf(scores[b]):
            assert sc[b] == scores[b]
        else:
            assert abs(sc[b] - scores[b]) < 1e-12


def test_maxsim_closed_forms():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 4, 6))
    # documents = the standard basis: the best match of q_i is its largest component
    d = np.broadcast_to(np.eye(6), (2, 6, 6)).copy()
    rm, sc = oracle.maxsim(q, d)
    np.testing.assert_array_equal(rm, q.max(axis=2))
    np.testing.assert_allclose(sc, q.max(axis=2).sum(axis=1) / 4, rtol=0, atol=1e-15)
    # one document: rowmax is that dot product
    d1 = rng.standard_normal((2, 1, 6))
    rm, _ = oracle.maxsim(q, d1)
    for b in range(2):
        for i in range(4):
            assert abs(rm[b, i] - sum(q[b, i, k] * d1[b, 0, k] for k in range(6))) < 1e-13
    # zero queries score 0 against any valid documents
    rm, sc = oracle.maxsim(np.zeros((2, 4, 6)), rng.standard_normal((2, 5, 6)))
    assert np.all(rm == 0) and np.all(sc == 0)


def test_maxsim_invariants():
    rng = np.random.default_rng(6)
    B, Lq, Ld, D = 2, 5, 9, 7
    q, d = rng.standard_normal((B, Lq, D)), rng.standard_normal((B, Ld, D))
    dv = rng.random((B, Ld)) < 0.6
    dv[:, 0] = True
    rm, sc = oracle.maxsim(q, d, d_valid=dv)
    # permuting the documents (with their mask) changes nothing
    perm = rng.permutation(Ld)
    rm2, sc2 = oracle.maxsim(q, d[:, perm], d_valid=dv[:, perm])
    np.testing.assert_allclose(rm2, rm, rtol=0, atol=1e-13)
    np.testing.assert_allclose(sc2, sc, rtol=0, atol=1e-13)
    # an invalid document never wins, whatever it holds
    d3 = d.copy()
    d3[~dv] = 1e6
    rm3, _ = oracle.maxsim(q, d3, d_valid=dv)
    np.testing.assert_array_equal(rm3, rm)
    # padding documents at the end equals dropping them
    lens = np.array([3, 9])
    dvp = np.arange(Ld)[None, :] < lens[:, None]
    rmp, scp = oracle.maxsim(q, d, d_valid=dvp)
    for b in range(B):
        rmt, sct = oracle.maxsim(q[b:b + 1], d[b:b + 1, :lens[b]])
        np.testing.assert_allclose(rmp[b], rmt[0], rtol=0, atol=1e-13)
        assert abs(scp[b] - sct[0]) < 1e-13
    # scaling the queries by c > 0 scales every max by c
    rm4, sc4 = oracle.maxsim(2.5 * q, d, d_valid=dv)
    np.testing.assert_allclose(rm4, 2.5 * rm, rtol=1e-13)


def test_maxsim_against_torch_on_the_pages_shapes():
    # the page's example sizes: 4 samples, 32 query and 256 document tokens, width 768,
    # no masks; torch float64 matmul, max over documents, sum / L_q
    g = torch.Generator().manual_seed(11)
    q = torch.randn(4, 32, 768, generator=g, dtype=torch.float64)
    d = torch.randn(4, 256, 768, generator=g, dtype=torch.float64)
    sim = torch.matmul(q, d.transpose(1, 2))
    want_rm = sim.max(dim=2).values
    want = want_rm.sum(dim=1) / 32
    rm, sc = oracle.maxsim(q, d)
    np.testing.assert_allclose(rm, want_rm.numpy(), rtol=1e-13, atol=1e-12)
    np.testing.assert_allclose(sc, want.numpy(), rtol=1e-13)


def test_maxsim_query_mask_and_empty_cases():
    rng = np.random.default_rng(7)
    q, d = rng.standard_normal((2, 4, 3)), rng.standard_normal((2, 5, 3))
    qv = np.array([[True, False, True, True], [False] * 4])
    rm, sc = oracle.maxsim(q, d, q_valid=qv)
    full, _ = oracle.maxsim(q, d)
    assert rm[0, 1] == -np.inf and np.all(rm[1] == -np.inf)
    assert abs(sc[0] - (full[0, 0] + full[0, 2] + full[0, 3]) / 4) < 1e-14
    assert sc[1] == 0.0                                  # no valid query token
    # no valid document: every valid query row is -inf, and so is the score
    rm, sc = oracle.maxsim(q, d, d_valid=np.zeros((2, 5), dtype=bool))
    assert np.all(rm == -np.inf) and np.all(sc == -np.inf)
    rm, sc = oracle.maxsim(q, np.zeros((2, 0, 3)))
    assert np.all(rm == -np.inf) and np.all(sc == -np.inf)
    # no query tokens at all
    rm, sc = oracle.maxsim(np.zeros((2, 0, 3)), d)
    assert rm.shape == (2, 0) and np.all(sc == 0.0)


# ----------------------------------------------------------------------------------
# the bias gradient dS (a learnable dense pse)

@pytest.mark.parametrize("extra", [dict(), dict(causal=True), dict(keep_prob=0.7, dropout_seed=9)],
                         ids=["dense", "dense_causal", "dense_dropout"])
def test_bias_gradient_central_differences(extra):
    B, H, Sq, Sk, D = 1, 2, 4, 5, 3
    q, k, v, do = rnd((B, H, Sq, D), 191), rnd((B, H, Sk, D), 192), rnd((B, H, Sk, D), 193), \
        rnd((B, H, Sq, D), 194)
    pse = rnd((B, H, Sq, Sk), 195)
    scale = 0.6

    def loss(ps):
        O, _ = oracle.attention_fwd(q, k, v, scale, pse=ps, **extra)
        return float((O * do).sum())

    *_, dbias = oracle.attention_bwd(q, k, v, do, scale, pse=pse, return_dbias=True, **extra)
    eps = 1e-6
    it = np.nditer(pse, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        plus, minus = pse.copy(), pse.copy()
        plus[idx] += eps
        minus[idx] -= eps
        fd = (loss(plus) - loss(minus)) / (2 * eps)
        assert abs(fd - dbias[idx]) <= 1e-7 * max(1.0, abs(fd)), (idx, fd, dbias[idx])
    # rows of dS sum to zero (adding a constant to a row's bias changes nothing)
    np.testing.assert_allclose(dbias.sum(axis=3), 0, atol=1e-12)
    if extra.get("causal"):
        assert np.all(dbias[..., np.triu_indices(Sq, 1, Sk)[0], np.triu_indices(Sq, 1, Sk)[1]] == 0)


# ----------------------------------------------------------------------------------
# fp8 inputs: the e4m3 decoding the fp8 forward's oracle inputs go through

def test_e4m3_decode_all_codes_against_torch():
    codes = np.arange(256)
    got = oracle.e4m3_decode(codes)
    want = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], want[~nan])
    # a few values written out: 1.0, the largest normal, the smallest subnormal, -2
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9
    assert got[0xC0] == -2.0


# ----------------------------------------------------------------------------------
# the row-restricted oracle (full-size sampled checks) against independent references

@pytest.mark.parametrize("name,masks,rule,bias_fn", CASES, ids=[c[0] for c in CASES])
def test_attention_rows_against_bruteforce_and_torch(name, masks, rule, bias_fn):
    """attention_rows on a subset of rows (in any order, repeats allowed) equals the
    term-by-term brute force (O, LSE) and torch autograd of the same masked,
    biased softmax in float64 (dQ) on those rows."""
    B, H, Sq, Sk = SHAPE
    D = 5
    q, k, v, do = rnd((B, H, Sq, D), 121), rnd((B, H, Sk, D), 122), rnd((B, H, Sk, D), 123), \
        rnd((B, H, Sq, D), 124)
    rows = np.array([6, 0, 3, 3, 5])
    for b in range(B):
        for h in range(H):
            O, L, dQ = oracle.attention_rows(q, k, v, do, 0.45, rows, b, h, **masks)
            NO, NL = naive_attention(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), 0.45,
                                     lambda i, j: rule(b, h, i, j),
                                     None if bias_fn is None else lambda i, j: bias_fn(b, h, i, j))
            for n, i in enumerate(rows):
                if NL[i] == -math.inf:
                    assert L[n] == -math.inf and np.all(O[n] == 0) and np.all(dQ[n] == 0)
                    continue
                np.testing.assert_allclose(O[n], NO[i], atol=1e-13)
                assert abs(L[n] - NL[i]) < 1e-13
            # dQ of the live rows: torch autograd of the same function of q
            add = np.array([[(bias_fn(b, h, i, j) if bias_fn else 0.0) if rule(b, h, i, j)
                             else -np.inf for j in range(Sk)] for i in range(Sq)])
            live = np.isfinite(add).any(axis=-1)
            tq = torch.tensor(q[b, h], requires_grad=True)
            s = 0.45 * tq @ torch.tensor(k[b, h]).T + torch.tensor(add)
            p = torch.softmax(s, dim=-1)
            out = torch.nan_to_num(p @ torch.tensor(v[b, h]))
            (out * torch.tensor(do[b, h] * live[:, None])).sum().backward()
            for n, i in enumerate(rows):
                if live[i]:
                    np.testing.assert_allclose(dQ[n], tq.grad.numpy()[i], atol=1e-12)


def test_attention_rows_match_the_whole_head_forms():
    """Every row at once equals attention_fwd / attention_bwd of the whole problem."""
    B, H, Sq, Sk = SHAPE
    D = 4
    q, k, v, do = rnd((B, H, Sq, D), 131), rnd((B, H, Sk, D), 132), rnd((B, H, Sk, D), 133), \
        rnd((B, H, Sq, D), 134)
    masks = CASES[-1][1]
    O, L = oracle.attention_fwd(q, k, v, 0.3, **masks)
    dq, _, _ = oracle.attention_bwd(q, k, v, do, 0.3, **masks)
    for b in range(B):
        for h in range(H):
            Or, Lr, dQr = oracle.attention_rows(q, k, v, do, 0.3, np.arange(Sq), b, h, **masks)
            np.testing.assert_allclose(Or, O[b, h], atol=1e-14)
            np.testing.assert_array_equal(np.isneginf(Lr), np.isneginf(L[b, h]))
            fin = np.isfinite(Lr)
            np.testing.assert_allclose(Lr[fin], L[b, h][fin], atol=1e-14)
            np.testing.assert_allclose(dQr, dq[b, h], atol=1e-13)
