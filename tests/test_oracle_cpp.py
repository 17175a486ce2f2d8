"""Pins for the plain C++ fp64 oracle (oracle/fa_ref.cpp through oracle.cpp).

It is checked against things other than itself:
* the published Philox4x32-10 known-answer vectors (tests/golden);
* the pure-Python brute force of test_oracle_pins (math.fsum, its own mask
  rules) on every mask and bias case, forward;
* central finite differences of L = sum(O * dO) for the backward, including
  a dropout case;
* closed forms: Q = 0 gives the mean of the allowed V rows and LSE = ln of
  their count; one visible key returns its V row;
* the numpy oracle, an independently written implementation of the same
  definition, on problems with every field (masks, biases, dropout, BSH through
  the problem wrappers), forward, backward and dS.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import cpp
from tiled_attention_03_amd import inputs

from test_oracle_pins import CASES, GOLDEN, SHAPE, naive_attention, rnd


def test_philox_known_answer_vectors():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "philox4x32_10_kat.txt"))
            if ln.strip() and not ln.startswith("#")]
    for r in rows:
        v = [int(x, 16) for x in r]
        got = cpp.philox4x32_10(v[:4], v[4], v[5])
        assert [int(x) for x in got] == v[6:], r


@pytest.mark.parametrize("name,masks,rule,bias_fn", CASES, ids=[c[0] for c in CASES])
def test_bruteforce_forward(name, masks, rule, bias_fn):
    B, H, Sq, Sk = SHAPE
    q, k, v = rnd((B, H, Sq, 5), 1), rnd((B, H, Sk, 5), 2), rnd((B, H, Sk, 5), 3)
    scale = 0.37
    O, L = cpp.attention_fwd(q, k, v, scale, **masks)
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


@pytest.mark.parametrize("name,masks,rule,bias_fn", CASES[::2], ids=[c[0] for c in CASES[::2]])
@pytest.mark.parametrize("kp", [1.0, 0.6])
def test_backward_central_differences(name, masks, rule, bias_fn, kp):
    B, H, Sq, Sk = SHAPE
    D = 3
    q, k, v, do = rnd((B, H, Sq, D), 121), rnd((B, H, Sk, D), 122), rnd((B, H, Sk, D), 123), \
        rnd((B, H, Sq, D), 124)
    scale, seed = 0.55, 99

    def loss(q_, k_, v_):
        O, _ = cpp.attention_fwd(q_, k_, v_, scale, keep_prob=kp, dropout_seed=seed, **masks)
        return float((O * do).sum())

    grads = cpp.attention_bwd(q, k, v, do, scale, keep_prob=kp, dropout_seed=seed, **masks)
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


def test_closed_forms():
    B, H, Sq, Sk, D = 1, 2, 9, 9, 4
    v = rnd((B, H, Sk, D), 7)
    O, L = cpp.attention_fwd(np.zeros((B, H, Sq, D)), rnd((B, H, Sk, D), 8), v, 0.5, causal=True)
    for i in range(Sq):
        np.testing.assert_allclose(O[0, :, i], v[0, :, :i + 1].mean(axis=1), atol=1e-14)
        np.testing.assert_allclose(L[0, :, i], math.log(i + 1), atol=1e-14)
    em = np.zeros((Sq, Sk), dtype=bool)
    em[np.arange(Sq), (3 * np.arange(Sq)) % Sk] = True
    O, _ = cpp.attention_fwd(rnd((B, H, Sq, D), 9), rnd((B, H, Sk, D), 10), v, 0.5,
                             explicit_mask=em)
    for i in range(Sq):
        np.testing.assert_allclose(O[0, :, i], v[0, :, (3 * i) % Sk], atol=1e-15)


def numpy_vs_cpp_problem(kind):
    B, H, Sq, Sk, D = 2, 3, 23, 29, 6
    g = torch.Generator().manual_seed(17)
    q, k, v, do = (torch.randn(s, generator=g, dtype=torch.float64) for s in
                   ((B, H, Sq, D), (B, H, Sk, D), (B, H, Sk, D), (B, H, Sq, D)))
    pr = inputs.Problem("cpp_vs_numpy", B, H, Sq, Sk, D, "BNSD", torch.float64, 0.41, q, k, v, do)
    rng = np.random.default_rng(5)
    if kind in ("masks", "all"):
        pr.causal = True
        pr.explicit_mask = torch.from_numpy(rng.random((B, 1, Sq, Sk)) < 0.8)
        pr.q_modality = torch.from_numpy(rng.integers(0, 3, (B, Sq)).astype(np.int8))
        pr.k_modality = torch.from_numpy(rng.integers(0, 3, (B, Sk)).astype(np.int8))
        pr.modality_allow = torch.tensor([[1, 1, 0], [0, 1, 1], [1, 0, 1]], dtype=torch.bool)
        pr.modality_allow_diag = True
        pr.key_valid = torch.from_numpy(rng.random((B, Sk)) < 0.85)
    if kind in ("bias", "all"):
        pr.pse = torch.from_numpy(rng.standard_normal((1, H, Sq, Sk)))
    if kind == "alibi":
        pr.causal = True
        pr.alibi_slopes = inputs.alibi_slopes(H)
    if kind in ("dropout", "all"):
        pr.keep_prob, pr.dropout_seed = 0.7, 0x1234_5678_9ABC_DEF0
    return pr


@pytest.mark.parametrize("kind", ["plain", "masks", "bias", "alibi", "dropout", "all"])
def test_agrees_with_numpy_oracle(kind):
    pr = numpy_vs_cpp_problem(kind)
    kw = dict(keep_prob=pr.keep_prob, dropout_seed=pr.dropout_seed, **oracle.problem_masks(pr))
    O1, L1 = oracle.attention_fwd(pr.q, pr.k, pr.v, pr.scale, **kw)
    O2, L2 = cpp.attention_fwd(pr.q, pr.k, pr.v, pr.scale, **kw)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(L1), np.isneginf(L2))
    fin = np.isfinite(L1)
    np.testing.assert_allclose(L2[fin], L1[fin], rtol=0, atol=1e-12)
    G1 = oracle.attention_bwd(pr.q, pr.k, pr.v, pr.do, pr.scale, return_dbias=True, **kw)
    G2 = cpp.attention_bwd(pr.q, pr.k, pr.v, pr.do, pr.scale, return_dbias=True, **kw)
    for a, b in zip(G1, G2):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-11)


@pytest.mark.parametrize("layout", ["BNSD", "BSH"])
def test_problem_wrappers_agree_with_numpy_oracle(layout):
    pr = numpy_vs_cpp_problem("all")
    if layout == "BSH":
        to = lambda x: x.permute(0, 2, 1, 3).reshape(x.shape[0], x.shape[2], -1).contiguous()
        pr.q, pr.k, pr.v, pr.do = (to(t) for t in (pr.q, pr.k, pr.v, pr.do))
        pr.layout = "BSH"
    O1, L1 = oracle.problem_fwd(pr)
    O2, L2 = cpp.problem_fwd(pr)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-12)
    for a, b in zip(oracle.problem_bwd(pr), cpp.problem_bwd(pr)):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-11)
