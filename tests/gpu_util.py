"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compare it with the fp64 oracle element by element.

The bar (the stated tolerances: max-abs 2e-2 / mean-abs 2e-3 for bf16 inputs,
5e-3 / 5e-4 for fp16, 1e-4 for the fp32 path; LSE 1e-3) is applied to the
value each kernel computes before its one final rounding to the output
format, and nothing more is allowed for that rounding than what it does.
Rounding to nearest is monotone, so an output element ``got`` can come from
some value x with |x - ref| <= tol exactly when

    |got - ref| <= tol + half the gap between got and its neighbour (in the
                        output format) on the side of ref,

which is what :func:`assert_close` checks.  It is never looser than the
plain bar plus half a spacing of the output format, the most one rounding
to nearest can move a value; and for values of the output format it is the
same test as "got lies between round(ref - tol) and round(ref + tol)".  The
mean-abs bar takes the same reading: the mean over elements of the distance
from ref to the values that round to got (|got - ref| less that half gap, or
0).  Applied to |got - ref| itself it would fail outputs that are ref
correctly rounded wherever they are large (a bf16 value near 19 has a
spacing of 1/8).  Comparing with round(ref)
instead would double the final rounding (the reference's and the kernel's)
and turn a difference of one part in 10^5 into a whole spacing wherever the
two straddle a rounding boundary.

Dropout (keep_prob < 1) adds, per element, the bound :func:`dropout_terms`
derives from the roundings the method itself performs: P o Z (Z = 1/kp on
kept entries) rounded to the input format before the P V, P^T dO products,
dS rounded before dS K and dS^T Q, and the backward's row terms
D_i = dO_i . O_i read from the forward's rounded O.  Its mean is added to the
mean bar.
"""
import json
import os

import numpy as np
import torch

import oracle
from tiled_attention_03_amd import binding as fa
from tiled_attention_03_amd import inputs

DEV = "cuda:0"

# (max-abs, mean-abs) per input dtype, for O, dQ, dK, dV; LSE: 1e-3 absolute
TOL = {torch.float32: (1e-4, 1e-4), torch.float16: (5e-3, 5e-4), torch.bfloat16: (2e-2, 2e-3)}
LSE_TOL = 1e-3
# unit roundoff (half a spacing, relative) of the 16-bit input formats
UNIT = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11, torch.float32: 2.0 ** -24}


def kwargs(pr):
    return fa.problem_kwargs(pr, DEV)


def gpu_fwd(pr):
    q, k, v = (t.to(DEV) for t in (pr.q, pr.k, pr.v))
    o, lse = fa.fwd(q, k, v, heads=pr.heads, layout=pr.layout, **kwargs(pr))
    torch.cuda.synchronize()
    return o, lse


def gpu_bwd(pr, o, lse):
    q, k, v, do = (t.to(DEV) for t in (pr.q, pr.k, pr.v, pr.do))
    g = fa.bwd(q, k, v, o, lse, do, heads=pr.heads, layout=pr.layout, **kwargs(pr))
    torch.cuda.synchronize()
    return g


def _log(rec):
    path = os.environ.get("FA_PARITY_LOG")
    if path:
        rec["test"] = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def rounding_slack(got_t: torch.Tensor, ref: np.ndarray) -> np.ndarray:
    """Half the gap between each element of ``got_t`` (in its own format) and
    its neighbour on the side of ``ref``: how far beyond ``got`` a value may
    lie and still round to it."""
    toward = torch.from_numpy(np.where(ref >= got_t.double().numpy(), np.inf, -np.inf))
    nb = torch.nextafter(got_t, toward.to(got_t.dtype)).double().numpy()
    g = got_t.double().numpy()
    gap = np.where(np.isfinite(nb), np.abs(nb - g), 0.0)
    return 0.5 * gap


def assert_close(name, got, ref, dtype, extra=None):
    """``got`` (a tensor in its output format) against the fp64 ``ref``, both bars
    applied to the values before their final rounding: every element within tol
    (+ ``extra``, a derived per-element bound, for dropout) of some value that
    rounds to it, and the mean over elements of the distance from ref to the
    values that round to got <= tol_mean (+ the mean of ``extra``)."""
    g_t = got.detach().to("cpu")
    if g_t.dtype not in (torch.float32, torch.float16, torch.bfloat16):
        g_t = g_t.float()
    g = g_t.double().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, f"{name}: shape {g.shape} != {ref.shape}"
    if g.size == 0:
        return
    assert np.all(np.isfinite(g)), f"{name}: non-finite values in the HIP output"
    tmax, tmean = TOL[dtype]
    bar = np.full(g.shape, tmax) if extra is None else tmax + np.asarray(extra)
    mean_bar = tmean if extra is None else tmean + float(np.mean(extra))
    e = np.abs(g - ref)
    slack = rounding_slack(g_t, ref)
    allowed = bar + slack
    ratio = e / allowed
    worst = int(np.argmax(ratio))
    mx, mean_raw = float(e.max()), float(e.mean())
    mean = float(np.maximum(e - slack, 0.0).mean())   # beyond what the output's rounding allows
    # for information: the difference from the reference rounded to the output format
    rr = float(np.abs(g - torch.from_numpy(ref).to(g_t.dtype).double().numpy()).max())
    print(f"  {name}: max-abs {mx:.3e} (tol {tmax:g}{' + derived' if extra is not None else ''}), "
          f"vs rounded ref {rr:.3e}, worst/bar {ratio.flat[worst]:.3f}, mean-abs {mean_raw:.3e}, "
          f"beyond rounding {mean:.3e} (tol {mean_bar:.3g}), max|ref| {np.abs(ref).max():.3g}")
    _log({"name": name, "max_abs": mx, "max_vs_rounded_ref": rr, "worst_ratio": float(ratio.flat[worst]),
          "mean_abs": mean_raw, "mean_beyond_rounding": mean, "mean_bar": mean_bar,
          "ref_at_worst": float(ref.flat[worst]),
          "max_ref": float(np.abs(ref).max()), "derived": extra is not None})
    assert ratio.flat[worst] <= 1.0, (f"{name}: error {e.flat[worst]:.3e} > bar {bar.flat[worst]:.3e} "
                                      f"(+ rounding {allowed.flat[worst] - bar.flat[worst]:.2e}) "
                                      f"at ref {ref.flat[worst]:.4g}")
    assert mean <= mean_bar, (f"{name}: mean-abs beyond the output's rounding {mean:.3e} > "
                              f"{mean_bar:.3e} (raw mean-abs {mean_raw:.3e})")


def assert_lse(got, ref):
    g = got.detach().cpu().double().numpy()
    dead_g, dead_r = np.isneginf(g), np.isneginf(ref)
    assert np.array_equal(dead_g, dead_r), "-inf LSE rows differ"
    assert np.all(np.isfinite(g[~dead_g])), "non-finite LSE"
    if (~dead_r).any():
        e = np.abs(g[~dead_r] - ref[~dead_r]).max()
        print(f"  LSE: max-abs {e:.3e} (tol {LSE_TOL:g})")
        _log({"name": "LSE", "max_abs": float(e), "worst_ratio": float(e / LSE_TOL)})
        assert e <= LSE_TOL


def _bnsd(x, pr):
    x = x.double().numpy() if hasattr(x, "double") else np.asarray(x, dtype=np.float64)
    return oracle.bsh_to_bnsd(x, pr.heads) if pr.layout == "BSH" else x


def _own_layout(x, pr):
    return oracle.bnsd_to_bsh(x) if pr.layout == "BSH" else x


def dropout_terms(pr, with_bwd=True):
    """Per-element bounds (in the problem's layout) on what the method's own
    roundings can add under dropout, with u the unit roundoff of the input
    format, P the undropped probabilities, Z = M / keep_prob:

      O_id : u sum_j P_ij Z_ij |v_jd|              (P o Z rounded before P V)
      dD_i : u sum_d |dO_id| (|O_id| + A_id)        (D_i read from the rounded O,
             A_id = sum_j P_ij Z_ij |v_jd|;          which carries the error above)
      dS_ij: P_ij dD_i + u |dS_ij|                   (dS rounded before its products)
      dQ_id: scale sum_j dS-bound_ij |k_jd|,   dK_jd: scale sum_i dS-bound_ij |q_id|
      dV_jd: u sum_i P_ij Z_ij |dO_id|               (P o Z rounded before P^T dO)

    First-order bounds: products of two roundings are dropped (they are
    below 2^-16 relative)."""
    u = UNIT[pr.dtype]
    q, k, v = _bnsd(pr.q, pr), _bnsd(pr.k, pr), _bnsd(pr.v, pr)
    masks = oracle.problem_masks(pr)
    B, H, Sq = q.shape[:3]
    Sk = k.shape[2]
    kp = float(np.float32(pr.keep_prob))
    tO = np.zeros(q.shape)
    out = {"O": tO}
    if with_bwd:
        do = _bnsd(pr.do, pr)
        O_ref, _ = oracle.attention_fwd(q, k, v, pr.scale, keep_prob=pr.keep_prob,
                                        dropout_seed=pr.dropout_seed, **masks)
        _, _, _, dS = oracle.attention_bwd(q, k, v, do, pr.scale, keep_prob=pr.keep_prob,
                                           dropout_seed=pr.dropout_seed, return_dbias=True,
                                           **masks)
        tQ, tK, tV = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
        tS = np.zeros((B, H, Sq, Sk))
    for b in range(B):
        for h in range(H):
            P = oracle.probabilities(q, k, pr.scale, b, h, **masks)
            Z = oracle.dropout_mask(b, h, Sq, Sk, pr.keep_prob, pr.dropout_seed) / kp
            PZ = P * Z
            A = PZ @ np.abs(v[b, h])
            tO[b, h] = u * A
            if not with_bwd:
                continue
            dD = u * (np.abs(do[b, h]) * (np.abs(O_ref[b, h]) + A)).sum(axis=1)
            sb = P * dD[:, None] + u * np.abs(dS[b, h])
            tS[b, h] = P * dD[:, None]
            tQ[b, h] = pr.scale * (sb @ np.abs(k[b, h]))
            tK[b, h] = pr.scale * (sb.T @ np.abs(q[b, h]))
            tV[b, h] = u * (PZ.T @ np.abs(do[b, h]))
    out["O"] = _own_layout(tO, pr)
    if with_bwd:
        out.update(dQ=_own_layout(tQ, pr), dK=_own_layout(tK, pr), dV=_own_layout(tV, pr), dS=tS)
    return out


def _dropout(pr):
    return float(np.float32(pr.keep_prob)) < 1.0


def check_fwd(pr, o=None, lse=None):
    if o is None:
        o, lse = gpu_fwd(pr)
    O, L = oracle.problem_fwd(pr)
    extra = dropout_terms(pr, with_bwd=False)["O"] if _dropout(pr) else None
    assert_close("O", o, O, pr.dtype, extra)
    assert_lse(lse, L)
    return o, lse


def check_bwd(pr, o, lse):
    dq, dk, dv = gpu_bwd(pr, o, lse)
    rq, rk, rv = oracle.problem_bwd(pr)
    t = dropout_terms(pr) if _dropout(pr) else {}
    assert_close("dQ", dq, rq, pr.dtype, t.get("dQ"))
    assert_close("dK", dk, rk, pr.dtype, t.get("dK"))
    assert_close("dV", dv, rv, pr.dtype, t.get("dV"))
    return dq, dk, dv


def head_slice(pr, h, o=None):
    """The sub-problem of head h (same batch), for sampled checks at full size."""
    sl = (lambda t: t[:, h:h + 1].contiguous()) if pr.layout == "BNSD" else \
        (lambda t: t[:, :, h * pr.head_dim:(h + 1) * pr.head_dim].contiguous())
    sub = inputs.Problem(f"{pr.name}_h{h}", pr.batch, 1, pr.seq_q, pr.seq_k, pr.head_dim,
                         pr.layout, pr.dtype, pr.scale, sl(pr.q), sl(pr.k), sl(pr.v),
                         None if pr.do is None else sl(pr.do), causal=pr.causal,
                         q_modality=pr.q_modality, k_modality=pr.k_modality,
                         modality_allow=pr.modality_allow,
                         modality_allow_diag=pr.modality_allow_diag, key_valid=pr.key_valid,
                         alibi_slopes=None if pr.alibi_slopes is None else
                         pr.alibi_slopes[h:h + 1].clone())
    if pr.explicit_mask is not None:
        em = pr.explicit_mask
        sub.explicit_mask = em[:, h:h + 1] if em.shape[1] > 1 else em
    if pr.pse is not None:
        ps = pr.pse
        sub.pse = ps[:, h:h + 1] if ps.shape[1] > 1 else ps
    return sub


def slice_out(t, pr, h):
    if pr.layout == "BNSD":
        return t[:, h:h + 1]
    return t[:, :, h * pr.head_dim:(h + 1) * pr.head_dim]
