"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compare it with the fp64 oracle element by element."""
import numpy as np
import torch

import oracle
from tiled_attention_03_amd import binding as fa
from tiled_attention_03_amd import inputs

DEV = "cuda:0"

# (max-abs, mean-abs) per input dtype, for O, dQ, dK, dV; LSE: 1e-3 absolute
TOL = {torch.float32: (1e-4, 1e-4), torch.float16: (5e-3, 5e-4), torch.bfloat16: (2e-2, 2e-3)}
LSE_TOL = 1e-3


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


# bits of mantissa of each output dtype (for its spacing at a given magnitude)
_MANT = {torch.float32: 23, torch.float16: 10, torch.bfloat16: 7}


def ulp(ref, dtype):
    """Spacing of ``dtype`` at |ref| (normal range; fp16 subnormals floor at 2^-24)."""
    a = np.abs(ref)
    floor = -14.0 if dtype == torch.float16 else -126.0
    e = np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0))), floor)
    return np.exp2(np.maximum(e, floor) - _MANT[dtype])


def errors(got, ref):
    g = got.detach().to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(g)), "non-finite values in the HIP output"
    e = np.abs(g - ref)
    return e


def assert_close(name, got, ref, dtype, grow=1.0):
    """Element-wise bar: |got - ref| <= tol_max + one ulp of the output dtype at
    |ref| (an output stored in a 16-bit format cannot be closer to the exact
    value than its own spacing allows), and mean |got - ref| <= tol_mean.

    ``grow`` widens both tolerances: with dropout the probabilities that
    multiply V and dP are P * Z with Z = 1/keep_prob on kept entries, and
    they, and O (which the backward's row terms D_i = dO_i . O_i read), are
    rounded to the 16-bit input format on the way; every absolute rounding
    error downstream is then up to 1/keep_prob times larger, so dropout
    cases use grow = 1/keep_prob."""
    e = errors(got, ref)
    if e.size == 0:
        return
    tmax, tmean = (t * grow for t in TOL[dtype])
    bar = tmax + ulp(ref, dtype)
    worst = int(np.argmax(e - bar))
    mx, mean = float(e.max()), float(e.mean())
    print(f"  {name}: max-abs {mx:.3e} (tol {tmax:g} + ulp), mean-abs {mean:.3e} "
          f"(tol {tmean:g}), max|ref| {np.abs(ref).max():.3g}")
    assert np.all(e <= bar), (f"{name}: error {e.flat[worst]:.3e} > bar {bar.flat[worst]:.3e} "
                              f"at ref {ref.flat[worst]:.4g}")
    assert mean <= tmean, f"{name}: mean-abs {mean:.3e}"


def assert_lse(got, ref):
    g = got.detach().cpu().double().numpy()
    dead_g, dead_r = np.isneginf(g), np.isneginf(ref)
    assert np.array_equal(dead_g, dead_r), "-inf LSE rows differ"
    assert np.all(np.isfinite(g[~dead_g])), "non-finite LSE"
    if (~dead_r).any():
        e = np.abs(g[~dead_r] - ref[~dead_r]).max()
        print(f"  LSE: max-abs {e:.3e} (tol {LSE_TOL:g})")
        assert e <= LSE_TOL


def check_fwd(pr, o=None, lse=None):
    if o is None:
        o, lse = gpu_fwd(pr)
    O, L = oracle.problem_fwd(pr)
    assert_close("O", o, O, pr.dtype, grow=_grow(pr))
    assert_lse(lse, L)
    return o, lse


def _grow(pr):
    return 1.0 / float(np.float32(pr.keep_prob))


def check_bwd(pr, o, lse):
    dq, dk, dv = gpu_bwd(pr, o, lse)
    rq, rk, rv = oracle.problem_bwd(pr)
    assert_close("dQ", dq, rq, pr.dtype, grow=_grow(pr))
    assert_close("dK", dk, rk, pr.dtype, grow=_grow(pr))
    assert_close("dV", dv, rv, pr.dtype, grow=_grow(pr))
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
