"""The allocation-free backward (fa_bwd_noalloc, called through the C ABI)
against fa_bwd on the same inputs: two calls in a row, the second with a
smaller problem, so that the second reads row terms its own prep wrote over
the first call's in the shared device scratch.  Both must equal fa_bwd bit for
bit (the same kernels on the same inputs), and meet the oracle's bar."""
import math

import numpy as np
import pytest
import torch

import oracle
from tiled_attention_03_amd import binding as fa
from tiled_attention_03_amd import inputs

from gpu_util import DEV, assert_close, gpu_bwd, gpu_fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def problem(B, H, S, D, dtype, seed, causal=True, alibi=True):
    q, k, v, do = inputs.make_qkv(B, H, S, S, D, "BNSD", dtype, seed)
    pr = inputs.Problem(f"noalloc{seed}", B, H, S, S, D, "BNSD", dtype, 1.0 / math.sqrt(D),
                        q, k, v, do, causal=causal,
                        alibi_slopes=inputs.alibi_slopes(H) if alibi else None)
    return pr


def run_noalloc(pr, o, lse):
    q, k, v, do = (t.to(DEV) for t in (pr.q, pr.k, pr.v, pr.do))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa.bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, heads=pr.heads, layout=pr.layout,
                   **fa.problem_kwargs(pr, DEV))
    torch.cuda.synchronize()
    return dq, dk, dv


def test_noalloc_matches_fa_bwd_on_two_calls():
    big = problem(2, 4, 700, 128, torch.bfloat16, 5100)
    small = problem(1, 3, 300, 64, torch.float16, 5200, alibi=False)
    for pr in (big, small):
        print(f"\n{pr.name}: B={pr.batch} H={pr.heads} S={pr.seq_q} D={pr.head_dim}")
        o, lse = gpu_fwd(pr)
        got = run_noalloc(pr, o, lse)
        ref = gpu_bwd(pr, o, lse)
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(a, b), f"{name}: fa_bwd_noalloc differs from fa_bwd"
        rq, rk, rv = oracle.problem_bwd(pr)
        for name, a, r in zip(("dQ", "dK", "dV"), got, (rq, rk, rv)):
            assert_close(name, a, r, pr.dtype)


def test_noalloc_refuses_a_problem_past_its_scratch():
    q = torch.empty(1, 64, 70000, 64, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(1, 64, 70000, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError) as ei:
        fa.bwd_noalloc(q, q, q, q, lse, q, q, q, q, heads=64, scale=0.125)
    assert ei.value.status == fa.FA_ERR_WORKSPACE
