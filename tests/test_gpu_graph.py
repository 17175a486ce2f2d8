"""The forward and the allocation-free backward captured in a HIP graph (through
torch.cuda.CUDAGraph, the C ABI launching on the capturing stream) and
replayed.  The library makes no memset, allocation or synchronisation in these
calls, so the graph holds only its kernels.  Each replay runs on fresh input
values written into the captured buffers, with the outputs overwritten by NaN
and eager calls of the same entry points between replays; every replay must
equal the eager calls bit for bit (the kernels are deterministic), and the
first must meet the oracle's bar."""
import math

import pytest
import torch

import oracle
from tiled_attention_03_amd import binding as fa
from tiled_attention_03_amd import inputs

from gpu_util import DEV, assert_close, assert_lse

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    # (B, H, S, D, dtype, layout, causal, alibi)
    (1, 4, 333, 128, torch.bfloat16, "BNSD", True, True),
    (2, 3, 200, 64, torch.float16, "BSH", False, False),
]


def _problem(case, seed):
    B, H, S, D, dtype, layout, causal, alibi = case
    q, k, v, do = inputs.make_qkv(B, H, S, S, D, layout, dtype, seed)
    return inputs.Problem(f"graph{seed}", B, H, S, S, D, layout, dtype, 1.0 / math.sqrt(D),
                          q, k, v, do, causal=causal,
                          alibi_slopes=inputs.alibi_slopes(H) if alibi else None)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[5]}-D{c[3]}-{str(c[4])[6:]}")
def test_graph_replays_match_eager_calls(case):
    pr0 = _problem(case, 6100)
    print(f"\ngraph: B={pr0.batch} H={pr0.heads} S={pr0.seq_q} D={pr0.head_dim} {pr0.layout}",
          flush=True)
    kw = dict(heads=pr0.heads, layout=pr0.layout, **fa.problem_kwargs(pr0, DEV))
    q, k, v, do = (t.to(DEV).contiguous() for t in (pr0.q, pr0.k, pr0.v, pr0.do))
    o, dq, dk, dv = (torch.empty_like(t) for t in (q, q, k, v))
    lse = torch.empty(pr0.batch, pr0.heads, pr0.seq_q, dtype=torch.float32, device=DEV)

    def step():
        fa.fwd(q, k, v, out=o, lse=lse, **kw)
        fa.bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, **kw)

    # warm-up on a side stream (the noalloc entry point finds its scratch on
    # its first call), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        pr = _problem(case, 6100 + rep)   # rep 0: the captured values themselves
        for dst, src in zip((q, k, v, do), (pr.q, pr.k, pr.v, pr.do)):
            dst.copy_(src.to(DEV))
        for t in (o, dq, dk, dv, lse):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv)]
        # the same calls, eager, on the same inputs
        for t in (o, dq, dk, dv, lse):
            t.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), got, (o, lse, dq, dk, dv)):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
        if rep == 0:
            ro, rl = oracle.problem_fwd(pr)
            assert_close("O", got[0], ro, pr.dtype)
            assert_lse(got[1], rl)
            for name, a, r in zip(("dQ", "dK", "dV"), got[2:], oracle.problem_bwd(pr)):
                assert_close(name, a, r, pr.dtype)
