"""GPU parity: the HIP path (called through the C ABI) against the fp64 oracle.

* the five workloads at their full sizes (the long-sequence one on sampled
  heads, which the oracle computes whole);
* a sweep over head_dim, dtype, layout, every mask kind and their
  combinations, ragged and unequal sequence lengths, forward and backward;
* edge cases: no keys, fully masked rows, zero inputs, large scores, ALiBi
  equal to the same bias given densely, repeatability, no writes outside the
  outputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tiled_attention_03_amd import binding as fa
from tiled_attention_03_amd import inputs

from gpu_util import (DEV, TOL, assert_close, assert_lse, check_bwd, check_fwd, dropout_terms, gpu_bwd,
                      gpu_fwd, head_slice, slice_out)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ----------------------------------------------------------------------------------
# the five workloads

@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_workload_forward_and_backward(cid):
    pr = inputs.config(cid)
    print(f"\n{pr.name}")
    o, lse = check_fwd(pr)
    check_bwd(pr, o, lse)


def test_long_sequence_sampled_heads():
    pr = inputs.config(5)
    print(f"\n{pr.name}")
    o, lse = gpu_fwd(pr)
    dq, dk, dv = gpu_bwd(pr, o, lse)
    for h in (0, 13, 22, 31):
        sub = head_slice(pr, h)
        print(f" head {h}")
        O, L = oracle.problem_fwd(sub)
        assert_close("O", slice_out(o, pr, h), O, pr.dtype)
        assert_lse(lse[:, h:h + 1], L)
        rq, rk, rv = oracle.problem_bwd(sub)
        assert_close("dQ", slice_out(dq, pr, h), rq, pr.dtype)
        assert_close("dK", slice_out(dk, pr, h), rk, pr.dtype)
        assert_close("dV", slice_out(dv, pr, h), rv, pr.dtype)


def _assert_plain(name, got, ref, tmax, tmean):
    """The stated bar with nothing allowed for an output rounding: max and
    mean of |got - ref| over every element."""
    e = np.abs(got.detach().cpu().double().numpy() - np.asarray(ref, dtype=np.float64))
    print(f"  {name} (plain bar): max-abs {e.max():.3e} (tol {tmax:g}), "
          f"mean-abs {e.mean():.3e} (tol {tmean:g})")
    assert e.max() <= tmax and e.mean() <= tmean, name


def test_long_sequence_plain_bar_float32_gradients():
    """The long workload in the launch configuration the benchmark times, O and
    LSE as produced (bf16 O, whose values lie well inside (-4, 4), so its
    rounding moves them by less than 2^-7) and dQ, dK, dV written in float32
    (no output rounding at all), against the stated tolerances taken
    literally: |got - ref| <= 2e-2 for every element, mean <= 2e-3."""
    pr = inputs.config(5)
    pr.grad_f32 = True
    print(f"\n{pr.name}, float32 gradients")
    o, lse = gpu_fwd(pr)
    dq, dk, dv = gpu_bwd(pr, o, lse)
    assert dq.dtype == torch.float32
    tmax, tmean = TOL[torch.bfloat16]
    for h in (0, 31):
        sub = head_slice(pr, h)
        print(f" head {h}")
        O, L = oracle.problem_fwd(sub)
        _assert_plain("O", slice_out(o, pr, h), O, tmax, tmean)
        assert_lse(lse[:, h:h + 1], L)
        rq, rk, rv = oracle.problem_bwd(sub)
        _assert_plain("dQ", slice_out(dq, pr, h), rq, tmax, tmean)
        _assert_plain("dK", slice_out(dk, pr, h), rk, tmax, tmean)
        _assert_plain("dV", slice_out(dv, pr, h), rv, tmax, tmean)


def test_long_sequence_every_head_sampled_rows():
    """Every head of the long workload at full size, in the launch configuration
    the benchmark times: O, LSE and dQ of sampled query rows (tile edges, the
    first and last rows, and seeded random ones) against the row-restricted
    oracle, which forms only those rows of each head's score matrix."""
    pr = inputs.config(5)
    print(f"\n{pr.name}")
    o, lse = gpu_fwd(pr)
    dq, _, _ = gpu_bwd(pr, o, lse)
    edges = [0, 1, 31, 32, 63, 64, 127, 128, 129, 2047, 4096, 6143, 8190, 8191]
    rng = np.random.default_rng(5151)
    for h in range(pr.heads):
        rows = np.array(edges + sorted(rng.choice(pr.seq_q, 6, replace=False).tolist()))
        O, L, dQ = oracle.attention_rows(pr.q[:, h:h + 1], pr.k[:, h:h + 1], pr.v[:, h:h + 1],
                                         pr.do[:, h:h + 1], pr.scale, rows, causal=pr.causal,
                                         alibi_slopes=pr.alibi_slopes[h:h + 1])
        idx = torch.tensor(rows, device=o.device)
        assert_close(f"O h{h}", o[0, h].index_select(0, idx), O, pr.dtype)
        assert_lse(lse[0, h].index_select(0, idx), L)
        assert_close(f"dQ h{h}", dq[0, h].index_select(0, idx), dQ, pr.dtype)


def test_long_sequence_forward_more_heads():
    pr = inputs.config(5, with_do=False)
    o, lse = gpu_fwd(pr)
    for h in (7, 16, 24):
        sub = head_slice(pr, h)
        print(f"\n head {h}")
        O, L = oracle.problem_fwd(sub)
        assert_close("O", slice_out(o, pr, h), O, pr.dtype)
        assert_lse(lse[:, h:h + 1], L)


# ----------------------------------------------------------------------------------
# sweep

def make_case(B, H, Sq, Sk, D, dtype, layout, mask, seed):
    q, k, v, do = inputs.make_qkv(B, H, Sq, Sk, D, layout, dtype, 100 * seed)
    g = torch.Generator().manual_seed(seed)
    pr = inputs.Problem(f"sweep{seed}", B, H, Sq, Sk, D, layout, dtype, 1.0 / math.sqrt(D),
                        q, k, v, do)
    if "causal" in mask:
        pr.causal = True
    if "explicit" in mask:
        pr.explicit_mask = torch.rand(B, 1, Sq, Sk, generator=g) < 0.7
    if "modality" in mask:
        M = 3
        pr.q_modality = torch.randint(0, M, (B, Sq), generator=g, dtype=torch.int8)
        pr.k_modality = torch.randint(0, M, (B, Sk), generator=g, dtype=torch.int8)
        pr.modality_allow = torch.tensor([[1, 1, 0], [0, 1, 1], [1, 0, 1]], dtype=torch.bool)
        pr.modality_allow_diag = "diag" in mask
    if "padding" in mask:
        lens = torch.randint(1, Sk + 1, (B,), generator=g)
        pr.key_valid = torch.arange(Sk)[None, :] < lens[:, None]
    if "holes" in mask:
        pr.key_valid = torch.rand(B, Sk, generator=g) < 0.8
    if "alibi" in mask:
        pr.alibi_slopes = inputs.alibi_slopes(H)
    if "dense" in mask:
        pr.pse = torch.randn(1, H, Sq, Sk, generator=g)
    return pr


SWEEP = []
_seed = 1
for D in (64, 128):
    for dtype in (torch.bfloat16, torch.float16):
        for (Sq, Sk) in ((1, 1), (7, 65), (64, 64), (65, 129), (130, 63), (200, 333)):
            for mask in ("none", "causal", "padding", "causal+alibi"):
                if dtype == torch.float16 and mask == "padding":
                    continue
                SWEEP.append((1, 2, Sq, Sk, D, dtype, "BNSD", mask, _seed))
                _seed += 1
for mask in ("explicit", "modality", "modality+diag", "holes", "dense", "causal+explicit+alibi",
             "modality+holes+causal", "dense+padding"):
    SWEEP.append((2, 3, 97, 150, 64, torch.bfloat16, "BNSD", mask, _seed))
    _seed += 1
    SWEEP.append((2, 2, 160, 96, 128, torch.bfloat16, "BSH", mask, _seed))
    _seed += 1
for D in (32, 64, 128):
    for mask in ("none", "causal+alibi", "explicit+holes", "modality+diag+dense"):
        SWEEP.append((2, 2, 70, 45, D, torch.float32, "BNSD", mask, _seed))
        _seed += 1
SWEEP.append((2, 3, 33, 70, 64, torch.float32, "BSH", "causal+padding", _seed))
_seed += 1
# ALiBi without the causal rule, large enough for full tiles wholly below and
# wholly above the diagonal (the forward's per-element fold on both sides)
for D, dtype, layout in ((64, torch.bfloat16, "BNSD"), (128, torch.bfloat16, "BNSD"),
                         (128, torch.float16, "BSH")):
    SWEEP.append((1, 2, 600, 600, D, dtype, layout, "alibi", _seed))
    _seed += 1


@pytest.mark.parametrize("B,H,Sq,Sk,D,dtype,layout,mask,seed", SWEEP,
                         ids=[f"{c[5]}-D{c[4]}-{c[6]}-{c[2]}x{c[3]}-{c[7]}".replace("torch.", "")
                              for c in SWEEP])
def test_sweep(B, H, Sq, Sk, D, dtype, layout, mask, seed):
    pr = make_case(B, H, Sq, Sk, D, dtype, layout, mask, seed)
    o, lse = check_fwd(pr)
    check_bwd(pr, o, lse)


# ----------------------------------------------------------------------------------
# edge cases

def test_no_keys_gives_zero_output_and_minus_inf_lse():
    pr = make_case(2, 2, 40, 0, 64, torch.bfloat16, "BNSD", "none", 901)
    o, lse = gpu_fwd(pr)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    dq, dk, dv = gpu_bwd(pr, o, lse)
    assert torch.all(dq == 0) and dk.numel() == 0 and dv.numel() == 0


@pytest.mark.parametrize("dtype,mask,gf32", [(torch.bfloat16, "causal", False),
                                             (torch.bfloat16, "none", False),
                                             (torch.float16, "padding", False),
                                             (torch.bfloat16, "causal+alibi", True),
                                             (torch.float32, "none", False)])
def test_no_queries_gives_zero_key_gradients(dtype, mask, gf32):
    """S_q = 0 with keys: no query sees a key, so dK = dV = 0 (written, not left as they were)."""
    pr = make_case(2, 2, 0, 70, 64, dtype, "BNSD", mask, 909)
    pr.grad_f32 = gf32
    o, lse = gpu_fwd(pr)
    assert o.numel() == 0 and lse.numel() == 0
    q, k, v, do = (t.to(DEV) for t in (pr.q, pr.k, pr.v, pr.do))
    gdt = torch.float32 if gf32 else dtype
    dk = torch.full(k.shape, 7.0, dtype=gdt, device=DEV)
    dv = torch.full(v.shape, 7.0, dtype=gdt, device=DEV)
    plan = fa.Plan(q, k, heads=pr.heads, layout=pr.layout, **fa.problem_kwargs(pr, DEV))
    plan.bwd_main(q, k, v, lse, do, dk, dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)
    dq, dk2, dv2 = gpu_bwd(pr, o, lse)
    assert dq.numel() == 0 and torch.all(dk2 == 0) and torch.all(dv2 == 0)
    rq, rk, rv = oracle.problem_bwd(pr)
    assert np.all(np.asarray(rk) == 0) and np.all(np.asarray(rv) == 0)


def test_fully_masked_rows():
    pr = make_case(1, 2, 50, 70, 128, torch.bfloat16, "BNSD", "explicit", 902)
    pr.explicit_mask[:, :, 5] = False
    pr.explicit_mask[:, :, 33] = False
    o, lse = check_fwd(pr)
    assert torch.all(o[:, :, 5] == 0) and torch.all(torch.isneginf(lse[:, :, 5]))
    dq, _, _ = check_bwd(pr, o, lse)
    assert torch.all(dq[:, :, 33] == 0)


def test_zero_inputs():
    pr = make_case(1, 2, 100, 100, 64, torch.bfloat16, "BNSD", "causal", 903)
    pr.q.zero_(); pr.k.zero_(); pr.v.zero_()
    o, lse = check_fwd(pr)
    assert torch.all(o == 0)
    ref = torch.log(torch.arange(1, 101, dtype=torch.float64))
    assert torch.allclose(lse[0, 0].double().cpu(), ref, atol=1e-3)
    check_bwd(pr, o, lse)


@pytest.mark.parametrize("D,dtype,mask", [(128, torch.bfloat16, "causal+alibi"),
                                          (64, torch.float16, "causal"),
                                          (128, torch.float16, "causal"),
                                          (64, torch.bfloat16, "causal+alibi")])
def test_causal_band_several_workgroups(D, dtype, mask):
    """Causal problems whose diagonal band tiles and blocks take the pipelined
    paths with a per-element mask: several 128-row and 128-key workgroups."""
    pr = make_case(1, 2, 512, 512, D, dtype, "BNSD", mask, 960 + D)
    o, lse = check_fwd(pr)
    check_bwd(pr, o, lse)


SPLIT = [(2, 3, 300, 300, 128, torch.bfloat16, "BSH", "causal+alibi", 980),
         (2, 3, 257, 250, 64, torch.float16, "BSH", "causal", 981),
         (2, 3, 100, 260, 128, torch.bfloat16, "BSH", "none", 982),
         (1, 3, 260, 140, 64, torch.bfloat16, "BNSD", "causal+alibi", 983)]


@pytest.mark.parametrize("B,H,Sq,Sk,D,dtype,layout,mask,seed", SPLIT,
                         ids=[f"{c[6]}-D{c[4]}-{c[2]}x{c[3]}-{c[7]}" for c in SPLIT])
def test_producer_consumer_key_pass(B, H, Sq, Sk, D, dtype, layout, mask, seed):
    """Problems the producer/consumer key pass serves (causal rule with or without
    ALiBi, or no mask): several heads and batches, both layouts, ragged S_q and S_k."""
    pr = make_case(B, H, Sq, Sk, D, dtype, layout, mask, seed)
    o, lse = check_fwd(pr)
    check_bwd(pr, o, lse)


@pytest.mark.parametrize("mask", ["alibi", "causal+alibi", "causal"])
def test_scale_zero(mask):
    """scale = 0: the logits are the bias alone (uniform rows without ALiBi);
    the fast ALiBi forms divide the slope by the scale, so they stand aside."""
    pr = make_case(1, 2, 300, 300, 128, torch.bfloat16, "BNSD", mask, 970)
    pr.scale = 0.0
    o, lse = check_fwd(pr)
    check_bwd(pr, o, lse)


@pytest.mark.parametrize("scale", [1e-38, 1e-12])
@pytest.mark.parametrize("mask", ["alibi", "causal+alibi"])
def test_tiny_scale(mask, scale):
    """A positive scale small enough that slope / (scale log2 e) overflows
    (1e-38: slope / c near 1e38, past the float range once multiplied by a key
    offset) sends the ALiBi tiles to the per-element path; at 1e-12 the
    raw-unit forms run with slope / c near 1e12.  Either way the logits are the
    bias plus a negligible score term."""
    pr = make_case(1, 2, 300, 300, 128, torch.bfloat16, "BNSD", mask, 975)
    pr.scale = scale
    o, lse = check_fwd(pr)
    check_bwd(pr, o, lse)


@pytest.mark.parametrize("D", [64, 128])
def test_large_scores_exercise_running_max(D):
    pr = make_case(1, 2, 300, 300, D, torch.bfloat16, "BNSD", "causal", 904 + D)
    pr.q = (pr.q.float() * 4).to(torch.bfloat16)
    pr.k = (pr.k.float() * 4).to(torch.bfloat16)
    check_fwd(pr)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("mask", ["none", "causal+alibi", "alibi"])
def test_score_spike_in_a_late_tile(D, dtype, mask):
    """One key of head 0 (key 3, in the tile the forward visits last outside
    the causal band) scores about 180 base-2 units above every other key of
    the head: after the first tiles, an exponential taken against the running
    reference would overflow, so the workgroups of head 0 that meet it late
    must redo their tiles with the row max taken on each.  Head 1 is plain."""
    pr = make_case(1, 2, 300, 600, D, dtype, "BNSD", mask, 980 + D)
    if "causal" in mask:
        pr = make_case(1, 2, 600, 600, D, dtype, "BNSD", mask, 980 + D)
    g = torch.Generator().manual_seed(981 + D)
    u = torch.randn(D, generator=g)
    q, k = pr.q.float(), pr.k.float()
    q[0, 0] += u
    k[0, 0, 3] = 16.0 * u
    pr.q, pr.k = q.to(dtype), k.to(dtype)
    o, lse = check_fwd(pr)
    check_bwd(pr, o, lse)


@pytest.mark.parametrize("mask", ["none", "padding"])
def test_short_query_score_spike_in_a_late_tile(mask):
    """The short-query forward (S_q <= 32): one key of batch 0, head 0 (key 400,
    tile 12 of 32-key tiles) scores about 180 base-2 units above the rest, so
    the tiles after the first overflow against the reference the first tile
    set, and that wave must compute its tiles again with the row max on each."""
    D = 64
    pr = make_case(2, 2, 32, 500, D, torch.bfloat16, "BNSD", "none", 990)
    if mask == "padding":
        pr.key_valid = torch.arange(500)[None, :] < torch.tensor([[450], [300]])
    g = torch.Generator().manual_seed(991)
    u = torch.randn(D, generator=g)
    q, k = pr.q.float(), pr.k.float()
    q[0, 0] += u
    k[0, 0, 400] = 16.0 * u
    pr.q, pr.k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    o, lse = check_fwd(pr)
    check_bwd(pr, o, lse)


def test_alibi_equals_dense_bias_on_gpu():
    pr = make_case(1, 4, 150, 150, 64, torch.bfloat16, "BNSD", "causal+alibi", 905)
    o1, l1 = gpu_fwd(pr)
    sl = pr.alibi_slopes.double()
    i = torch.arange(150, dtype=torch.float64)
    dense = (-sl[:, None, None] * (i[:, None] - i[None, :]).abs()).float()[None]
    pr2 = make_case(1, 4, 150, 150, 64, torch.bfloat16, "BNSD", "causal", 905)
    pr2.pse = dense
    o2, l2 = gpu_fwd(pr2)
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-3


def test_forward_is_bitwise_repeatable():
    pr = make_case(2, 4, 300, 300, 128, torch.bfloat16, "BNSD", "causal+alibi", 906)
    o1, l1 = gpu_fwd(pr)
    o2, l2 = gpu_fwd(pr)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_outputs_do_not_spill_into_neighbours():
    """Outputs live in the middle of larger buffers filled with a sentinel."""
    pr = make_case(2, 3, 77, 90, 64, torch.bfloat16, "BSH", "causal+padding", 907)
    q, k, v, do = (t.to(DEV) for t in (pr.q, pr.k, pr.v, pr.do))
    pad = 2048

    def guarded(like):
        buf = torch.full((like.numel() + 2 * pad,), 7.0, dtype=like.dtype, device=DEV)
        return buf, buf[pad:pad + like.numel()].view(like.shape)

    ob, o = guarded(q)
    lb = torch.full((pr.batch * pr.heads * pr.seq_q + 2 * pad,), 7.0, device=DEV)
    lse = lb[pad:pad + pr.batch * pr.heads * pr.seq_q].view(pr.batch, pr.heads, pr.seq_q)
    fa.fwd(q, k, v, heads=pr.heads, layout=pr.layout, out=o, lse=lse, **fa.problem_kwargs(pr, DEV))
    torch.cuda.synchronize()
    for buf in (ob, lb):
        assert torch.all(buf[:pad] == 7) and torch.all(buf[-pad:] == 7)
    O, L = oracle.problem_fwd(pr)
    assert_close("O", o, O, pr.dtype)
    # backward through the step entry points into guarded buffers
    plan = fa.Plan(q, k, heads=pr.heads, layout=pr.layout, **fa.problem_kwargs(pr, DEV))
    dqb, dq = guarded(q)
    dkb, dk = guarded(k)
    dvb, dv = guarded(v)
    plan.bwd_prep(o, do)
    plan.bwd_main(q, k, v, lse, do, dk, dv)
    plan.bwd_post(q, k, v, lse, do, dq)
    torch.cuda.synchronize()
    for buf in (dqb, dkb, dvb):
        assert torch.all(buf[:pad] == 7) and torch.all(buf[-pad:] == 7)
    rq, rk, rv = oracle.problem_bwd(pr)
    assert_close("dQ", dq, rq, pr.dtype)
    assert_close("dK", dk, rk, pr.dtype)
    assert_close("dV", dv, rv, pr.dtype)


def test_backward_is_bitwise_repeatable():
    """The backward uses no atomics: two runs give identical bits."""
    pr = make_case(2, 4, 300, 300, 128, torch.bfloat16, "BNSD", "causal+alibi", 908)
    o, lse = gpu_fwd(pr)
    g1 = gpu_bwd(pr, o, lse)
    g2 = gpu_bwd(pr, o, lse)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


# ----------------------------------------------------------------------------------
# dropout (keep_prob < 1): the kernels regenerate the Philox keep mask; the oracle
# draws it from its own Philox

DROP = []
_dseed = 1000
for D in (64, 128):
    for dtype in (torch.bfloat16, torch.float16):
        for (Sq, Sk) in ((7, 65), (65, 129), (200, 333), (256, 256)):
            for mask, kp in (("none", 0.9), ("causal", 0.6), ("causal+alibi", 0.8),
                             ("padding", 0.5)):
                DROP.append((1, 2, Sq, Sk, D, dtype, "BNSD", mask, kp, _dseed))
                _dseed += 1
for mask, kp in (("explicit", 0.7), ("modality+diag", 0.9), ("dense", 0.75),
                 ("causal+explicit+alibi", 0.2)):
    DROP.append((2, 3, 97, 150, 64, torch.bfloat16, "BNSD", mask, kp, _dseed))
    _dseed += 1
    DROP.append((2, 2, 160, 96, 128, torch.bfloat16, "BSH", mask, kp, _dseed))
    _dseed += 1
DROP.append((1, 2, 1024, 1024, 128, torch.bfloat16, "BNSD", "causal+alibi", 0.9, _dseed))
_dseed += 1
# the BSH layout through the fast (pipelined) dropout paths
DROP.append((1, 3, 384, 384, 128, torch.float16, "BSH", "causal", 0.7, _dseed))
_dseed += 1
DROP.append((2, 2, 320, 320, 64, torch.bfloat16, "BSH", "none", 0.85, _dseed))


@pytest.mark.parametrize("B,H,Sq,Sk,D,dtype,layout,mask,kp,seed", DROP,
                         ids=[f"{c[5]}-D{c[4]}-{c[6]}-{c[2]}x{c[3]}-{c[7]}-kp{c[8]}"
                              .replace("torch.", "") for c in DROP])
def test_dropout(B, H, Sq, Sk, D, dtype, layout, mask, kp, seed):
    pr = make_case(B, H, Sq, Sk, D, dtype, layout, mask, seed)
    pr.keep_prob = kp
    pr.dropout_seed = (seed * 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
    o, lse = check_fwd(pr)
    check_bwd(pr, o, lse)


@pytest.mark.parametrize("D", [64, 128])
def test_dropout_mask_is_bit_exact(D):
    """Q = 0 makes P uniform (1/S_k) and V = I_D (S_k = D) copies P * keep / kp into O,
    so O * kp * S_k is the 0/1 keep mask itself; likewise dO = I_D (S_q = D) makes
    dV^T the mask as the key pass draws it."""
    B, H, kp, seed = 2, 3, 0.5, 0xDEADBEEF12345678
    S = D
    eye = torch.eye(D, dtype=torch.bfloat16)
    q = torch.zeros(B, H, S, D, dtype=torch.bfloat16)
    k = inputs.randn((B, H, S, D), torch.bfloat16, 77)
    v = eye.expand(B, H, S, D).contiguous()
    do = eye.expand(B, H, S, D).contiguous()
    pr = inputs.Problem("dropmask", B, H, S, S, D, "BNSD", torch.bfloat16, 1.0 / math.sqrt(D),
                        q, k, v, do, keep_prob=kp, dropout_seed=seed)
    o, lse = gpu_fwd(pr)
    dq, dk, dv = gpu_bwd(pr, o, lse)
    fm = (o.float().cpu() * kp * S).numpy()
    bm = (dv.float().cpu() * kp * S).numpy()
    for b in range(B):
        for h in range(H):
            want = oracle.dropout_mask(b, h, S, S, kp, seed)
            assert 0.3 < want.mean() < 0.7
            np.testing.assert_array_equal(fm[b, h], want.astype(np.float64))
            np.testing.assert_array_equal(bm[b, h].T, want.astype(np.float64))


def test_dropout_seed_changes_the_mask_and_repeats():
    pr = make_case(1, 2, 130, 130, 64, torch.bfloat16, "BNSD", "causal", 1900)
    pr.keep_prob = 0.7
    pr.dropout_seed = 5
    o1, _ = gpu_fwd(pr)
    o2, _ = gpu_fwd(pr)
    assert torch.equal(o1, o2)
    pr.dropout_seed = 6
    o3, _ = gpu_fwd(pr)
    assert not torch.equal(o1, o3)


# ----------------------------------------------------------------------------------
# float32 gradient outputs and the bias gradient

GRADF32 = []
_gseed = 2000
for D in (64, 128):
    for dtype in (torch.bfloat16, torch.float16):
        for mask, kp in (("none", 1.0), ("causal+alibi", 1.0), ("padding", 1.0), ("dense", 1.0),
                         ("causal", 0.8)):
            GRADF32.append((2, 2, 200, 333, D, dtype, "BNSD", mask, kp, _gseed))
            _gseed += 1
GRADF32.append((2, 2, 160, 96, 128, torch.bfloat16, "BSH", "modality+holes+causal", 1.0, _gseed))
GRADF32.append((1, 4, 1024, 1024, 128, torch.bfloat16, "BNSD", "causal+alibi", 1.0, _gseed + 1))


@pytest.mark.parametrize("B,H,Sq,Sk,D,dtype,layout,mask,kp,seed", GRADF32,
                         ids=[f"{c[5]}-D{c[4]}-{c[6]}-{c[2]}x{c[3]}-{c[7]}-kp{c[8]}"
                              .replace("torch.", "") for c in GRADF32])
def test_float32_gradients(B, H, Sq, Sk, D, dtype, layout, mask, kp, seed):
    """grad_f32 writes the kernels' own float32 values: rounded to the input dtype
    they are bit-identical to the 16-bit outputs, and they meet the parity bar."""
    pr = make_case(B, H, Sq, Sk, D, dtype, layout, mask, seed)
    pr.keep_prob, pr.dropout_seed = kp, seed
    o, lse = gpu_fwd(pr)
    g16 = gpu_bwd(pr, o, lse)
    pr.grad_f32 = True
    g32 = gpu_bwd(pr, o, lse)
    ref = oracle.problem_bwd(pr)
    terms = dropout_terms(pr) if kp < 1.0 else {}
    for name, a, b, r in zip(("dQ", "dK", "dV"), g16, g32, ref):
        assert b.dtype == torch.float32 and a.dtype == dtype
        # rounding the float32 value gives the 16-bit one, except at an exact tie between two
        # 16-bit neighbours: the fp16 key pass forms dK = acc * scale and its rounding in one
        # fused step (v_fma_mixlo_f16), i.e. from the exact product, not its float32 rounding
        rb = b.to(dtype)
        bad = rb != a
        if bad.any():
            bf, af, rf = b[bad].double(), a[bad].double(), rb[bad].double()
            assert torch.all((bf - af).abs() == (bf - rf).abs()), \
                f"{name}: float32 output does not round to the 16-bit one"
            print(f"  {name}: {int(bad.sum())} exact ties rounded the other way")
        assert_close(name, b, r, dtype, terms.get(name))


DPSE = [
    (2, 3, 97, 150, 64, torch.bfloat16, "BNSD", "dense", 1.0, 2100),
    (2, 2, 130, 130, 128, torch.bfloat16, "BNSD", "dense+causal", 1.0, 2101),
    (1, 2, 70, 300, 128, torch.float16, "BNSD", "dense+padding", 1.0, 2102),
    (2, 2, 160, 96, 128, torch.bfloat16, "BSH", "dense+causal", 0.75, 2103),
    (1, 2, 33, 65, 64, torch.bfloat16, "BNSD", "dense+explicit", 1.0, 2104),
]


@pytest.mark.parametrize("B,H,Sq,Sk,D,dtype,layout,mask,kp,seed", DPSE,
                         ids=[f"{c[7]}-{c[6]}-{c[2]}x{c[3]}-kp{c[8]}" for c in DPSE])
def test_bias_gradient(B, H, Sq, Sk, D, dtype, layout, mask, kp, seed):
    pr = make_case(B, H, Sq, Sk, D, dtype, layout, mask, seed)
    pr.keep_prob, pr.dropout_seed = kp, seed
    o, lse = gpu_fwd(pr)
    q, k, v, do = (t.to(DEV) for t in (pr.q, pr.k, pr.v, pr.do))
    dpse = torch.full((B, H, Sq, Sk), float("nan"), dtype=torch.float32, device=DEV)
    dq, dk, dv, dp = fa.bwd(q, k, v, o, lse, do, heads=pr.heads, layout=pr.layout, dpse=dpse,
                            **fa.problem_kwargs(pr, DEV))
    torch.cuda.synchronize()
    rq, rk, rv, rds = oracle.problem_bwd(pr, return_dbias=True)
    assert torch.isfinite(dp).all(), "bias gradient elements left unwritten"
    # dS_ij = P_ij (Z_ij dP_ij - D_i) is written in float32 before any rounding, but the row
    # term D_i = dO_i . O_i is read from O in the input format, which carries the forward's
    # roundings: dS may carry P_ij times that error bound (dropout_terms), undiluted by any sum
    extra = dropout_terms(pr)["dS"]
    assert_close("dpse", dp, rds, dtype, extra)
    if "causal" in mask:
        assert torch.all(dp.triu(1) == 0)
    # the other gradients are unchanged by asking for the bias gradient
    g = gpu_bwd(pr, o, lse)
    for a, b in zip((dq, dk, dv), g):
        assert torch.equal(a, b)


# ----------------------------------------------------------------------------------
# the fp32 path against the 16-bit path on the same values

@pytest.mark.parametrize("mask", ["none", "causal+alibi", "padding"])
def test_fp32_path_agrees_with_bf16_path(mask):
    """bf16 inputs, and the same values as float32: the two GPU paths (MFMA with
    16-bit operands, and fp32 FMA throughout) agree within the bf16 bar."""
    pr16 = make_case(2, 2, 150, 170, 64, torch.bfloat16, "BNSD", mask, 2500)
    pr32 = make_case(2, 2, 150, 170, 64, torch.bfloat16, "BNSD", mask, 2500)
    pr32.dtype = torch.float32
    pr32.q, pr32.k, pr32.v, pr32.do = (t.float() for t in (pr16.q, pr16.k, pr16.v, pr16.do))
    o16, l16 = gpu_fwd(pr16)
    o32, l32 = gpu_fwd(pr32)
    g16 = gpu_bwd(pr16, o16, l16)
    g32 = gpu_bwd(pr32, o32, l32)
    assert o32.dtype == torch.float32
    assert_close("O", o16, o32.double().cpu().numpy(), torch.bfloat16)
    assert_lse(l16, l32.double().cpu().numpy())
    for name, a, b in zip(("dQ", "dK", "dV"), g16, g32):
        assert_close(name, a, b.double().cpu().numpy(), torch.bfloat16)


# ----------------------------------------------------------------------------------
# explicit masks with block structure: the forward summarises each (query tile,
# key tile) of the mask, skips tiles it hides entirely and runs tiles it allows
# entirely without per-element work

def block_mask(B, Sq, Sk, seed, bq=64, bk=64, heads=1):
    """[B, heads, Sq, Sk] bool: blocks of bq x bk that are all True, all False or
    random, so that tiles of every kind occur (blocks do not align with every
    tile, on purpose, in some cases)."""
    g = torch.Generator().manual_seed(seed)
    nbq, nbk = (Sq + bq - 1) // bq, (Sk + bk - 1) // bk
    kind = torch.randint(0, 3, (B, heads, nbq, nbk), generator=g)
    rnd = torch.rand(B, heads, Sq, Sk, generator=g) < 0.5
    full = kind.repeat_interleave(bq, 2).repeat_interleave(bk, 3)[:, :, :Sq, :Sk]
    return torch.where(full == 0, torch.zeros_like(rnd), torch.where(full == 1,
                       torch.ones_like(rnd), rnd))


BLOCKS = [
    (2, 3, 256, 320, 64, torch.bfloat16, "BNSD", "explicit", 64, 64, 3100),
    (1, 2, 384, 384, 128, torch.bfloat16, "BNSD", "causal+explicit+alibi", 64, 64, 3101),
    (2, 2, 300, 200, 128, torch.float16, "BSH", "explicit", 128, 64, 3102),
    (1, 3, 200, 500, 64, torch.bfloat16, "BNSD", "explicit+holes", 50, 70, 3103),
    (1, 2, 256, 256, 64, torch.bfloat16, "BNSD", "explicit+dense", 64, 64, 3104),
]


@pytest.mark.parametrize("B,H,Sq,Sk,D,dtype,layout,mask,bq,bk,seed", BLOCKS,
                         ids=[f"{c[6]}-D{c[4]}-{c[2]}x{c[3]}-{c[7]}-b{c[8]}x{c[9]}" for c in BLOCKS])
def test_block_structured_explicit_mask(B, H, Sq, Sk, D, dtype, layout, mask, bq, bk, seed):
    pr = make_case(B, H, Sq, Sk, D, dtype, layout, mask, seed)
    pr.explicit_mask = block_mask(B, Sq, Sk, seed, bq, bk)
    o, lse = check_fwd(pr)
    check_bwd(pr, o, lse)


def test_block_mask_per_head_with_empty_query_tiles():
    """A per-head mask [B, H, S_q, S_k] that hides every key from whole query tiles
    (their rows get O = 0, LSE = -inf) and shows every key to others."""
    B, H, Sq, Sk = 1, 2, 300, 260
    pr = make_case(B, H, Sq, Sk, 128, torch.bfloat16, "BNSD", "explicit", 3110)
    em = block_mask(B, Sq, Sk, 3110, heads=H)
    em[:, 0, 128:256] = False
    em[:, 1, :128] = True
    pr.explicit_mask = em
    o, lse = check_fwd(pr)
    assert torch.all(o[:, 0, 128:256] == 0) and torch.all(torch.isneginf(lse[:, 0, 128:256]))
    check_bwd(pr, o, lse)


def test_explicit_mask_rows_with_padded_stride():
    """An explicit mask whose rows sit at a 16-byte-multiple stride wider than S_k
    (a view of a wider mask; the extra columns hold values that would change the
    result if read): the same result as the contiguous mask."""
    B, H, Sq, Sk = 2, 2, 200, 250
    pr = make_case(B, H, Sq, Sk, 64, torch.bfloat16, "BNSD", "explicit", 3120)
    pr.explicit_mask = block_mask(B, Sq, Sk, 3120, 64, 64)
    wide = torch.zeros(B, 1, Sq, 256, dtype=torch.bool, device=DEV)
    wide[..., Sk:] = True
    wide[..., :Sk] = pr.explicit_mask.to(DEV)
    view = wide[..., :Sk]
    assert view.stride(2) == 256
    kw = fa.problem_kwargs(pr, DEV)
    kw["explicit_mask"] = view
    q, k, v = (t.to(DEV) for t in (pr.q, pr.k, pr.v))
    o, lse = fa.fwd(q, k, v, heads=pr.heads, layout=pr.layout, **kw)
    torch.cuda.synchronize()
    check_fwd(pr, o, lse)


# ----------------------------------------------------------------------------------
# key ranges longer than one tile list (1024 tiles of 64 keys): the forward walks
# them in chunks

LONGK = [
    (1, 1, 64, 70000, 64, torch.bfloat16, "BNSD", "padding", 3200),
    (1, 2, 40, 66000, 128, torch.float16, "BSH", "none", 3201),
    (1, 1, 70, 65600, 128, torch.bfloat16, "BNSD", "alibi", 3202),
    (1, 1, 64, 66000, 64, torch.bfloat16, "BNSD", "holes+explicit", 3203),
]


@pytest.mark.parametrize("B,H,Sq,Sk,D,dtype,layout,mask,seed", LONGK,
                         ids=[f"{c[6]}-D{c[4]}-{c[2]}x{c[3]}-{c[7]}" for c in LONGK])
def test_key_range_past_one_tile_list(B, H, Sq, Sk, D, dtype, layout, mask, seed):
    pr = make_case(B, H, Sq, Sk, D, dtype, layout, mask, seed)
    if "explicit" in mask:
        pr.explicit_mask = block_mask(B, Sq, Sk, seed, 64, 4096)
    o, lse = check_fwd(pr)
    check_bwd(pr, o, lse)


# ----------------------------------------------------------------------------------
# short query blocks (S_q <= 32, S_k <= 2048, causal / padding masks, ALiBi or no
# bias): one wave per (batch, head) with K streamed into registers; every tile takes
# the per-element rules.  Past those limits the list-based one-wave workgroup runs.

SHORT = [
    (3, 4, 32, 512, 64, torch.bfloat16, "BSH", "padding", 3400),
    (2, 3, 17, 2048, 64, torch.bfloat16, "BNSD", "padding", 3401),
    (2, 3, 32, 2049, 64, torch.bfloat16, "BNSD", "padding", 3402),
    (2, 2, 1, 33, 128, torch.float16, "BSH", "causal+alibi", 3403),
    (2, 2, 32, 100, 128, torch.bfloat16, "BNSD", "alibi", 3404),
    (2, 2, 20, 31, 64, torch.float16, "BNSD", "causal+padding", 3405),
    (4, 2, 32, 700, 64, torch.bfloat16, "BSH", "holes", 3406),
    (2, 3, 29, 96, 128, torch.bfloat16, "BSH", "none", 3407),
    (1, 2, 32, 1, 64, torch.bfloat16, "BNSD", "none", 3408),
    (2, 2, 24, 500, 64, torch.bfloat16, "BNSD", "explicit", 3409),
    (2, 2, 32, 2048, 128, torch.float16, "BSH", "alibi+padding", 3411),
    (2, 3, 32, 1000, 64, torch.bfloat16, "BNSD", "causal+alibi+holes", 3412),
    (3, 2, 9, 300, 128, torch.bfloat16, "BNSD", "holes", 3413),
]


@pytest.mark.parametrize("B,H,Sq,Sk,D,dtype,layout,mask,seed", SHORT,
                         ids=[f"{c[6]}-D{c[4]}-{c[2]}x{c[3]}-{c[7]}" for c in SHORT])
def test_short_query_blocks(B, H, Sq, Sk, D, dtype, layout, mask, seed):
    pr = make_case(B, H, Sq, Sk, D, dtype, layout, mask, seed)
    o, lse = check_fwd(pr)
    check_bwd(pr, o, lse)


def test_short_query_sample_without_valid_keys():
    """A sample whose keys are all padding: its rows get O = 0 and LSE = -inf, the
    other samples are unaffected."""
    pr = make_case(3, 2, 32, 300, 64, torch.bfloat16, "BSH", "padding", 3410)
    pr.key_valid[1] = False
    o, lse = check_fwd(pr)
    assert torch.all(o[1] == 0) and torch.all(torch.isneginf(lse[1]))
    check_bwd(pr, o, lse)


# ----------------------------------------------------------------------------------
# run-time switches: FA_TILE picks the forward workgroup shape (results agree with
# the oracle either way), FA_LOG reports the kernel each call launches

@pytest.mark.parametrize("tile,Sq,want", [("wg4", 32, "NW=4"), ("wg1", 200, "NW=1"),
                                          ("wg1", 32, "NW=1"), ("auto", 32, "fwd_short_kernel"),
                                          ("short", 20, "fwd_short_kernel"),
                                          ("short", 200, "NW=4"), ("auto", 200, "NW=4")])
def test_tile_switch_and_launch_log(monkeypatch, capfd, tile, Sq, want):
    pr = make_case(2, 3, Sq, 300, 64, torch.bfloat16, "BSH", "padding", 3300 + Sq)
    monkeypatch.setenv("FA_TILE", tile)
    monkeypatch.setenv("FA_LOG", "1")
    capfd.readouterr()
    o, lse = check_fwd(pr)
    err = capfd.readouterr().err
    line = [ln for ln in err.splitlines() if ln.startswith("[libfa] fa_fwd")]
    assert line and want in line[-1] and "masks=padding" in line[-1], err
    check_bwd(pr, o, lse)
    err = capfd.readouterr().err
    if Sq <= 32 and tile in ("auto", "short"):
        assert "[libfa] fa_bwd: " in err and "bwd_short_kernel" in err, err
        assert "[libfa] fa_bwd_main" not in err, err
    else:
        assert "[libfa] fa_bwd_main" in err and "[libfa] fa_bwd_post" in err, err


# ----------------------------------------------------------------------------------
# the workloads against the plain C++ fp64 oracle as well (the tests above read the
# numpy one; the two agree to 1e-11 on the CPU pins)

@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_workloads_against_cpp_oracle(cid):
    from oracle import cpp
    pr = inputs.config(cid)
    print(f"\n{pr.name} (C++ oracle)")
    o, lse = gpu_fwd(pr)
    O, L = cpp.problem_fwd(pr)
    assert_close("O", o, O, pr.dtype)
    assert_lse(lse, L)
    g = gpu_bwd(pr, o, lse)
    for name, a, r in zip(("dQ", "dK", "dV"), g, cpp.problem_bwd(pr)):
        assert_close(name, a, r, pr.dtype)
