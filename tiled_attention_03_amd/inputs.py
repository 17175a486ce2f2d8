"""Seeded synthetic inputs for the fused attention operator.

This module only draws numbers and builds the mask/bias *inputs* that a
caller hands to the operator (index arrays, validity flags, ALiBi slopes).
It holds none of the attention arithmetic, so both the HIP path and the
CPU oracle can consume exactly the same bytes.

Recipes follow the workloads on the source pages:

* tiny fp32 self-attention (parity only);
* causal self-attention, BNSD, bf16 (the causal-mask style of the CogVLM
  guide, "technical implementation details - attention mask");
* multimodal joint attention: 64 text slots then 576 image patches
  (the ops-transformer multimodal FlashAttention page, "Layer 1: modality
  projection" puts text tokens first with modality id 0, image id 1),
  text attends to all, image attends to image only, text slots past the
  per-sample text length are padding;
* late-interaction cross attention in BSH layout with key padding (the
  retrieval page, "Layer 2: semantic modelling", masks invalid document
  tokens with -inf);
* long-sequence causal attention with ALiBi (FlashAttentionScore guide,
  section 3.2: pse supports ALiBi).

Every tensor is drawn from a CPU ``torch.Generator`` seeded with
``1000 * config_id + tensor_id`` (tensor ids: q 0, k 1, v 2, dO 3,
lengths 4), N(0,1) in float32 and rounded to nearest-even into the
storage dtype.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3, "len": 4}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def randn(shape, dtype, seed: int) -> torch.Tensor:
    """N(0,1) drawn in float32 from ``seed``, then rounded to ``dtype``."""
    x = torch.randn(tuple(shape), generator=_gen(seed), dtype=torch.float32)
    return x.to(dtype).contiguous()


def randint(lo: int, hi: int, n: int, seed: int) -> torch.Tensor:
    """``n`` integers uniform in the inclusive range [lo, hi]."""
    return torch.randint(lo, hi + 1, (n,), generator=_gen(seed), dtype=torch.int64)


def alibi_slopes(num_heads: int) -> torch.Tensor:
    """ALiBi slopes 2^(-8 i / H) for i = 1..H (head h, 0-based, gets i = h+1),
    stored as float32; both sides read these same float32 values."""
    h = torch.arange(1, num_heads + 1, dtype=torch.float64)
    return torch.pow(2.0, -8.0 * h / num_heads).to(torch.float32)


@dataclass
class Problem:
    """One attention call: tensors on the CPU plus the mask/bias description.

    Layout "BNSD": q [B,H,Sq,D], k/v [B,H,Sk,D].
    Layout "BSH":  q [B,Sq,H*D], k/v [B,Sk,H*D]; head h owns columns
    [h*D, (h+1)*D).
    """
    name: str
    batch: int
    heads: int
    seq_q: int
    seq_k: int
    head_dim: int
    layout: str
    dtype: torch.dtype
    scale: float
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: Optional[torch.Tensor] = None
    causal: bool = False
    explicit_mask: Optional[torch.Tensor] = None      # bool, broadcastable to [B,H,Sq,Sk]
    q_modality: Optional[torch.Tensor] = None         # int8 [B,Sq]
    k_modality: Optional[torch.Tensor] = None         # int8 [B,Sk]
    modality_allow: Optional[torch.Tensor] = None     # bool [M,M], row = query modality
    modality_allow_diag: bool = False
    key_valid: Optional[torch.Tensor] = None          # bool [B,Sk]
    alibi_slopes: Optional[torch.Tensor] = None       # float32 [H]
    pse: Optional[torch.Tensor] = None                # float32, broadcastable to [B,H,Sq,Sk]
    keep_prob: float = 1.0                            # < 1: dropout after the softmax
    dropout_seed: int = 0                             # Philox key of the dropout mask
    grad_f32: bool = False                            # backward writes float32 gradients
    meta: dict = field(default_factory=dict)


def make_qkv(B, H, Sq, Sk, D, layout, dtype, seed_base, with_do=True):
    if layout == "BNSD":
        qs, ks = (B, H, Sq, D), (B, H, Sk, D)
    elif layout == "BSH":
        qs, ks = (B, Sq, H * D), (B, Sk, H * D)
    else:
        raise ValueError(layout)
    q = randn(qs, dtype, seed_base + TENSOR_IDS["q"])
    k = randn(ks, dtype, seed_base + TENSOR_IDS["k"])
    v = randn(ks, dtype, seed_base + TENSOR_IDS["v"])
    do = randn(qs, dtype, seed_base + TENSOR_IDS["do"]) if with_do else None
    return q, k, v, do


def config(cid: int, with_do: bool = True) -> Problem:
    """The five workloads, by id 1..5, at their full sizes."""
    base = 1000 * cid
    if cid == 1:
        B, H, S, D = 1, 2, 128, 64
        q, k, v, do = make_qkv(B, H, S, S, D, "BNSD", torch.float32, base, with_do)
        return Problem("tiny_fp32_b1h2s128d64", B, H, S, S, D, "BNSD", torch.float32,
                       1.0 / math.sqrt(D), q, k, v, do)
    if cid == 2:
        B, H, S, D = 4, 16, 1024, 64
        q, k, v, do = make_qkv(B, H, S, S, D, "BNSD", torch.bfloat16, base, with_do)
        return Problem("causal_bf16_b4h16s1024d64", B, H, S, S, D, "BNSD", torch.bfloat16,
                       1.0 / 8.0, q, k, v, do, causal=True)
    if cid == 3:
        B, H, D, T, I = 8, 12, 64, 64, 576
        S = T + I
        q, k, v, do = make_qkv(B, H, S, S, D, "BNSD", torch.bfloat16, base, with_do)
        text_len = randint(16, 64, B, base + TENSOR_IDS["len"])
        mod = torch.zeros(B, S, dtype=torch.int8)
        mod[:, T:] = 1
        pos = torch.arange(S)
        valid = ~((pos[None, :] < T) & (pos[None, :] >= text_len[:, None]))
        allow = torch.tensor([[True, True], [False, True]])
        return Problem("multimodal_bf16_b8h12s640d64", B, H, S, S, D, "BNSD", torch.bfloat16,
                       1.0 / math.sqrt(D), q, k, v, do,
                       q_modality=mod.clone(), k_modality=mod.clone(), modality_allow=allow,
                       key_valid=valid, meta={"text_len": text_len})
    if cid == 4:
        B, H, Lq, Lk, D = 256, 12, 32, 512, 64
        q, k, v, do = make_qkv(B, H, Lq, Lk, D, "BSH", torch.bfloat16, base, with_do)
        doc_len = randint(128, 512, B, base + TENSOR_IDS["len"])
        valid = torch.arange(Lk)[None, :] < doc_len[:, None]
        return Problem("late_interaction_bf16_bsh_b256h12lq32lk512d64", B, H, Lq, Lk, D, "BSH",
                       torch.bfloat16, 1.0 / math.sqrt(D), q, k, v, do, key_valid=valid,
                       meta={"doc_len": doc_len})
    if cid == 5:
        B, H, S, D = 1, 32, 8192, 128
        q, k, v, do = make_qkv(B, H, S, S, D, "BNSD", torch.bfloat16, base, with_do)
        return Problem("long_causal_alibi_bf16_b1h32s8192d128", B, H, S, S, D, "BNSD",
                       torch.bfloat16, 1.0 / math.sqrt(D), q, k, v, do, causal=True,
                       alibi_slopes=alibi_slopes(H))
    raise ValueError(f"unknown config {cid}")


@dataclass
class MaxSimCase:
    """Operands of one MaxSim call: q [B, L_q, D], d [B, L_d, D] on the CPU."""
    name: str
    q: torch.Tensor
    d: torch.Tensor
    q_valid: Optional[torch.Tensor] = None     # bool [B, L_q]
    d_valid: Optional[torch.Tensor] = None     # bool [B, L_d]


def maxsim_workload() -> MaxSimCase:
    """The late-interaction workload's own tensors as MaxSim operands: its
    query and document embeddings (width 768) and its document padding."""
    pr = config(4, with_do=False)
    return MaxSimCase("maxsim_bf16_b256lq32ld512d768", pr.q, pr.k, None, pr.key_valid)


def maxsim_case(B, Lq, Ld, D, dtype, seed, q_mask=None, d_mask=None) -> MaxSimCase:
    """N(0,1) embeddings; masks: None, "pad" (valid prefix of random length) or
    "holes" (each token valid with probability 0.8)."""
    q = randn((B, Lq, D), dtype, seed)
    d = randn((B, Ld, D), dtype, seed + 1)
    g = _gen(seed + 2)

    def mask(kind, L):
        if kind is None:
            return None
        if kind == "pad":
            lens = torch.randint(0, L + 1, (B,), generator=g)
            return torch.arange(L)[None, :] < lens[:, None]
        if kind == "holes":
            return torch.rand(B, L, generator=g) < 0.8
        raise ValueError(kind)

    return MaxSimCase(f"maxsim_b{B}lq{Lq}ld{Ld}d{D}", q, d, mask(q_mask, Lq), mask(d_mask, Ld))


def fp8_quantize(x: torch.Tensor):
    """Per-tensor e4m3 quantization of a real tensor: descale = amax / 448 and
    x8 = round-to-nearest-even(x / descale) as torch.float8_e4m3fn.  The real
    input the fp8 path stands for is then x8 * descale (not x)."""
    xf = x.float()
    amax = float(xf.abs().max()) if xf.numel() else 0.0
    descale = amax / 448.0 if amax > 0 else 1.0
    return (xf / descale).to(torch.float8_e4m3fn).contiguous(), descale
