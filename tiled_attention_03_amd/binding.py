"""ctypes binding of libfa (include/fa.h).  Argument marshalling only.

Every step of the attention runs in the HIP library; this module checks
tensor shapes, builds the ``fa_problem`` struct, passes device pointers and
torch's current HIP stream, and allocates outputs/workspace with torch (the
device-memory plumbing).  If ``libfa.so`` is missing it raises at import.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_WORKSPACE = 0, -1, -2, -3, -4
FA_F32, FA_F16, FA_BF16, FA_FP8_E4M3 = 0, 1, 2, 3
FA_BNSD, FA_BSH = 0, 1
FA_MASK_NONE, FA_MASK_CAUSAL, FA_MASK_EXPLICIT, FA_MASK_MODALITY, FA_MASK_PADDING = 0, 1, 2, 4, 8
FA_PSE_NONE, FA_PSE_ALIBI, FA_PSE_DENSE = 0, 1, 2

ENTRY_POINTS = ("fa_fwd", "fa_bwd_workspace_size", "fa_bwd", "fa_bwd_noalloc", "fa_bwd_prep",
                "fa_bwd_main", "fa_bwd_post", "fa_fwd_fp8_workspace_size", "fa_fwd_fp8", "fa_maxsim",
                "fa_status_str", "fa_abi_version")

_DTYPES = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16,
           torch.float8_e4m3fn: FA_FP8_E4M3}
_LAYOUTS = {"BNSD": FA_BNSD, "BSH": FA_BSH}


class FaProblem(ctypes.Structure):
    """Mirror of ``fa_problem`` in include/fa.h (same field order and types)."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("head_num", ctypes.c_int32),
        ("seq_q", ctypes.c_int32),
        ("seq_k", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("keep_prob", ctypes.c_float),
        ("mask_flags", ctypes.c_uint32),
        ("num_modalities", ctypes.c_int32),
        ("modality_allow_diag", ctypes.c_int32),
        ("modality_allow", ctypes.c_uint8 * 64),
        ("pse_kind", ctypes.c_int32),
        ("pse_dtype", ctypes.c_int32),
        ("explicit_mask", ctypes.c_void_p),
        ("em_stride_b", ctypes.c_int64),
        ("em_stride_h", ctypes.c_int64),
        ("em_stride_q", ctypes.c_int64),
        ("q_modality", ctypes.c_void_p),
        ("k_modality", ctypes.c_void_p),
        ("key_valid", ctypes.c_void_p),
        ("alibi_slopes", ctypes.c_void_p),
        ("pse", ctypes.c_void_p),
        ("pse_stride_b", ctypes.c_int64),
        ("pse_stride_h", ctypes.c_int64),
        ("pse_stride_q", ctypes.c_int64),
        ("dropout_seed", ctypes.c_uint64),
        ("grad_f32", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("dpse", ctypes.c_void_p),
    ]


class FaMaxsimProblem(ctypes.Structure):
    """Mirror of ``fa_maxsim_problem`` in include/fa.h."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("len_q", ctypes.c_int32),
        ("len_d", ctypes.c_int32),
        ("dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("pad0", ctypes.c_int32),
        ("q_valid", ctypes.c_void_p),
        ("d_valid", ctypes.c_void_p),
    ]


class FaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} ({status})")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"libfa.so not found at {_LIB_PATH}; build it first "
            "(python -m tiled_attention_03_amd.build)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER(FaProblem)
    sig = {
        "fa_fwd": [P, vp, vp, vp, vp, vp, vp],
        "fa_bwd_workspace_size": [P, ctypes.POINTER(sz)],
        "fa_bwd": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "fa_bwd_noalloc": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "fa_bwd_prep": [P, vp, vp, vp, sz, vp],
        "fa_bwd_main": [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "fa_bwd_post": [P, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "fa_maxsim": [ctypes.POINTER(FaMaxsimProblem), vp, vp, vp, vp, vp],
        "fa_fwd_fp8_workspace_size": [P, ctypes.POINTER(sz)],
        "fa_fwd_fp8": [P, vp, vp, vp, ctypes.c_float, ctypes.c_float, ctypes.c_float, vp, vp, vp,
                       sz, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.fa_status_str.argtypes = [ctypes.c_int]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = ctypes.c_int
    return lib


lib = _load()


def status_str(status: int) -> str:
    return lib.fa_status_str(int(status)).decode()


def abi_version() -> int:
    return lib.fa_abi_version()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_problem(q: torch.Tensor, k: torch.Tensor, *, heads: int, layout: str = "BNSD",
                 scale: Optional[float] = None, keep_prob: float = 1.0, causal: bool = False,
                 explicit_mask: Optional[torch.Tensor] = None,
                 q_modality: Optional[torch.Tensor] = None,
                 k_modality: Optional[torch.Tensor] = None,
                 modality_allow: Optional[torch.Tensor] = None,
                 modality_allow_diag: bool = False,
                 key_valid: Optional[torch.Tensor] = None,
                 alibi_slopes: Optional[torch.Tensor] = None,
                 pse: Optional[torch.Tensor] = None, dropout_seed: int = 0,
                 grad_f32: bool = False, dpse: Optional[torch.Tensor] = None):
    """Build an ``FaProblem`` from tensors (shape checks only).  Returns the
    struct and the list of tensors whose memory it references."""
    if layout not in _LAYOUTS:
        raise ValueError(f"layout must be BNSD or BSH, got {layout}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype:
        raise TypeError("q and k must share one of float32/float16/bfloat16")
    if layout == "BNSD":
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("BNSD tensors are [B, H, S, D]")
        B, H, Sq, D = q.shape
        Sk = k.shape[2]
        if H != heads or tuple(k.shape) != (B, H, Sk, D):
            raise ValueError("k must be [B, H, S_k, D] with q's B, H, D")
    else:
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError("BSH tensors are [B, S, H*D]")
        B, Sq, HD = q.shape
        Sk = k.shape[1]
        if HD % heads:
            raise ValueError("hidden size is not a multiple of head_num")
        H, D = heads, HD // heads
        if tuple(k.shape) != (B, Sk, HD):
            raise ValueError("k must be [B, S_k, H*D] with q's B and hidden size")
    if scale is None:
        raise TypeError("scale is required (the operator has no default; 1/sqrt(D) is usual)")
    if k.device != q.device:
        raise ValueError("q and k must be on one device")
    p = FaProblem()
    p.batch, p.head_num, p.seq_q, p.seq_k, p.head_dim = B, H, Sq, Sk, D
    p.layout = _LAYOUTS[layout]
    p.dtype = _DTYPES[q.dtype]
    p.scale = float(scale)
    p.keep_prob = float(keep_prob)
    p.dropout_seed = int(dropout_seed) & 0xFFFFFFFFFFFFFFFF
    p.grad_f32 = int(bool(grad_f32))

    def on_dev(t, what):
        if t is not None and t.device != q.device:
            raise ValueError(f"{what} must be on q's device ({q.device}), not {t.device}")

    for t, what in ((explicit_mask, "explicit_mask"), (q_modality, "q_modality"),
                    (k_modality, "k_modality"), (key_valid, "key_valid"),
                    (alibi_slopes, "alibi_slopes"), (pse, "pse"), (dpse, "dpse")):
        on_dev(t, what)
    if dpse is not None:
        if dpse.dtype != torch.float32 or tuple(dpse.shape) != (B, H, Sq, Sk) or \
                not dpse.is_contiguous():
            raise ValueError("dpse must be a contiguous float32 [B, H, S_q, S_k]")
        p.dpse = dpse.data_ptr()
    keep = []
    flags = 0
    if causal:
        flags |= FA_MASK_CAUSAL
    if explicit_mask is not None:
        em = explicit_mask
        if em.dtype not in (torch.bool, torch.uint8):
            raise TypeError("explicit_mask must be bool or uint8")
        em = em.view(torch.uint8) if em.dtype == torch.bool else em
        while em.dim() < 4:
            em = em.unsqueeze(0)
        if em.shape[-2:] != (Sq, Sk) or em.stride(-1) != 1:
            raise ValueError("explicit_mask must end in a contiguous [S_q, S_k]")
        if em.shape[0] not in (1, B) or em.shape[1] not in (1, H):
            raise ValueError("explicit_mask must be [B|1, H|1, S_q, S_k]")
        flags |= FA_MASK_EXPLICIT
        p.explicit_mask = em.data_ptr()
        p.em_stride_b = em.stride(0) if em.shape[0] > 1 else 0
        p.em_stride_h = em.stride(1) if em.shape[1] > 1 else 0
        p.em_stride_q = em.stride(2)
        keep.append(em)
    if (q_modality is None) != (k_modality is None) or \
            (q_modality is not None and modality_allow is None):
        raise ValueError("a modality mask needs q_modality, k_modality and modality_allow")
    if q_modality is not None:
        qm = q_modality.to(torch.int8).contiguous()
        km = k_modality.to(torch.int8).contiguous()
        allow = torch.as_tensor(modality_allow, dtype=torch.bool).cpu()
        M = allow.shape[0]
        if allow.shape != (M, M) or not 1 <= M <= 8:
            raise ValueError("modality_allow must be [M, M] with M <= 8")
        if tuple(qm.shape) != (B, Sq) or tuple(km.shape) != (B, Sk):
            raise ValueError("modality ids must be [B, S_q] and [B, S_k]")
        flags |= FA_MASK_MODALITY
        p.num_modalities = M
        p.modality_allow_diag = int(bool(modality_allow_diag))
        for a in range(M):
            for c in range(M):
                p.modality_allow[a * M + c] = int(allow[a, c])
        p.q_modality, p.k_modality = qm.data_ptr(), km.data_ptr()
        keep += [qm, km]
    if key_valid is not None:
        kv = _as_bytes(key_valid)
        if tuple(kv.shape) != (B, Sk):
            raise ValueError("key_valid must be [B, S_k]")
        flags |= FA_MASK_PADDING
        p.key_valid = kv.data_ptr()
        keep.append(kv)
    p.mask_flags = flags
    if alibi_slopes is not None and pse is not None:
        raise ValueError("give either alibi_slopes or a dense pse")
    if alibi_slopes is not None:
        sl = alibi_slopes.to(torch.float32).contiguous()
        if sl.numel() != H:
            raise ValueError("alibi_slopes must hold H values")
        p.pse_kind = FA_PSE_ALIBI
        p.alibi_slopes = sl.data_ptr()
        keep.append(sl)
    elif pse is not None:
        ps = pse
        while ps.dim() < 4:
            ps = ps.unsqueeze(0)
        if ps.dtype not in _DTYPES or ps.shape[-2:] != (Sq, Sk) or ps.stride(-1) != 1:
            raise ValueError("pse must be float and end in a contiguous [S_q, S_k]")
        p.pse_kind = FA_PSE_DENSE
        p.pse_dtype = _DTYPES[ps.dtype]
        p.pse = ps.data_ptr()
        p.pse_stride_b = ps.stride(0) if ps.shape[0] > 1 else 0
        p.pse_stride_h = ps.stride(1) if ps.shape[1] > 1 else 0
        p.pse_stride_q = ps.stride(2)
        keep.append(ps)
    return p, keep


def _as_bytes(m: torch.Tensor) -> torch.Tensor:
    """A mask as contiguous uint8 (0/1): bool storage is reinterpreted, not copied."""
    m = m.contiguous()
    if m.dtype == torch.bool:
        return m.view(torch.uint8)
    return m if m.dtype == torch.uint8 else (m != 0).view(torch.uint8)


def _check(status: int, what: str):
    if status != FA_OK:
        raise FaError(status, what)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _lse_shape(p: FaProblem):
    return (p.batch, p.head_num, p.seq_q)


def _same(t, like, dtype, device, what):
    """``t`` must have ``like``'s shape, ``dtype`` and ``device``."""
    if tuple(t.shape) != tuple(like.shape) or t.dtype != dtype or t.device != device:
        raise ValueError(f"{what} must be {dtype} of shape {tuple(like.shape)} on {device}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")


def _lse_ok(lse, p: FaProblem, device):
    if lse.dtype != torch.float32 or tuple(lse.shape) != _lse_shape(p) or lse.device != device:
        raise ValueError(f"lse must be float32 of shape {_lse_shape(p)} on {device}")


def fwd(q, k, v, *, heads: int, layout: str = "BNSD", out=None, lse=None, **kw):
    """O, LSE = attention(q, k, v).  ``kw`` are the mask/bias arguments of
    :func:`make_problem`.  Returns (O in q's layout and dtype, LSE float32 [B,H,S_q])."""
    _contig(q, k, v, out, lse)
    p, keep = make_problem(q, k, heads=heads, layout=layout, **kw)
    _same(v, k, q.dtype, q.device, "v")
    o = torch.empty_like(q) if out is None else out
    l = torch.empty(_lse_shape(p), dtype=torch.float32, device=q.device) if lse is None else lse
    _same(o, q, q.dtype, q.device, "out")
    _lse_ok(l, p, q.device)
    _check(lib.fa_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), _stream()),
           "fa_fwd")
    return o, l


def fwd_fp8(q, k, v, q_descale: float, k_descale: float, v_descale: float, *, heads: int,
            layout: str = "BNSD", workspace=None, **kw):
    """Forward with float8_e4m3fn inputs (real value = element * descale):
    returns (O bf16 in q's layout, LSE float32 [B,H,S_q])."""
    _contig(q, k, v)
    p, keep = make_problem(q, k, heads=heads, layout=layout, **kw)
    _same(v, k, q.dtype, q.device, "v")
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    l = torch.empty(_lse_shape(p), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = ctypes.c_size_t(0)
        _check(lib.fa_fwd_fp8_workspace_size(ctypes.byref(p), ctypes.byref(n)),
               "fa_fwd_fp8_workspace_size")
        workspace = torch.empty(max(n.value, 256), dtype=torch.uint8, device=q.device)
    _check(lib.fa_fwd_fp8(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), float(q_descale),
                          float(k_descale), float(v_descale), _ptr(o), _ptr(l), _ptr(workspace),
                          workspace.numel(), _stream()), "fa_fwd_fp8")
    return o, l


def workspace_size(q, k, *, heads: int, layout: str = "BNSD", **kw) -> int:
    p, _ = make_problem(q, k, heads=heads, layout=layout, **kw)
    n = ctypes.c_size_t(0)
    _check(lib.fa_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)), "fa_bwd_workspace_size")
    return n.value


def bwd(q, k, v, o, lse, do, *, heads: int, layout: str = "BNSD", workspace=None,
        want_dpse: bool = False, dpse: Optional[torch.Tensor] = None, **kw):
    """dQ, dK, dV of L = sum(O * dO), recomputing P from ``lse``.  With
    ``grad_f32=True`` they are float32.  With ``want_dpse`` (or a ``dpse``
    buffer, float32 [B, H, S_q, S_k]) the bias gradient is written and
    returned as a fourth value."""
    _contig(q, k, v, o, lse, do)
    _same(v, k, q.dtype, q.device, "v")
    _same(o, q, q.dtype, q.device, "o")
    _same(do, q, q.dtype, q.device, "do")
    if want_dpse and dpse is None:
        B = q.shape[0]
        Sq, Sk = (q.shape[2], k.shape[2]) if layout == "BNSD" else (q.shape[1], k.shape[1])
        dpse = torch.empty(B, heads, Sq, Sk, dtype=torch.float32, device=q.device)
    p, keep = make_problem(q, k, heads=heads, layout=layout, dpse=dpse, **kw)
    _lse_ok(lse, p, q.device)
    n = ctypes.c_size_t(0)
    _check(lib.fa_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)), "fa_bwd_workspace_size")
    if workspace is not None and (workspace.device != q.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws = workspace if workspace is not None else torch.empty(max(n.value, 256), dtype=torch.uint8,
                                                             device=q.device)
    gdt = torch.float32 if p.grad_f32 else q.dtype
    dq, dk, dv = (torch.empty(t.shape, dtype=gdt, device=t.device) for t in (q, k, v))
    _check(lib.fa_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel() * ws.element_size(), _stream()), "fa_bwd")
    return (dq, dk, dv) if dpse is None else (dq, dk, dv, dpse)


def bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, *, heads: int, layout: str = "BNSD", **kw):
    """fa_bwd_noalloc: the backward into the caller's dq, dk, dv without a
    workspace (the library's static device scratch holds the row terms); the
    binding allocates nothing either."""
    _contig(q, k, v, o, lse, do, dq, dk, dv)
    _same(v, k, q.dtype, q.device, "v")
    _same(o, q, q.dtype, q.device, "o")
    _same(do, q, q.dtype, q.device, "do")
    p, keep = make_problem(q, k, heads=heads, layout=layout, **kw)
    _lse_ok(lse, p, q.device)
    gdt = torch.float32 if p.grad_f32 and q.dtype != torch.float32 else q.dtype
    for t, like, what in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _same(t, like, gdt, q.device, what)
    _check(lib.fa_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _stream()), "fa_bwd_noalloc")
    return dq, dk, dv


class Plan:
    """A prepared problem: the struct is built once and the device calls (fwd;
    the whole backward; or its steps: bwd prep = row terms, bwd main = dK/dV,
    bwd post = dQ) can be issued repeatedly, e.g. by a benchmark that brackets
    each call with events."""

    def __init__(self, q, k, *, heads: int, layout: str = "BNSD", **kw):
        self.p, self._keep = make_problem(q, k, heads=heads, layout=layout, **kw)
        n = ctypes.c_size_t(0)
        _check(lib.fa_bwd_workspace_size(ctypes.byref(self.p), ctypes.byref(n)), "workspace")
        self.ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=q.device)
        self._pp = ctypes.byref(self.p)

    def fwd(self, q, k, v, o, lse):
        _check(lib.fa_fwd(self._pp, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream()),
               "fa_fwd")

    def bwd(self, q, k, v, o, lse, do, dq, dk, dv):
        _check(lib.fa_bwd(self._pp, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(self.ws), self.ws.numel(), _stream()),
               "fa_bwd")

    def bwd_prep(self, o, do):
        _check(lib.fa_bwd_prep(self._pp, _ptr(o), _ptr(do), _ptr(self.ws), self.ws.numel(),
                               _stream()), "fa_bwd_prep")

    def bwd_main(self, q, k, v, lse, do, dk, dv):
        _check(lib.fa_bwd_main(self._pp, _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(do), _ptr(dk),
                               _ptr(dv), _ptr(self.ws), self.ws.numel(), _stream()), "fa_bwd_main")

    def bwd_post(self, q, k, v, lse, do, dq):
        _check(lib.fa_bwd_post(self._pp, _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(do), _ptr(dq),
                               _ptr(self.ws), self.ws.numel(), _stream()), "fa_bwd_post")


def problem_kwargs(pr, device) -> dict:
    """Mask/bias keyword arguments of a ``inputs.Problem`` moved to ``device``."""
    mv = lambda t: None if t is None else t.to(device)
    return dict(scale=pr.scale, causal=pr.causal, explicit_mask=mv(pr.explicit_mask),
                q_modality=mv(pr.q_modality), k_modality=mv(pr.k_modality),
                modality_allow=pr.modality_allow, modality_allow_diag=pr.modality_allow_diag,
                key_valid=mv(pr.key_valid), alibi_slopes=mv(pr.alibi_slopes), pse=mv(pr.pse),
                keep_prob=pr.keep_prob, dropout_seed=pr.dropout_seed, grad_f32=pr.grad_f32)


def maxsim_problem(q: torch.Tensor, d: torch.Tensor, q_valid: Optional[torch.Tensor] = None,
                   d_valid: Optional[torch.Tensor] = None):
    """Build an ``FaMaxsimProblem`` (shape checks only) and the tensors it references."""
    if q.dim() != 3 or d.dim() != 3 or q.shape[0] != d.shape[0] or q.shape[2] != d.shape[2]:
        raise ValueError("q must be [B, L_q, D] and d [B, L_d, D]")
    if q.dtype not in _DTYPES or d.dtype != q.dtype:
        raise TypeError("q and d must share one dtype")
    B, Lq, D = q.shape
    Ld = d.shape[1]
    p = FaMaxsimProblem()
    p.batch, p.len_q, p.len_d, p.dim, p.dtype = B, Lq, Ld, D, _DTYPES[q.dtype]
    keep = []
    for name, m, L in (("q_valid", q_valid, Lq), ("d_valid", d_valid, Ld)):
        if m is None:
            continue
        mm = _as_bytes(m)
        if tuple(mm.shape) != (B, L):
            raise ValueError(f"{name} must be [B, {L}]")
        setattr(p, name, mm.data_ptr())
        keep.append(mm)
    return p, keep


def maxsim(q, d, *, q_valid=None, d_valid=None, rowmax=None, score=None):
    """MaxSim late interaction: (rowmax float32 [B, L_q], score float32 [B])."""
    _contig(q, d)
    p, keep = maxsim_problem(q, d, q_valid, d_valid)
    B, Lq = q.shape[0], q.shape[1]
    rm = torch.empty(B, Lq, dtype=torch.float32, device=q.device) if rowmax is None else rowmax
    sc = torch.empty(B, dtype=torch.float32, device=q.device) if score is None else score
    _check(lib.fa_maxsim(ctypes.byref(p), _ptr(q), _ptr(d), _ptr(rm), _ptr(sc), _stream()),
           "fa_maxsim")
    return rm, sc
