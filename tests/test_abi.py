"""Host-only checks of the C ABI: the library loads, exports every entry
point include/fa.h declares, its struct layout matches the ctypes mirror,
and argument validation returns the documented codes before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

from tiled_attention_03_amd import binding as fa  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(fa.ENTRY_POINTS)
    lib = ctypes.CDLL(fa._LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fa._LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (fa_[a-z_0-9]+)$", out, flags=re.M))
    assert set(names) <= exported


def test_abi_version_and_status_strings():
    assert fa.abi_version() == 6
    assert fa.status_str(0) == "ok"
    assert fa.status_str(-2) == "unsupported configuration"


@pytest.mark.parametrize("cls,cname", [(fa.FaProblem, "fa_problem"),
                                       (fa.FaMaxsimProblem, "fa_maxsim_problem")])
def test_struct_layout_matches_c(tmp_path, cls, cname):
    fields = [f[0] for f in cls._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof({cname}, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "fa.h"\nint main(void){\n'
                   + body + f'\n  printf("sizeof %zu\\n", sizeof({cname}));\n  return 0;\n}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", "-I/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    got = dict(line.split() for line in out.strip().splitlines())
    for f in fields:
        assert int(got[f]) == getattr(cls, f).offset, f
    assert int(got["sizeof"]) == ctypes.sizeof(cls)


def base_problem(**over):
    p = fa.FaProblem()
    p.batch, p.head_num, p.seq_q, p.seq_k, p.head_dim = 2, 4, 64, 64, 64
    p.layout, p.dtype = fa.FA_BNSD, fa.FA_BF16
    p.scale, p.keep_prob = 0.125, 1.0
    for k, v in over.items():
        setattr(p, k, v)
    return p


FAKE = ctypes.c_void_p(1 << 20)     # aligned, never dereferenced: validation fails first


def call_fwd(p, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE):
    return fa.lib.fa_fwd(ctypes.byref(p), q, k, v, o, lse, None)


@pytest.mark.parametrize("over,code", [
    ({"keep_prob": 0.9, "dtype": fa.FA_F32}, fa.FA_ERR_UNSUPPORTED),
    ({"keep_prob": 0.0}, fa.FA_ERR_INVALID_ARG),
    ({"keep_prob": -0.5}, fa.FA_ERR_INVALID_ARG),
    ({"keep_prob": 1.5}, fa.FA_ERR_INVALID_ARG),
    ({"keep_prob": float("nan")}, fa.FA_ERR_INVALID_ARG),
    ({"head_dim": 48}, fa.FA_ERR_UNSUPPORTED),
    ({"head_dim": 256}, fa.FA_ERR_UNSUPPORTED),
    ({"dtype": fa.FA_F32, "head_dim": 96}, fa.FA_ERR_UNSUPPORTED),
    ({"batch": -1}, fa.FA_ERR_INVALID_ARG),
    ({"seq_k": -3}, fa.FA_ERR_INVALID_ARG),
    ({"head_dim": 0}, fa.FA_ERR_INVALID_ARG),
    ({"layout": 7}, fa.FA_ERR_INVALID_ARG),
    ({"dtype": 9}, fa.FA_ERR_INVALID_ARG),
    ({"mask_flags": 16}, fa.FA_ERR_INVALID_ARG),
    ({"mask_flags": fa.FA_MASK_EXPLICIT}, fa.FA_ERR_INVALID_ARG),
    ({"mask_flags": fa.FA_MASK_PADDING}, fa.FA_ERR_INVALID_ARG),
    ({"mask_flags": fa.FA_MASK_MODALITY, "q_modality": 1 << 20, "k_modality": 1 << 20,
      "num_modalities": 9}, fa.FA_ERR_INVALID_ARG),
    ({"mask_flags": fa.FA_MASK_MODALITY, "num_modalities": 2}, fa.FA_ERR_INVALID_ARG),
    ({"pse_kind": fa.FA_PSE_ALIBI}, fa.FA_ERR_INVALID_ARG),
    ({"pse_kind": fa.FA_PSE_DENSE}, fa.FA_ERR_INVALID_ARG),
    ({"pse_kind": 5}, fa.FA_ERR_INVALID_ARG),
    ({"scale": float("nan")}, fa.FA_ERR_INVALID_ARG),
    ({"scale": -0.125}, fa.FA_ERR_UNSUPPORTED),
    ({"reserved0": 1}, fa.FA_ERR_INVALID_ARG),
    ({"dpse": 1 << 20}, fa.FA_ERR_INVALID_ARG),                       # no dense pse
    ({"dpse": (1 << 20) + 4, "pse_kind": fa.FA_PSE_DENSE, "pse": 1 << 20}, fa.FA_ERR_INVALID_ARG),
    ({"dpse": 1 << 20, "pse_kind": fa.FA_PSE_DENSE, "pse": 1 << 20, "dtype": fa.FA_F32},
     fa.FA_ERR_UNSUPPORTED),
])
def test_validation_codes(over, code):
    assert call_fwd(base_problem(**over)) == code


def test_null_and_misaligned_tensors_are_rejected():
    p = base_problem()
    assert call_fwd(p, q=None) == fa.FA_ERR_INVALID_ARG
    assert call_fwd(p, v=None) == fa.FA_ERR_INVALID_ARG
    assert call_fwd(p, lse=None) == fa.FA_ERR_INVALID_ARG
    assert call_fwd(p, k=ctypes.c_void_p((1 << 20) + 2)) == fa.FA_ERR_INVALID_ARG
    assert fa.lib.fa_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == fa.FA_ERR_INVALID_ARG


def test_empty_problems_are_no_ops():
    for over in ({"batch": 0}, {"head_num": 0}, {"seq_q": 0}):
        assert call_fwd(base_problem(**over), q=None, k=None, v=None, o=None, lse=None) == 0


def test_workspace_size_and_checks():
    p = base_problem(batch=3, head_num=5, seq_q=77, head_dim=128)
    n = ctypes.c_size_t(0)
    assert fa.lib.fa_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    r256 = lambda x: (x + 255) // 256 * 256
    assert n.value == r256(3 * 5 * 77 * 4)
    assert fa.lib.fa_bwd_workspace_size(ctypes.byref(p), None) == fa.FA_ERR_INVALID_ARG
    # too small a workspace is refused before any launch
    st = fa.lib.fa_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                       FAKE, n.value - 1, None)
    assert st == fa.FA_ERR_WORKSPACE
    st = fa.lib.fa_bwd_post(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert st == fa.FA_ERR_WORKSPACE
    st = fa.lib.fa_bwd_prep(ctypes.byref(base_problem(keep_prob=0.5, dtype=fa.FA_F32)), FAKE, FAKE,
                            FAKE, 1 << 30, None)
    assert st == fa.FA_ERR_UNSUPPORTED
    st = fa.lib.fa_bwd_prep(ctypes.byref(base_problem(keep_prob=0.0)), FAKE, FAKE, FAKE, 1 << 30,
                            None)
    assert st == fa.FA_ERR_INVALID_ARG


def maxsim_problem(**over):
    p = fa.FaMaxsimProblem()
    p.batch, p.len_q, p.len_d, p.dim, p.dtype = 4, 32, 256, 768, fa.FA_BF16
    for k, v in over.items():
        setattr(p, k, v)
    return p


def call_maxsim(p, q=FAKE, d=FAKE, rowmax=FAKE, score=FAKE):
    return fa.lib.fa_maxsim(ctypes.byref(p), q, d, rowmax, score, None)


@pytest.mark.parametrize("over,code", [
    ({"dtype": fa.FA_F32}, fa.FA_ERR_UNSUPPORTED),
    ({"dim": 64}, fa.FA_ERR_UNSUPPORTED),
    ({"dim": 768 + 64}, fa.FA_ERR_UNSUPPORTED),
    ({"dim": 1152}, fa.FA_ERR_UNSUPPORTED),
    ({"len_d": 16385}, fa.FA_ERR_UNSUPPORTED),
    ({"batch": -1}, fa.FA_ERR_INVALID_ARG),
    ({"len_q": -1}, fa.FA_ERR_INVALID_ARG),
    ({"len_d": -1}, fa.FA_ERR_INVALID_ARG),
    ({"dim": 0}, fa.FA_ERR_INVALID_ARG),
    ({"dtype": 7}, fa.FA_ERR_INVALID_ARG),
    ({"pad0": 1}, fa.FA_ERR_INVALID_ARG),
])
def test_maxsim_validation_codes(over, code):
    assert call_maxsim(maxsim_problem(**over)) == code


def test_maxsim_pointer_checks():
    p = maxsim_problem()
    assert call_maxsim(p, q=None) == fa.FA_ERR_INVALID_ARG
    assert call_maxsim(p, d=None) == fa.FA_ERR_INVALID_ARG
    assert call_maxsim(p, rowmax=None) == fa.FA_ERR_INVALID_ARG
    assert call_maxsim(p, score=None) == fa.FA_ERR_INVALID_ARG
    assert call_maxsim(p, d=ctypes.c_void_p((1 << 20) + 8)) == fa.FA_ERR_INVALID_ARG
    assert call_maxsim(p, score=ctypes.c_void_p((1 << 20) + 2)) == fa.FA_ERR_INVALID_ARG
    assert fa.lib.fa_maxsim(None, FAKE, FAKE, FAKE, FAKE, None) == fa.FA_ERR_INVALID_ARG
    # B == 0 is a no-op that needs no pointers
    assert call_maxsim(maxsim_problem(batch=0), q=None, d=None, rowmax=None, score=None) == 0


def call_fwd_fp8(p, ws=FAKE, ws_bytes=1 << 30, scales=(1.0, 1.0, 1.0)):
    return fa.lib.fa_fwd_fp8(ctypes.byref(p), FAKE, FAKE, FAKE, *scales, FAKE, FAKE, ws, ws_bytes,
                             None)


def test_fp8_entry_points_validate():
    p8 = base_problem(dtype=fa.FA_FP8_E4M3, head_dim=128)
    # the 16-bit entry points refuse fp8 problems, and the fp8 one refuses the others
    assert call_fwd(p8) == fa.FA_ERR_UNSUPPORTED
    n = ctypes.c_size_t(0)
    assert fa.lib.fa_bwd_workspace_size(ctypes.byref(p8), ctypes.byref(n)) == fa.FA_ERR_UNSUPPORTED
    assert call_fwd_fp8(base_problem()) == fa.FA_ERR_INVALID_ARG
    # workspace: V^T per 64-key tile, B * H * ceil(S_k / 64) * D * 64 bytes
    assert fa.lib.fa_fwd_fp8_workspace_size(ctypes.byref(p8), ctypes.byref(n)) == 0
    assert n.value == 2 * 4 * 1 * 128 * 64
    assert call_fwd_fp8(p8, ws_bytes=n.value - 1) == fa.FA_ERR_WORKSPACE
    assert call_fwd_fp8(p8, ws=None, ws_bytes=n.value) == fa.FA_ERR_INVALID_ARG
    assert call_fwd_fp8(p8, scales=(1.0, float("inf"), 1.0)) == fa.FA_ERR_INVALID_ARG
    assert call_fwd_fp8(p8, scales=(-1.0, 1.0, 1.0)) == fa.FA_ERR_INVALID_ARG
    assert call_fwd_fp8(p8, scales=(1.0, 1.0, 0.0)) == fa.FA_ERR_INVALID_ARG
    assert call_fwd_fp8(base_problem(dtype=fa.FA_FP8_E4M3, keep_prob=0.9)) == fa.FA_ERR_UNSUPPORTED
    assert call_fwd_fp8(base_problem(dtype=fa.FA_FP8_E4M3, head_dim=96)) == fa.FA_ERR_UNSUPPORTED
    # empty problems need nothing
    assert fa.lib.fa_fwd_fp8(ctypes.byref(base_problem(dtype=fa.FA_FP8_E4M3, batch=0)), None, None,
                             None, 1.0, 1.0, 1.0, None, None, None, 0, None) == 0


# ----------------------------------------------------------------------------------
# the Python binding's checks: each raises before any pointer reaches the library

def _t(*shape, dtype=None, device="cpu"):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.bfloat16, device=device)


def test_binding_requires_an_explicit_scale():
    q, k = _t(1, 2, 8, 64), _t(1, 2, 8, 64)
    with pytest.raises(TypeError, match="scale"):
        fa.make_problem(q, k, heads=2)
    p, _ = fa.make_problem(q, k, heads=2, scale=0.25)
    assert abs(p.scale - 0.25) < 1e-12


@pytest.mark.parametrize("field", ["key_valid", "alibi_slopes", "explicit_mask", "pse",
                                   "q_modality"])
def test_binding_rejects_masks_on_another_device(field):
    import torch
    q, k = _t(1, 2, 8, 64), _t(1, 2, 8, 64)
    kw = {"key_valid": dict(key_valid=_t(1, 8, dtype=torch.bool, device="meta")),
          "alibi_slopes": dict(alibi_slopes=_t(2, dtype=torch.float32, device="meta")),
          "explicit_mask": dict(explicit_mask=_t(1, 1, 8, 8, dtype=torch.bool, device="meta")),
          "pse": dict(pse=_t(1, 2, 8, 8, dtype=torch.float32, device="meta")),
          "q_modality": dict(q_modality=_t(1, 8, dtype=torch.int8, device="meta"),
                             k_modality=_t(1, 8, dtype=torch.int8, device="meta"),
                             modality_allow=[[1, 1], [0, 1]])}[field]
    with pytest.raises(ValueError, match="device"):
        fa.make_problem(q, k, heads=2, scale=0.125, **kw)


def test_binding_rejects_partial_modality_arguments():
    import torch
    q, k = _t(1, 2, 8, 64), _t(1, 2, 8, 64)
    with pytest.raises(ValueError, match="modality"):
        fa.make_problem(q, k, heads=2, scale=0.125, q_modality=_t(1, 8, dtype=torch.int8))


@pytest.mark.parametrize("bad", ["v_shape", "o_dtype", "do_shape", "lse_dtype", "lse_shape"])
def test_binding_backward_checks_shapes_and_dtypes(bad):
    import torch
    B, H, S, D = 1, 2, 8, 64
    q, k, v, o, do = (_t(B, H, S, D) for _ in range(5))
    lse = _t(B, H, S, dtype=torch.float32)
    if bad == "v_shape":
        v = _t(B, H, S + 1, D)
    elif bad == "o_dtype":
        o = _t(B, H, S, D, dtype=torch.float16)
    elif bad == "do_shape":
        do = _t(B, H, S - 1, D)
    elif bad == "lse_dtype":
        lse = _t(B, H, S, dtype=torch.bfloat16)
    else:
        lse = _t(B, H, S + 2, dtype=torch.float32)
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o, lse, do, heads=H, scale=0.125)


@pytest.mark.parametrize("bad", ["v_dtype", "out_shape", "lse_shape"])
def test_binding_forward_checks_outputs(bad):
    import torch
    B, H, S, D = 1, 2, 8, 64
    q, k, v = _t(B, H, S, D), _t(B, H, S, D), _t(B, H, S, D)
    kw = {}
    if bad == "v_dtype":
        v = _t(B, H, S, D, dtype=torch.float16)
    elif bad == "out_shape":
        kw["out"] = _t(B, H, S - 1, D)
    else:
        kw["lse"] = _t(B, H, S, 1, dtype=torch.float32)
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, heads=H, scale=0.125, **kw)


def test_long_key_ranges_are_accepted():
    """The forward walks key tiles in chunks, so S_k past the size of one chunk's
    tile list (256 tiles of 64 keys) is a supported problem: validation passes and
    the call goes on to the pointer checks."""
    p = base_problem(seq_k=70000, mask_flags=fa.FA_MASK_PADDING)
    assert call_fwd(p) == fa.FA_ERR_INVALID_ARG           # key_valid missing: pointer check
    p.key_valid = 1 << 20
    assert call_fwd(p, q=None) == fa.FA_ERR_INVALID_ARG   # reached the tensor checks


def test_noalloc_backward_rejects_problems_past_its_scratch():
    """fa_bwd_noalloc keeps the row terms (4 bytes per query row of every head) in
    a fixed 16 MiB device array: a larger problem is refused before any launch."""
    def call(p):
        return fa.lib.fa_bwd_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, None)
    assert call(base_problem(batch=1, head_num=64, seq_q=70000, seq_k=64)) == fa.FA_ERR_WORKSPACE
    assert call(base_problem(keep_prob=0.0)) == fa.FA_ERR_INVALID_ARG
    assert call(base_problem(dtype=fa.FA_FP8_E4M3)) == fa.FA_ERR_UNSUPPORTED
    p = base_problem()
    assert fa.lib.fa_bwd_noalloc(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, None) == fa.FA_ERR_INVALID_ARG
    assert call(base_problem(batch=0)) == 0
