"""libfa: fused tiled attention for AMD MI355X (gfx950).

``binding`` holds the ctypes interface of the HIP library (fwd, bwd, Plan);
``inputs`` the seeded synthetic workloads.  The binding is loaded on first
use so that the input recipes import on machines without the library.
"""
import importlib

__all__ = ["binding", "inputs", "fwd", "bwd", "Plan"]

_BINDING_NAMES = ("fwd", "bwd", "Plan", "make_problem", "workspace_size", "FaError")


def __getattr__(name):
    if name in ("binding", "inputs"):
        return importlib.import_module(f"{__name__}.{name}")
    if name in _BINDING_NAMES:
        return getattr(importlib.import_module(f"{__name__}.binding"), name)
    raise AttributeError(name)
