"""The C ABI's host code (validation, sizes, dispatch up to the launch) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

fa_api.hip is compiled again with both sanitizers on its host side only (the
device side is unchanged) and linked with the library's other objects; the
driver ``host_abi_check.c`` calls every entry point with edge-value and seeded
random problems and null tensor pointers, so that no call reaches a launch.
A sanitizer report aborts the driver; the driver itself fails on a status or
size that breaks the contract in fa.h."""
import os
import subprocess

import pytest

from tiled_attention_03_amd import build as b

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run([str(c) for c in cmd], capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r


def test_abi_host_code_under_sanitizers(tmp_path):
    objs = [os.path.join(b.OBJDIR, os.path.splitext(s)[0] + ".o") for s in b.SOURCES
            if s != "fa_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built (build() first)")
    if not os.path.exists(CLANG):
        pytest.skip("no clang with sanitizer runtimes")
    # host-side sanitizers only: each flag goes to the host compilation
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    api_o = tmp_path / "fa_api_san.o"
    _run([b.HIPCC, *b.FLAGS, *host_san, "-c", os.path.join(b.CSRC, "fa_api.hip"), "-o", api_o],
         timeout=600)
    lib = tmp_path / "libfa_san.so"
    _run([b.HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", api_o, *objs, "-o", lib],
         timeout=600)
    exe = tmp_path / "host_abi_check"
    _run([CLANG, *SAN, "-O1", "-g", "-D__HIP_PLATFORM_AMD__", f"-I{b.INCLUDE}",
          "-I/opt/rocm/include", os.path.join(HERE, "host_abi_check.c"), f"-L{tmp_path}",
          "-lfa_san", f"-Wl,-rpath,{tmp_path}", "-o", exe], timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe), "100000"], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr[-4000:]
