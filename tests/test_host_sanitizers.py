"""The C ABI's host code under the address and undefined-behaviour
sanitizers (no GPU needed).

api.cpp is rebuilt with both sanitizers on its host pass (the device code of
the library is unchanged and comes from the regular build's objects) and
linked into tests/host_sanitize_driver.cpp, which runs the sliding-tile
planner, the step and key-tile helpers and the size helpers on valid and
hostile sizes with exact-size output arrays, and every validation path of the
device entry points with arguments that must be rejected before the first HIP
call.  Any sanitizer report aborts that program; the test also requires its
own checks to pass.
"""
import os
import subprocess

import pytest

from precision_attention_block_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = "/opt/rocm/llvm/bin/clang++"
KERNEL_OBJECTS = ["quant.o", "attention.o", "attention_bwd.o"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, msg


def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not available")
    objdir = os.path.join(B.PKG, "_build")
    objs = [os.path.join(objdir, o) for o in KERNEL_OBJECTS]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined"]
    api_o = str(tmp_path / "api_san.o")
    rc, msg = _run([hipcc] + B.flags() + ["-O1", "-g"] + host_san +
                   ["-x", "hip", "-c", os.path.join(B.CSRC, "api.cpp"), "-o", api_o])
    assert rc == 0, msg
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    drv_o = str(tmp_path / "driver.o")
    rc, msg = _run([CLANG, "-O1", "-g", "-std=c++17"] + san +
                   ["-I" + os.path.join(B.ROOT, "include"), "-c",
                    os.path.join(HERE, "host_sanitize_driver.cpp"), "-o", drv_o])
    assert rc == 0, msg
    exe = str(tmp_path / "driver")
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))), "lib")
    rc, msg = _run([CLANG] + san + [drv_o, api_o] + objs +
                   ["-L" + rocm_lib, "-lamdhip64", "-Wl,-rpath," + rocm_lib, "-o", exe])
    assert rc == 0, msg
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    rc, msg = _run([exe], env=env)
    assert rc == 0 and "checks passed" in msg, msg
    assert "runtime error" not in msg and "AddressSanitizer" not in msg, msg
