"""Builds libpab.so (HIP kernels + C ABI) for gfx950 in the package directory,
and libpab_probe.so, the matrix-instruction probe that tests use
(include/pab_probe.h).

    python -m precision_attention_block_amd.build

Every HIP source is compiled with the packed-FP32 target feature disabled
(`-Xclang -target-feature -Xclang -packed-fp32-ops`): the host pass warns that
it does not know the feature, which is harmless.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpab.so")
SOURCES = ["api.cpp", "quant.hip", "attention.hip", "attention_bwd.hip"]
PROBE_LIB = os.path.join(PKG, "libpab_probe.so")
PROBE_SOURCES = ["probe_mfma.hip"]
# The attention kernel's inputs are finite by contract (scores, exponentials
# and maxima never see NaN), so its fmax needs no NaN-quieting of operands.
EXTRA = {"attention.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpab)")


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def build(verbose=False, out=LIB):
    """Builds libpab.so (at `out`) and libpab_probe.so."""
    _build_lib(SOURCES, out, verbose)
    _build_lib(PROBE_SOURCES, PROBE_LIB, verbose)
    return out


def _build_lib(sources, out, verbose):
    hipcc = _hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        extra = EXTRA.get(src, [])
        cmd = [hipcc] + flags() + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stderr or "").splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), msg))
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(sources)) as ex:
        objs = list(ex.map(compile_one, sources))
    tmp = out + ".tmp"
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
