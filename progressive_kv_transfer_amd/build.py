"""Build liblynx.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m progressive_kv_transfer_amd.build

Device translation units are compiled with -ffp-contract=off (one rounding
per operation, the arithmetic contract of the codec), packed FP32 disabled,
and IEEE mode off with -fno-honor-nans (inputs are finite by contract, so
min/max need no NaN canonicalisation).  The host API keeps full NaN
semantics for argument validation.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblynx.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-ffp-contract=off", "-fno-honor-nans",
          "-Xarch_device", "-mno-amdgpu-ieee", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops"]
HOST = ["-ffp-contract=off", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include"]

DEVICE_SOURCES = ["lynx_quant.hip", "lynx_dequant.hip", "lynx_attn.hip", "lynx_verify.hip"]
HOST_SOURCES = ["lynx_api.cpp"]


def sources():
    return [os.path.join(CSRC, s) for s in DEVICE_SOURCES + HOST_SOURCES]


def build(verbose: bool = False, isa_dir: str | None = None) -> str:
    """Compile every source and link liblynx.so; returns its path.

    With ``isa_dir`` the gfx950 assembly of each device source is also
    written there (for instruction counts)."""
    tmp = tempfile.mkdtemp(prefix="lynx_build_")
    if isa_dir:
        isa_dir = os.path.abspath(isa_dir)
    try:
        objs = []
        for src in DEVICE_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            _run([HIPCC, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj],
                 verbose, cwd=tmp)
            objs.append(obj)
            if isa_dir:
                os.makedirs(isa_dir, exist_ok=True)
                _run([HIPCC, *COMMON, *DEVICE, "--cuda-device-only", "-S",
                      os.path.join(CSRC, src), "-o",
                      os.path.join(isa_dir, src.replace(".hip", ".s"))], verbose, cwd=tmp)
        for src in HOST_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            _run([HIPCC, *COMMON, *HOST, "-x", "c++", "-c", os.path.join(CSRC, src),
                  "-o", obj], verbose, cwd=tmp)
            objs.append(obj)
        out = LIB + ".tmp%d" % os.getpid()
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out, *objs],
             verbose, cwd=tmp)
        os.replace(out, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


PROBE_SRC = os.path.join(CSRC, "stream_ceiling.hip")
PROBE = os.path.join(PKG, "stream_ceiling")


def build_stream_probe(verbose: bool = False) -> str:
    """Compile the stand-alone streaming-ceiling probe (run by
    `bench.py --hbm-probe`; not part of the library)."""
    out = PROBE + ".tmp%d" % os.getpid()
    _run([HIPCC, "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops", PROBE_SRC, "-o", out], verbose, cwd=PKG)
    os.replace(out, PROBE)
    return PROBE


def _run(cmd, verbose, cwd):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, cwd=cwd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "--hip-link" not in l)
    if p.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + out)
    if verbose and out.strip():
        print(out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv,
                isa_dir=(sys.argv[sys.argv.index("--isa") + 1]
                         if "--isa" in sys.argv else None)))
    print(build_stream_probe(verbose="-v" in sys.argv))
