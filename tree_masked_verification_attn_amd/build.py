"""Compile libtav.so (the HIP kernels + C ABI) for gfx950 with hipcc.

Every source is compiled to an object in parallel, then linked into
``tree_masked_verification_attn_amd/libtav.so`` next to this file.  Packed
fp32 VALU instructions are disabled for all device code.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtav.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-variable", "-Wno-unused-function",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    return obj, r.returncode, " ".join(cmd), msgs


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libtav.so; raise on any failure."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    objs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for obj, rc, cmd, msgs in ex.map(_compile, srcs):
            if rc != 0:
                raise RuntimeError(f"hipcc failed:\n{cmd}\n{msgs}")
            if verbose and msgs:
                print(msgs, file=sys.stderr)
            objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    _build_probe()
    return LIB


PROBE_SRC = os.path.join(CSRC, "probe", "roofline_probe.hip")
PROBE_LIB = os.path.join(PKG, "libtavprobe.so")


def _build_probe():
    """The measurement library of the benchmark (a streaming-read and a matrix-core kernel)."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, PROBE_LIB)


if __name__ == "__main__":
    print(build(verbose=True))
