"""Builds libadahop.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Objects are compiled in parallel into _build/ and linked in-tree, next to this
file, where the Python binding loads it.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
OUT = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libadahop.so")
# Measurement probe of the FP4 matrix cores' clock ceiling (bench.py
# --mfma-ceiling); not part of the AdaHOP path, built as its own library.
PROBE_SRC = "probe_mfma.hip"
PROBE_LIB = os.path.join(HERE, "libadahop_probe.so")
SOURCES = ["adahop_api.hip", "foid.hip", "iht_quant.hip", "gemm_mx.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off", "-Wall",
    # Keep the compiler from forming packed fp32 instructions (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(src, verbose):
    obj = os.path.join(OUT, src + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(SRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    pobj = _compile(PROBE_SRC, verbose)
    ptmp = PROBE_LIB + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", pobj, "-o", ptmp], check=True)
    os.replace(ptmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
