"""Build libbitopt.so (gfx950) in-tree with hipcc.

Every translation unit under csrc/ is compiled to an object in parallel, then
linked into bit_optimizers_block_amd/libbitopt.so.

Flags that fix the arithmetic: -ffp-contract=off (no FMA contraction: each fp32
operation is rounded on its own), -fhip-fp32-correctly-rounded-divide-sqrt
(IEEE division and square root), and packed-fp32 instructions disabled.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
GEN = os.path.join(BUILD, "gen")
LIB = os.path.join(PKG, "libbitopt.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}", f"-I{GEN}",
]

SOURCES = ["bitopt_api.cpp", "codec.hip", "step_adam.hip", "step_ademamix.hip",
           "step_momentum.hip", "step_lion.hip", "step_rmsprop.hip", "step_adagrad.hip", "tensorwise.hip"]


def _compile(src: str, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def generate_tables() -> str:
    """Compile and run the host generator of the standard maps' search tables."""
    os.makedirs(GEN, exist_ok=True)
    exe = os.path.join(BUILD, "gen_tables")
    cmd = ["g++", "-O2", "-std=c++17", f"-I{CSRC}", os.path.join(CSRC, "gen_tables.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    out = os.path.join(GEN, "bitopt_tables.h")
    subprocess.run([exe, out], check=True)
    return out


def build(jobs: int = 8, extra=()) -> str:
    """Generate the search tables, compile every HIP source and link libbitopt.so;
    returns its path."""
    generate_tables()
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(jobs=int(os.environ.get("MAX_JOBS", "8")), extra=sys.argv[1:]))
