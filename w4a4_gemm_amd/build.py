"""Build the NVFP4 HIP library in-tree: ``w4a4_gemm_amd/libnvfp4.so`` (gfx950 only).

Every source is compiled with hipcc for ``--offload-arch=gfx950`` and linked
into one shared library that exports the C ABI of ``include/nvfp4.h``.

Flags:
* ``-Xclang -target-feature -Xclang -packed-fp32-ops`` -- no packed fp32
  instructions are generated (the host pass warns that it does not know the
  feature; that warning is harmless).
* ``-fno-gpu-flush-denormals-to-zero`` -- fp32 subnormals are kept, which the
  exact rounding in the kernels relies on.

Usage:  python w4a4_gemm_amd/build.py  [-v]

Run it as a script (or load it by path): importing the package loads the
library and checks its symbols, which fails while the library is stale.
"""

import importlib.util
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnvfp4.so")
SOURCES = ["capi.cpp", "quant.hip", "kv.hip", "kv_attn.hip", "gemm.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # NewGVN: the classic GVN pass takes minutes on the unrolled GEMM main loop
    "-mllvm", "-enable-newgvn=true",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


# Flags of single sources.  kv_attn.hip: the attention's logits and weights are
# finite, and without NaNs to honour the compiler takes a float max in one
# instruction instead of first canonicalizing both operands.
SOURCE_FLAGS = {"kv_attn.hip": ["-fno-honor-nans"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (p.stderr or "").splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err)


def _source_hash():
    spec = importlib.util.spec_from_file_location("nvfp4_srchash", os.path.join(HERE, "srchash.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.source_hash()


def build(verbose: bool = False) -> str:
    """Compile every source and link libnvfp4.so; returns the library path.
    The library carries the hash of the sources it was built from
    (nvfp4_source_hash), which the binding checks when it loads."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    tag = [f"-DNVFP4_SOURCE_HASH=\"{_source_hash()}\""]
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        extra = (tag if src == "capi.cpp" else []) + SOURCE_FLAGS.get(src, [])
        cmds.append([HIPCC, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
