"""Build liblynx.so (HIP, gfx950) in-tree: long_context_serving_amd/_lib/.

hipcc cross-compiles for gfx950 without a GPU.  Device code is compiled
without fused multiply-add contraction (the encoder's statistics are
specified as separate IEEE fp32 operations) and without packed-fp32
instructions.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "liblynx.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["lynx_tables.cpp", "lynx_api.cpp", "lynx_encode.hip",
           "lynx_attention.hip", "lynx_attention_mfma.hip", "lynx_tail.hip",
           "lynx_split.hip", "lynx_verify.hip", "lynx_scratch.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall",
          "-I", INCLUDE]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source flags.  The encoder's and the matrix-core attention's inputs are
# finite by contract; without NaN semantics their min/max need no
# canonicalising instructions (every operation and its rounding are
# unchanged; infinities keep their meaning).
EXTRA = {"lynx_encode.hip": ["-fno-honor-nans"], "lynx_attention_mfma.hip": ["-fno-honor-nans"],
         "lynx_verify.hip": ["-fno-honor-nans"]}


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    """Compile every source and link liblynx.so; returns its path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    for src in sources():
        obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
        cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip", *DEVICE]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
