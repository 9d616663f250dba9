"""Builds libdsa.so (the C-ABI library in include/dsa.h) and libdsa_ceiling.so (the streaming-read
ceiling kernel of include/stream_read.h) in-tree with hipcc for gfx950."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdsa.so")
CEILING_LIB = os.path.join(PKG, "libdsa_ceiling.so")
SOURCES = ["indexer.hip", "sfa.hip", "quant.hip", "dsa_api.cpp", "dsa_profile.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 VALU ops stay disabled: the compiler would otherwise form v_pk_*_f32 from plain
# float code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# The score kernel's MFMA accumulators are selected in VGPR form (its weighted reduction reads
# them with VALU every tile).  The attention kernel keeps its 256-register output accumulator in
# the accumulation registers, so it uses the default selection.
FILE_FLAGS = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


TIMELINE_LIB = os.path.join(PKG, "libdsa_timeline.so")


def build_timeline_library(verbose: bool = False) -> str:
    """The timeline variant of libdsa.so (-DDSA_TIMELINE: per-workgroup time stamps in the decode
    score and attention kernels, read by sparse_attention_15_amd.timeline); returns its path."""
    return build_library(verbose, ["-DDSA_TIMELINE"], out=TIMELINE_LIB, objdir_name="_build_timeline",
                         ceiling=False)


def build_library(verbose: bool = False, extra_flags=(), out: str = LIB, objdir_name: str = "_build",
                  ceiling: bool = True) -> str:
    """Compiles every source and links libdsa.so (or `out`); returns its path.  Always rebuilds."""
    objdir = os.path.join(PKG, objdir_name)
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *extra_flags, *lang, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if not ceiling:
        return out
    # the streaming-read ceiling kernel bench.py measures against, in a library of its own
    obj = os.path.join(objdir, "stream_read.hip.o")
    for cmd in ([HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, "stream_read.hip"), "-o", obj],
                [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", CEILING_LIB + ".tmp", obj]):
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"building {os.path.basename(CEILING_LIB)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(CEILING_LIB + ".tmp", CEILING_LIB)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
