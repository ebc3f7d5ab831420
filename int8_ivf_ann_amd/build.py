"""Build step for the gfx950 search library: compiles csrc/ with hipcc into libsvt.so (in-tree)."""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsvt.so")
ARCH = "gfx950"
# packed-fp32 instructions are kept out of every kernel (the host pass warns that it does not know
# the feature; that warning is harmless)
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# (source, holds device code); svt_api.cpp is host-only
SOURCES = (("svt_kernels.hip", True), ("svt_tile.hip", True), ("svt_noalloc.hip", True), ("svt_rerank.hip", True),
           ("svt_largek.hip", True), ("svt_api.cpp", False))
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    with tempfile.TemporaryDirectory(prefix="svt_build_") as td:
        objs = []
        for src, dev in SOURCES:
            obj = os.path.join(td, src + ".o")
            cmd = [hipcc] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
            if dev:
                cmd += ["--offload-arch=" + ARCH] + DEVICE_FLAGS
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            objs.append(obj)
        cmd = [hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", LIB + ".tmp", "-lpthread"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
