"""Build step for the synthetic workload generator: compiles synth.c into libsynth.so with gcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "libsynth.so")
    cmd = ["gcc", "-O3", "-ffp-contract=off", "-fno-fast-math", "-std=c99", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread",
           os.path.join(HERE, "synth.c"), "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
