"""Build step for the CPU oracle (test infrastructure): compiles svt_oracle.c with gcc."""
import os
import subprocess
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))


def build(out: Optional[str] = None, mutant: int = 0, verbose: bool = False) -> str:
    """Compile the oracle into ``out`` (default oracle/liboracle.so).  ``mutant`` > 0 plants the
    numbered deliberate mistake (used only by the planted-mistake test, into a temporary path)."""
    out = out or os.path.join(HERE, "liboracle.so")
    cmd = ["gcc", "-O2", "-std=c99", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread",
           f"-DORACLE_MUTANT={int(mutant)}", os.path.join(HERE, "svt_oracle.c"), "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
