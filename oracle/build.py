"""Build step for the C oracle (test infrastructure): gcc, -O2, no intrinsics, no fast-math."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "qvref.c")
OUT = os.path.join(_HERE, "libqvref.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def build_oracle(force: bool = True, extra_flags=None, out: str | None = None) -> str:
    """Compile the oracle; ``extra_flags`` lets a test build a variant into another file."""
    out = out or OUT
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
        return out
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *(extra_flags or []), SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle())
