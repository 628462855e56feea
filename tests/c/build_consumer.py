"""Build tests/c/q4_consumer (a plain C99 program against include/q4.h and libq4.so).

    python tests/c/build_consumer.py

gcc compiles it as C (no hipcc, no C++); it links the in-tree libq4.so and the
HIP runtime, with an rpath to both so it runs from the repository root.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "q4_consumer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    libdir = os.path.join(ROOT, "w4a16_decode_amd")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "q4_consumer.c"), "-o", BIN,
           "-L", libdir, "-lq4", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode:
        raise RuntimeError("building q4_consumer failed:\n" + " ".join(cmd) + "\n" + p.stdout + p.stderr)
    return BIN


if __name__ == "__main__":
    print(build())
    sys.exit(0)
