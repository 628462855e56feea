"""Build libq4.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m w4a16_decode_amd.build        # or __graft_entry__.build()

Each source is compiled by hipcc in parallel, then linked into
w4a16_decode_amd/libq4.so next to this file. The library links the
libamdhip64.so.7 soname; when torch is imported first, the dynamic loader
binds it to the HIP runtime torch already loaded, so streams and device
pointers from torch are valid in the library (one runtime per process).
"""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libq4.so")
SOURCES = ["q4_api.cpp", "q4_quant.hip", "q4_gemm.hip", "q4_kv.hip", "q4_probe.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_*_f32 (float2 arithmetic is issued as scalar VALU ops).
# The float32 divide stays IEEE correctly rounded (no fast-math flags anywhere).
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def code_only(src: str) -> str:
    """C++ source without comments and with all whitespace runs collapsed (string and
    character literals kept as they are)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(extra_flags=()) -> str:
    """Hash of everything the library is built from: the compile flags, the code of
    the sources and headers under csrc/ and of the public headers under include/
    (comments and layout ignored). The build bakes it into q4_version(); the loader
    compares it with the tree it runs from, so a library left over from other
    sources is never used."""
    flags = " ".join(COMMON + list(extra_flags)).replace(ROOT, ".")  # the same wherever the tree is
    h = hashlib.sha256(flags.encode())
    inc = os.path.join(ROOT, "include")
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))] + \
        [os.path.join(inc, f) for f in sorted(os.listdir(inc))]
    for path in files:
        if path.endswith((".cpp", ".hip", ".h")):
            h.update(os.path.basename(path).encode())
            with open(path, encoding="utf-8") as f:
                h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libq4)")


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("command failed:\n  " + " ".join(cmd) + "\n" + p.stdout + p.stderr)
    return p


def build(verbose: bool = False, extra_flags=None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    extra = list(extra_flags or [])
    flags = COMMON + extra + [f'-DQ4_SOURCE_HASH="{source_hash(extra)}"']
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.rsplit(".", 1)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        for p, cmd in zip(ex.map(_run, cmds), cmds):
            if verbose:
                print(" ".join(cmd))
                print(p.stderr, end="")
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
