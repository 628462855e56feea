"""The oracle and the product path share no code and do not import each other."""

import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sources(sub, exts):
    for dp, _, fs in os.walk(os.path.join(ROOT, sub)):
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(dp, f)


def test_oracle_imports_only_numpy():
    code = ("import sys; sys.path.insert(0, %r); import oracle; "
            "bad = [m for m in sys.modules if m.split('.')[0] in ('torch', 'w4a16_decode_amd')]; "
            "print(','.join(bad))" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True).stdout.strip()
    assert out == "", out


def test_oracle_does_not_reference_product():
    for p in _sources("oracle", (".py", ".c", ".h")):
        src = open(p, encoding="utf-8").read()
        assert not re.search(r"^\s*(from|import)\s+(w4a16_decode_amd|torch|ctypes)\b", src, re.M), p
        assert "libq4" not in src and "CDLL" not in src, p


def test_product_does_not_reference_oracle():
    pat = re.compile(r"^\s*(from|import)\s+oracle\b|['\"]oracle['\"]|oracle/", re.M)
    for p in _sources("w4a16_decode_amd", (".py", ".hip", ".cpp", ".h")):
        src = open(p, encoding="utf-8").read()
        assert not pat.search(src), p
    for p in _sources("include", (".h",)):
        assert "oracle" not in open(p, encoding="utf-8").read().lower(), p


def test_synth_holds_no_method_arithmetic():
    src = open(os.path.join(ROOT, "synth", "__init__.py"), encoding="utf-8").read()
    for word in ("rint", "clip(", "amax", "/ 7", "/7", "pack", "quantiz"):
        assert word not in src, word
