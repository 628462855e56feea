"""The skinny-GEMM launch-shape model (host logic, no GPU).

For B > 16 and symmetric INT4 codes the host picks the skinny GEMM's launch shape
from a linear model whose coefficients are written into csrc/q4_api.cpp
(skinny_model_us). These tests refit the coefficients from the committed MI355X
measurements and check that the code's constants are that fit, that the fit's picks
are close to the fastest measured shapes and faster than the fixed rules they
replaced, and -- through the host front end built with stand-ins for the device (256
CUs, 160 KiB of LDS, MI355X's per-CU residency of each kernel) -- that the library's
pick is the model's.
"""

import os
import re
import shutil
import subprocess

import pytest

from w4a16_decode_amd import tune_skinny

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
API = os.path.join(ROOT, "w4a16_decode_amd", "csrc", "q4_api.cpp")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _code_coefficients():
    src = open(API).read()
    body = src[src.index("double skinny_model_us("):]
    body = body[:body.index("\n}\n")]
    red = re.search(r"KS > 1 \? ([0-9.]+) \+ ([0-9.]+) \*", body)
    ret = body[body.index("return "):]
    a = re.search(r"return ([0-9.]+) \* codes \+", ret).group(1)
    b = re.search(r"\+ ([0-9.]+) \* codes \* CT", ret).group(1)
    c = re.search(r"\+ ([0-9.]+) \* staged", ret).group(1)
    f = re.search(r"\+ ([0-9.]+) \* codes / \(8 \* conc\)", ret).group(1)
    g = re.search(r"\+\s*([0-9.]+);", ret).group(1)
    return [float(a), float(b), float(c), float(red.group(1)), float(red.group(2)), float(f), float(g)]


@pytest.fixture(scope="module")
def rows():
    return tune_skinny.load([tune_skinny.GRID])


@pytest.fixture(scope="module")
def coef(rows):
    return tune_skinny.fit(rows)


def test_code_constants_are_the_fit(coef):
    code = _code_coefficients()
    for c, f in zip(code, coef):
        assert abs(c - f) <= 0.002 * max(1.0, abs(f)) + 0.0002, (code, list(coef))


def test_fit_picks_near_fastest(rows, coef):
    reg = tune_skinny.regret(rows, coef)
    best = [v[1] for v in reg.values()]
    old = [v[2] for v in reg.values() if v[2] is not None]
    assert len(best) >= 140 and len(old) == len(best)
    assert sum(best) / len(best) < 0.01
    assert max(best) < 0.12
    # against the fixed rules the model replaced, measured in the same grid
    assert sum(old) / len(old) < -0.05
    assert max(old) < 0.05


def test_features_hand_case():
    # 28672 x 8192 (1792 row tiles, 64 blocks), B = 96, R = 2, KS = 2, CT = 6 on 256 CUs:
    # 112 row workgroups x 1 column group x 2 splits = 224 workgroups, one per CU, each
    # 8 wavefronts x 2 tiles x 32 blocks = 512 KiB of codes, 6 x 32 staged tile-blocks;
    # partials 2 x 96 x 28672 x 4 bytes
    f = tune_skinny.features(28672, 8192, 96, 2, 2, 6, per_cu=1)
    assert f[:5] == [512.0, 3072.0, 192.0, 1.0, pytest.approx(2 * 96 * 28672 * 4 / 1e6)]
    assert f[5] == pytest.approx(512 / 8)
    # candidates never leave two 16-row tiles of one group empty
    assert {ct for _, _, ct in tune_skinny.candidates(33)} == {2, 3, 4}
    assert {ct for _, _, ct in tune_skinny.candidates(96)} == {2, 3, 4, 6}


@pytest.fixture(scope="module")
def shape_tool(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    exe = tmp_path_factory.mktemp("shapes") / "host_shapes"
    cmd = ["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), API, os.path.join(ROOT, "tests", "c", "host_sanitize.cpp"),
           "-o", str(exe)]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stdout + p.stderr
    return exe


def _library_shapes(exe, cases):
    inp = "".join(f"{B} {N} {K} 128\n" for B, N, K in cases)
    r = subprocess.run([str(exe), "shapes"], input=inp, capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    return [tuple(map(int, line.split())) for line in r.stdout.split("\n") if line.strip()]


def _model_time(N, K, B, shape, coef):
    R, _, KS, CT = shape
    return sum(a * b for a, b in zip(tune_skinny.features(N, K, B, R, KS, CT, tune_skinny.per_cu_mi355x(R, CT)), coef))


def test_library_picks_follow_the_model(rows, shape_tool):
    """The host front end, with MI355X's limits stood in, picks the model's shape for
    every matrix and batch size of the grid and for other 70B / 8B shapes."""
    code = _code_coefficients()
    cases = sorted({(r["B"], r["N"], r["K"]) for r in rows})
    cases += [(B, N, K) for B in (20, 33, 70, 100, 130, 200, 250)
              for N, K in ((8192, 8192), (14336, 4096), (2048, 28672), (1024, 8192), (300, 1280))]
    got = _library_shapes(shape_tool, cases)
    assert len(got) == len(cases)
    for (B, N, K), lib in zip(cases, got):
        want = tune_skinny.pick(N, K, B, code)
        assert want is not None
        if lib != want:  # equal modelled times may be summed in another order
            tl, tw = _model_time(N, K, B, lib, code), _model_time(N, K, B, want, code)
            assert abs(tl - tw) <= 1e-9 * tw, (B, N, K, lib, want, tl, tw)


def test_gemv_batches_keep_one_column_tile(shape_tool):
    got = _library_shapes(shape_tool, [(B, 8192, 28672) for B in (1, 2, 3, 4, 8, 16)])
    assert all(s[3] == 1 for s in got), got
