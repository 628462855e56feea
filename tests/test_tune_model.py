"""The GEMV launch-shape model (host logic, no GPU).

The host picks the GEMV launch shape at 4 <= B <= 16 from a linear model whose
coefficients are written into csrc/q4_api.cpp (gemv_model_us). These tests refit the
coefficients from the committed MI355X measurements and check that the code's
constants are that fit, that the fit's picks are close to the fastest measured shapes,
and that the library's choice of channel splits (visible through q4_workspace_bytes)
is the model's pick for the device limits the library assumes without a GPU.
"""

import os
import re

import pytest

from w4a16_decode_amd import _lib, tune_gemv

API = os.path.join(os.path.dirname(tune_gemv.__file__), "csrc", "q4_api.cpp")


def _code_coefficients():
    src = open(API).read()
    body = src[src.index("double gemv_model_us("):]
    body = body[:body.index("\n}\n")]
    ret = body[body.index("return "):]
    red = re.search(r"KS > 1 \? ([0-9.]+) \+ ([0-9.]+) \*", body)
    nums = [float(v) for v in re.findall(r"(-?[0-9]+\.[0-9]+) \*", ret)]
    # return a * codes + b * xs + red - e * codes / (W * wgs_cu)
    a, b, e = nums[0], nums[1], re.search(r"- ([0-9.]+) \* codes / \(W", ret).group(1)
    return [a, b, float(red.group(1)), float(red.group(2)), -float(e)]


@pytest.fixture(scope="module")
def coef():
    return tune_gemv.fit(tune_gemv.load([tune_gemv.GRID]))


def test_code_constants_are_the_fit(coef):
    code = _code_coefficients()
    for c, f in zip(code, coef[:5]):
        assert abs(c - f) <= 0.006 * max(1.0, abs(f)) + 0.0006, (code, list(coef))


def test_fit_picks_near_fastest(coef):
    reg = tune_gemv.regret(tune_gemv.load([tune_gemv.GRID]), coef)
    vals = [v for _, v in reg.values()]
    assert len(vals) >= 80
    assert sum(vals) / len(vals) < 0.02
    assert max(vals) < 0.12


def test_features_hand_case():
    # 10240 x 8192 (640 tiles, 64 blocks), B = 8, R = 1, W = 16, KS = 4 on 256 CUs with
    # 160 KiB of LDS: one 16-wavefront workgroup per CU, 64 per split, 10 row blocks each,
    # 16 blocks per split: 160 KiB of codes and 8 * 16 / 4 = 32 KiB of activations
    f = tune_gemv.features(10240, 8192, 8, 1, 16, 4)
    assert f[:3] == [160.0, 32.0, 1.0]
    assert f[3] == pytest.approx(4 * 8 * 10240 * 4 / 1e6)
    assert f[4] == pytest.approx(160 / 16)


@pytest.mark.parametrize("N,K", [(10240, 8192), (8192, 8192), (8192, 28672), (57344, 8192), (4096, 4096),
                                 (6144, 4096), (28672, 4096), (4096, 14336), (2048, 28672), (1024, 8192)])
@pytest.mark.parametrize("B", [4, 6, 8, 12, 16])
def test_library_splits_follow_the_model(N, K, B):
    """Without a GPU the library sizes for 64 KiB of LDS per workgroup and 256 CUs; its
    channel splits (the workspace it asks for) must be the model's pick for those."""
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a visible GPU sets the library's limits; the GPU tests run its launches")
    lib = _lib.load()
    code = _code_coefficients() + [0.0]
    p = tune_gemv.pick(N, K, B, code, lds_limit=64 * 1024, cus=256)
    if p is None:
        pytest.skip("no candidate shape fits 64 KiB")
    ks = p[2]
    want = ks * B * N * 4 if ks > 1 else 0
    assert lib.q4_workspace_bytes(B, N, K, 128) == want, p
