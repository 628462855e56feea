"""The launch-shape models on the device (needs an MI355X).

The host picks GEMV shapes (4 <= B <= 16) and skinny-GEMM shapes (B > 16) for
symmetric INT4 codes from linear cost models over the device's limits: its CU count,
LDS per workgroup and, for the skinny GEMM, how many workgroups of each kernel one CU
holds (asked of the runtime). The CPU tests check the host logic with MI355X's limits
stood in; these check that the limits the library reads on the device are those, so
the launches it makes are the models' picks (q4_gemm_shape reports them).
"""

import pytest

from test_tune_model import _code_coefficients as gemv_code
from test_tune_skinny import _code_coefficients as skinny_code, _model_time

from w4a16_decode_amd import tune_gemv, tune_skinny

pytestmark = pytest.mark.gpu

SHAPES = [(28672, 8192), (8192, 28672), (57344, 8192), (10240, 8192), (8192, 8192), (4096, 14336),
          (6144, 4096), (14336, 4096), (28672, 4096), (4096, 4096), (2048, 28672), (1024, 8192)]


@pytest.fixture(scope="module")
def q4():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_decode_amd as q4mod

    return q4mod


@pytest.mark.parametrize("N,K", SHAPES)
def test_skinny_picks_on_device(q4, N, K):
    code = skinny_code()
    for B in (17, 24, 32, 40, 48, 64, 80, 96, 112, 128, 144, 160, 192, 224, 256):
        got = q4.gemm_shape(B, N, K, 128)
        want = tune_skinny.pick(N, K, B, code)
        if got != want:
            tg, tw = _model_time(N, K, B, got, code), _model_time(N, K, B, want, code)
            assert abs(tg - tw) <= 1e-9 * tw, (N, K, B, got, want)


@pytest.mark.parametrize("N,K", SHAPES)
def test_gemv_picks_on_device(q4, N, K):
    code = gemv_code() + [0.0]
    for B in (4, 6, 8, 12, 16):
        got = q4.gemm_shape(B, N, K, 128)
        want = tune_gemv.pick(N, K, B, code)
        assert got[3] == 1 and want is not None
        if got[:3] != want:  # equal modelled times may be summed in another order
            tg = sum(a * b for a, b in zip(tune_gemv.features(N, K, B, *got[:3]), code))
            tw = sum(a * b for a, b in zip(tune_gemv.features(N, K, B, *want), code))
            assert abs(tg - tw) <= 1e-9 * abs(tw), (N, K, B, got, want)
