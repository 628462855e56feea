"""q4_gemm_noalloc through the C ABI against q4_gemm (needs an MI355X).

The no-allocation entry point runs the same kernels with the library's own device
scratch in place of the caller's workspace, so its output must equal q4_gemm's bit
for bit; both stay within the product tolerance of the oracle on sampled rows. Two
calls in a row, the second with a smaller input, show that the scratch left by the
first call does not leak into the second.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, say, to_gpu, to_np

pytestmark = pytest.mark.gpu

CASES = [  # (B, N, K): channel-split GEMV, skinny GEMM with a channel split, then smaller inputs
    [(64, 8192, 28672), (4, 1024, 28672)],
    [(4, 8192, 28672), (2, 300, 4096)],
    [(16, 4096, 8192), (1, 17, 128)],
]


@pytest.fixture(scope="module")
def q4():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_decode_amd as q4mod

    say("libq4", q4mod.version())
    return q4mod


def _noalloc(lib, x, qw, y):
    import torch

    st = lib.q4_gemm_noalloc(x.data_ptr(), x.shape[0], qw.packed.data_ptr(), qw.scales.data_ptr(), qw.out_features,
                             qw.in_features, qw.group, y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.q4_last_error()


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_equals_gemm_twice(q4, case):
    import torch

    from w4a16_decode_amd import _lib

    lib = _lib.load()
    for B, N, K in CASES[case]:
        say(f"q4_gemm_noalloc B={B} N={N} K={K}")
        W = synth.weight(N, K, seed=B + N)
        x = synth.activation(B, K, seed=B + K)
        qw = q4.quantize_pack(to_gpu(W), 128)
        xg = to_gpu(x)
        y_ref = q4.gemm(xg, qw)
        y = torch.full((B, N), float("nan"), dtype=torch.float16, device=xg.device)
        _noalloc(lib, xg, qw, y)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"B={B} N={N} K={K}: q4_gemm_noalloc differs from q4_gemm"
        q_o, s_o = oracle.quantize_sym(W, 128)
        rows = np.unique(np.concatenate([np.arange(0, N, max(1, N // 64)), [N - 1]]))
        assert_close(to_np(y)[:, rows], oracle.gemm_ref_rows(x, q_o, s_o, 128, rows), f"noalloc B={B} {N}x{K}")
