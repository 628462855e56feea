"""Seeded random shapes through the whole path (needs an MI355X).

Each case draws out_features, in_features (a multiple of the group), the group, the
batch and the code kind from a fixed seed, so the launch-shape rules meet shapes no
hand-written case names (ragged row tiles, channel ranges that do not divide into
the chunks of the strided units, splits of uneven length, odd column-tile counts).
Codes and scales must match the oracle bit for bit and every output the tolerance.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, say, to_gpu, to_np

pytestmark = pytest.mark.gpu

GROUPS = (32, 64, 128, 256)
BATCHES = tuple(range(1, 21)) + (24, 31, 33, 48, 64, 65, 100, 129, 200, 256)


def _cases(n=48, seed=20261203):
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        g = int(r.choice(GROUPS))
        K = g * int(r.integers(1, max(2, 6144 // g)))
        N = int(r.integers(1, 2049))
        B = int(r.choice(BATCHES))
        asym = bool(r.integers(0, 2))
        out.append((N, K, g, B, asym))
    return out


@pytest.fixture(scope="module")
def q4():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_decode_amd as q4mod

    return q4mod


@pytest.mark.parametrize("N,K,g,B,asym", _cases())
def test_random_shape(q4, N, K, g, B, asym):
    say(f"fuzz N={N} K={K} g={g} B={B} asym={asym}")
    W = synth.weight(N, K, seed=N * 7 + K)
    x = synth.activation(B, K, seed=B * 13 + K)
    qw = q4.quantize_pack(to_gpu(W), g, asym=asym)
    if asym:
        q_o, s_o, z_o = oracle.quantize_asym(W, g)
    else:
        (q_o, s_o), z_o = oracle.quantize_sym(W, g), None
    codes, scales, zeros = q4.to_canonical(qw)
    assert np.array_equal(to_np(codes), oracle.pack_canonical(q_o))
    assert np.array_equal(to_np(scales).view(np.uint16), s_o.view(np.uint16))
    if asym:
        assert np.array_equal(to_np(zeros), z_o)
    y = to_np(q4.gemm(to_gpu(x), qw))
    w_hat = oracle.dequant_asym(q_o, s_o, z_o, g) if asym else oracle.dequant_sym(q_o, s_o, g)
    assert_close(y, oracle.gemm_ref(x, w_hat), f"N={N} K={K} g={g} B={B} asym={asym}")
