"""Act-order (g_idx) HIP path vs the oracle, through the C ABI (needs an MI355X).

The library stores act-order weights with their channels permuted group by group
(perm from q4_actorder_perm) and gathers x through perm inside the product. Codes
and scales must equal the oracle's act-order RTN bit for bit (column i of the
stored matrix is channel perm[i]); products must meet the output tolerance against
the oracle's float64 product with the per-channel scale gather.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, say, to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_decode_amd as q4mod

    say("libq4", q4mod.version())
    return q4mod


def _check_actorder_exact(q4, W, g, h, rows=None):
    q_o, s_o, gi = oracle.quantize_sym_actorder(W if rows is None else W[rows], g, h)
    perm = q4.actorder_perm(gi, g)
    aw = q4.quantize_pack_perm(to_gpu(W), g, to_gpu(perm))
    codes, scales, _ = q4.to_canonical(aw.qw)
    c = to_np(codes) if rows is None else to_np(codes)[rows]
    sc = to_np(scales) if rows is None else to_np(scales)[rows]
    assert np.array_equal(oracle.unpack_canonical(c), q_o[:, perm]), (W.shape, g, "codes")
    assert np.array_equal(sc.view(np.uint16), s_o.view(np.uint16)), (W.shape, g, "scales")
    if rows is None:
        assert np.array_equal(to_np(aw.qw.packed), oracle.codes_to_device(q_o[:, perm])), "device codes"
    return aw, q_o, s_o, gi


SHAPES = [(17, 256, 32), (40, 384, 128), (100, 1280, 64), (64, 2048, 512), (33, 768, 256), (129, 640, 128)]


@pytest.mark.parametrize("N,K,g", SHAPES)
def test_actorder_quantize_bit_exact(q4, N, K, g):
    say(f"act-order quantize N={N} K={K} g={g}")
    W = synth.weight(N, K, seed=N + K)
    _check_actorder_exact(q4, W, g, synth.channel_energy(K, seed=N))


def test_actorder_identity_is_rtn(q4):
    """Equal channel energies: perm is the identity and the codes are plain RTN's."""
    W = synth.weight(48, 1024, seed=3)
    aw, q_o, s_o, gi = _check_actorder_exact(q4, W, 128, np.ones(1024))
    assert np.array_equal(gi, np.arange(1024) // 128)
    qw = q4.quantize_pack(to_gpu(W), 128)
    assert np.array_equal(to_np(qw.packed), to_np(aw.qw.packed))


@pytest.mark.parametrize("B", [1, 3, 8, 16, 17, 40, 100])
@pytest.mark.parametrize("N,K,g", [(100, 1280, 64), (300, 2048, 128), (33, 768, 256)])
def test_actorder_gemm(q4, N, K, g, B):
    say(f"act-order gemm B={B} N={N} K={K} g={g}")
    W = synth.weight(N, K, seed=B + N)
    x = synth.activation(B, K, seed=K + B)
    aw, q_o, s_o, gi = _check_actorder_exact(q4, W, g, synth.channel_energy(K, seed=K))
    y1 = to_np(q4.gemm_perm(to_gpu(x), aw))
    y2 = to_np(q4.gemm_perm(to_gpu(x), aw))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16)), "non-deterministic"
    assert_close(y1, oracle.gemm_gidx_rows(x, q_o, s_o, gi, np.arange(N)), f"act-order B={B} N={N} K={K} g={g}")


def test_actorder_gemm_empty_batch(q4):
    import torch

    K = 256
    perm = q4.actorder_perm(np.arange(K) // 128, 128)
    aw = q4.quantize_pack_perm(to_gpu(synth.weight(32, K)), 128, to_gpu(perm))
    y = q4.gemm_perm(torch.empty((0, K), dtype=torch.float16, device="cuda"), aw)
    assert tuple(y.shape) == (0, 32)


def _full_actorder(q4, N, K, g, Bs, seed, heavy=False, nrows=64):
    import torch

    if heavy:
        W, cols = synth.heavy_tailed_weight(N, K, seed=seed)
        h = np.ones(K)
        h[cols] = 50.0                       # the outlier channels first
    else:
        W = synth.weight(N, K, seed=seed)
        h = synth.channel_energy(K, seed=seed)
    r = np.random.default_rng(seed + 1)
    rows = np.unique(np.concatenate([[0, N - 1], r.choice(N, size=nrows, replace=False)]))
    aw, q_o, s_o, gi = _check_actorder_exact(q4, W, g, h, rows=rows)
    for B in Bs:
        x = synth.activation(B, K, seed=seed + B)
        y = to_np(q4.gemm_perm(to_gpu(x), aw))
        rel, mx = assert_close(y[:, rows], oracle.gemm_gidx_rows(x, q_o, s_o, gi, np.arange(len(rows))),
                               f"act-order N={N} K={K} B={B}")
        say(f"  act-order N={N} K={K} g={g} B={B}: rel L2 {rel:.2e} max {mx:.2e}")
    del aw
    torch.cuda.empty_cache()


def test_actorder_full_28672x8192(q4):
    say("act-order 28672x8192")
    _full_actorder(q4, 28672, 8192, 128, (1, 4, 16, 32), seed=4)


def test_actorder_full_down_8192x28672(q4):
    say("act-order 8192x28672")
    _full_actorder(q4, 8192, 28672, 128, (1, 8), seed=6)


def test_actorder_full_heavy_tailed(q4):
    say("act-order heavy-tailed 14336x4096")
    _full_actorder(q4, 14336, 4096, 128, (1, 4), seed=5, heavy=True)
