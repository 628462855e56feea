"""W8A16 (per-channel INT8) HIP path vs the oracle, through the C ABI (needs an MI355X).

Quantization must match bit for bit (codes, scales, device layout with its
padding); products must meet relative L2 <= 1e-3 and max |dy| <= 1e-3 * max |y|
against the oracle's float64 product of the oracle's own codes.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, say, to_gpu, to_np

pytestmark = pytest.mark.gpu

SHAPES = [  # (N, K): several tiles, ragged rows, channel counts off the 128-channel blocks
    (1, 8), (17, 96), (33, 200), (40, 352), (48, 384), (100, 1280), (129, 640), (64, 4096), (16, 136), (31, 8200),
]


@pytest.fixture(scope="module")
def q4():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_decode_amd as q4mod

    say("libq4", q4mod.version())
    return q4mod


def _check_w8_exact(q4, W, device_layout=True, rows=None):
    """q8_quantize_pack against oracle.quantize_w8: canonical codes and scales bit for
    bit (on `rows` only when given: rows are quantized independently)."""
    N, K = W.shape
    qw = q4.q8_quantize_pack(to_gpu(W))
    codes, scales = q4.q8_to_canonical(qw)
    Wo = W if rows is None else W[rows]
    q_o, s_o = oracle.quantize_w8(Wo)
    c = to_np(codes) if rows is None else to_np(codes)[rows]
    sc = to_np(scales) if rows is None else to_np(scales)[rows]
    assert np.array_equal(c, q_o), (N, K, "codes")
    assert np.array_equal(sc.view(np.uint16), s_o.view(np.uint16)), (N, K, "scales")
    if device_layout:
        assert np.array_equal(to_np(qw.packed), oracle.w8_codes_to_device(q_o)), (N, K, "device codes")
        assert np.array_equal(to_np(qw.scales).view(np.uint16), oracle.w8_scales_to_device(s_o, N).view(np.uint16))
    return qw, q_o, s_o


@pytest.mark.parametrize("N,K", SHAPES)
def test_w8_quantize_bit_exact(q4, N, K):
    say(f"w8 quantize N={N} K={K}")
    _check_w8_exact(q4, synth.weight(N, K, seed=N * 5 + K))


def test_w8_quantize_edge_values(q4):
    N, K = 37, 384
    ties = np.zeros((N, K), dtype=np.float16)
    ties[:, 0] = np.float16(127 * 2.0 ** -6)               # scale exactly 2^-6
    ties[:, 1:] = ((np.arange(K - 1) % 255 - 127) * 0.5 * 2.0 ** -6).astype(np.float16)  # half-integer quotients
    tiny = np.zeros((N, K), dtype=np.float16)
    tiny[:, 3] = np.float16(-1e-5)                          # subnormal scale: clamped codes
    tiny[:, 5] = (np.arange(N) * 2.0 ** -24).astype(np.float16)
    cases = {
        "ties": ties,
        "all_zero": np.zeros((N, K), dtype=np.float16),
        "tiny_rows": tiny,
        "small": (synth.weight(N, K, seed=2).astype(np.float32) * np.float32(1e-3)).astype(np.float16),
        "huge": (synth.weight(N, K, seed=3).astype(np.float32) * np.float32(2.0e4)).clip(-65504, 65504).astype(np.float16),
        "constant_rows": np.full((N, K), -0.5, dtype=np.float16),
        "heavy_tailed": synth.heavy_tailed_weight(N, K, seed=6)[0],
    }
    for name, W in cases.items():
        say(f"  w8 {name}")
        _check_w8_exact(q4, W)


def test_w8_quantize_heavy_tailed_full(q4):
    """The heavy-tailed 14336x4096 workload, checked bit for bit on 512 sampled rows."""
    W, _ = synth.heavy_tailed_weight(14336, 4096, seed=5)
    rows = np.sort(np.random.default_rng(8).choice(14336, 512, replace=False))
    _check_w8_exact(q4, W, device_layout=False, rows=rows)


def test_w8_canonical_round_trip(q4):
    r = np.random.default_rng(4)
    for N, K in ((40, 352), (33, 200), (100, 1280)):
        q = r.integers(-128, 128, size=(N, K)).astype(np.int8)   # -128 included: imported codes
        s = (r.uniform(1e-4, 1e-2, size=N)).astype(np.float16)
        qw = q4.q8_from_canonical(to_gpu(q), to_gpu(s))
        dev = to_np(qw.packed)
        want = np.full_like(dev, 128)
        ok = q != -128
        want_ok = oracle.w8_codes_to_device(np.where(ok, q, 0))
        pos = oracle.w8_codes_to_device(np.where(ok, 0, 1)) != 128   # device positions of the -128 codes
        want[:] = want_ok
        want[pos] = 0
        assert np.array_equal(dev, want)
        assert np.array_equal(to_np(qw.scales).view(np.uint16), oracle.w8_scales_to_device(s, N).view(np.uint16))
        c, sc = q4.q8_to_canonical(qw)
        assert np.array_equal(to_np(c), q) and np.array_equal(to_np(sc).view(np.uint16), s.view(np.uint16))
        x = synth.activation(3, K, seed=N)
        y = to_np(q4.q8_gemm(to_gpu(x), qw))
        assert_close(y, oracle.gemm_w8_rows(x, q, s, np.arange(N)), f"imported codes N={N} K={K}")


GEMM_CASES = [  # (B, N, K): GEMV up to B = 16, skinny GEMM above (2, 4 and 8 column tiles, k-splits)
    (1, 1, 8), (1, 17, 96), (3, 40, 352), (2, 33, 200), (4, 48, 384), (7, 100, 1280), (8, 129, 640),
    (9, 64, 2048), (16, 200, 1024), (17, 100, 512), (40, 33, 1024), (1, 16, 8192), (2, 4000, 256), (5, 31, 8200),
    (32, 300, 2048), (64, 129, 1000), (100, 300, 1280), (129, 40, 4096), (256, 96, 1024), (33, 1024, 8192),
]


@pytest.mark.parametrize("B,N,K", GEMM_CASES)
def test_w8_gemm_small(q4, B, N, K):
    say(f"w8 gemm B={B} N={N} K={K}")
    W = synth.weight(N, K, seed=B + N)
    x = synth.activation(B, K, seed=K + B)
    qw, q_o, s_o = _check_w8_exact(q4, W, device_layout=False)
    y = to_np(q4.q8_gemm(to_gpu(x), qw))
    assert_close(y, oracle.gemm_w8_rows(x, q_o, s_o, np.arange(N)), f"w8 B={B} N={N} K={K}")


def test_w8_gemm_launch_shapes_agree(q4):
    """Every GEMV tuning shape meets the tolerance and is deterministic."""
    B, N, K = 4, 300, 2048
    W = synth.weight(N, K, seed=1)
    x = synth.activation(B, K, seed=2)
    qw, q_o, s_o = _check_w8_exact(q4, W, device_layout=False)
    ref = oracle.gemm_w8_rows(x, q_o, s_o, np.arange(N))
    xg = to_gpu(x)
    ran = 0
    for R in (1, 2, 4):
        for Wv in (1, 2, 4, 8, 16):
            for KS in (1, 3, 16):
                say(f"  w8 config R={R} W={Wv} KS={KS}")
                try:
                    y1 = to_np(q4.q8_gemm_config(xg, qw, R, Wv, KS))
                except q4.Q4Error as e:
                    nsb = -(-(K // 128) // KS)
                    assert e.status == 5 and B * nsb * 16 > 8 * Wv * 64, str(e)
                    continue
                y2 = to_np(q4.q8_gemm_config(xg, qw, R, Wv, KS))
                assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16)), "non-deterministic"
                assert_close(y1, ref, f"w8 R={R} W={Wv} KS={KS}")
                ran += 1
    assert ran >= 40


def test_w8_gemm_empty_batch(q4):
    import torch

    qw = q4.q8_quantize_pack(to_gpu(synth.weight(32, 128)))
    y = q4.q8_gemm(torch.empty((0, 128), dtype=torch.float16, device="cuda"), qw)
    assert tuple(y.shape) == (0, 32)


def _full_w8(q4, N, K, Bs, seed, nrows=96, heavy=False):
    import torch

    W = synth.heavy_tailed_weight(N, K, seed=seed)[0] if heavy else synth.weight(N, K, seed=seed)
    Wg = to_gpu(W)
    qw = q4.q8_quantize_pack(Wg)
    del Wg
    r = np.random.default_rng(seed + 1)
    rows = np.unique(np.concatenate([[0, N - 1], r.choice(N, size=min(nrows, N), replace=False)]))
    q_o, s_o = oracle.quantize_w8(W[rows])
    c, s = q4.q8_to_canonical(qw)
    idx = torch.from_numpy(rows).cuda()
    assert np.array_equal(to_np(c[idx]), q_o)
    assert np.array_equal(to_np(s[idx]).view(np.uint16), s_o.view(np.uint16))
    for B in Bs:
        x = synth.activation(B, K, seed=seed + B)
        y = to_np(q4.q8_gemm(to_gpu(x), qw))
        rel, mx = assert_close(y[:, rows], oracle.gemm_w8_rows(x, q_o, s_o, np.arange(len(rows))),
                               f"w8 N={N} K={K} B={B}")
        say(f"  w8 N={N} K={K} B={B}: rel L2 {rel:.2e} max {mx:.2e}")


@pytest.mark.parametrize("name", list(synth.LLAMA3_70B))
def test_w8_full_70b_shapes(q4, name):
    N, K = synth.LLAMA3_70B[name]
    say(f"w8 70B {name} {N}x{K}")
    _full_w8(q4, N, K, (1, 2, 4, 8), seed=3)


def test_w8_full_batch_28672x8192(q4):
    say("w8 28672x8192 B = 1, 16, 32, 64, 256")
    _full_w8(q4, 28672, 8192, (1, 16, 32, 64, 256), seed=4, nrows=64)


def test_w8_full_fused_gate_up_b128(q4):
    """The fused 70B gate/up matrix (57344x8192, device-generated weights) at B = 128,
    where the skinny GEMM takes wider column groups to stay within one round of
    workgroups, and at B = 64 and 256 beside it; codes, scales, products on sampled rows."""
    import torch

    N, K = 57344, 8192
    say(f"w8 fused gate/up {N}x{K}")
    Wd = synth.device_weight(N, K, seed=6, layer=0, matrix=1)
    qw = q4.q8_quantize_pack(Wd)
    r = np.random.default_rng(8)
    rows = np.unique(np.concatenate([[0, N - 1], r.choice(N, size=64, replace=False)]))
    idx = torch.from_numpy(rows).cuda()
    W = to_np(Wd[idx])
    del Wd
    q_o, s_o = oracle.quantize_w8(W)
    c, s = q4.q8_to_canonical(qw)
    assert np.array_equal(to_np(c[idx]), q_o)
    assert np.array_equal(to_np(s[idx]).view(np.uint16), s_o.view(np.uint16))
    for B in (64, 128, 256):
        x = synth.activation(B, K, seed=B + 1)
        y = to_np(q4.q8_gemm(to_gpu(x), qw))
        rel, mx = assert_close(y[:, rows], oracle.gemm_w8_rows(x, q_o, s_o, np.arange(len(rows))),
                               f"w8 gate/up B={B}")
        say(f"  w8 gate/up B={B}: rel L2 {rel:.2e} max {mx:.2e}")


def test_w8_full_heavy_tailed(q4):
    say("w8 heavy-tailed 14336x4096")
    _full_w8(q4, 14336, 4096, (1, 4), seed=5, heavy=True)
