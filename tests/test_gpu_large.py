"""Inputs past 2^31 elements (needs an MI355X).

65541 x 32896 float16 weights (2,156,036,736 elements, 4.3 GB; the last row a ragged
16-row tile, 257 blocks of 128 channels per row) cross every 32-bit element and
byte offset: the quantizers' reads, the packed codes and scales, the canonical
converters and the products' weight streams. Weights come from the device
generator; sampled rows (the first and last included) are checked against the
oracle: INT4 codes and scales bit for bit, products within the tolerance of the
other parity tests, for the GEMV (B = 1, 4: the latter with a channel split) and
the skinny GEMM (B = 32); likewise the per-row INT8 path, and a KV cache of more
than 2^31 code words.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, say, to_gpu, to_np

pytestmark = pytest.mark.gpu

N, K = 65541, 32896


@pytest.fixture(scope="module")
def q4():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_decode_amd as q4mod

    return q4mod


@pytest.fixture(scope="module")
def big(q4):
    import torch

    assert N * K > 2**31
    Wd = synth.device_weight(N, K, seed=11, layer=0, matrix=0)
    r = np.random.default_rng(12)
    rows = np.unique(np.concatenate([[0, N - 2, N - 1], r.choice(N, size=61, replace=False)]))
    idx = torch.from_numpy(rows).cuda()
    W = to_np(Wd[idx])
    yield Wd, rows, idx, W
    del Wd
    torch.cuda.empty_cache()


def test_int4_over_2g_weights(q4, big):
    Wd, rows, idx, W = big
    g = 128
    say(f"INT4 {N}x{K} ({N * K} weights)")
    qw = q4.quantize_pack(Wd, g)
    q_o, s_o = oracle.quantize_sym(W, g)
    c, s, _ = q4.to_canonical(qw)
    assert np.array_equal(to_np(c[idx]), oracle.pack_canonical(q_o))
    assert np.array_equal(to_np(s[idx]).view(np.uint16), s_o.view(np.uint16))
    del c, s
    w_hat = oracle.dequant_sym(q_o, s_o, g)
    for B in (1, 4, 32):
        x = synth.activation(B, K, seed=100 + B)
        y = to_np(q4.gemm(to_gpu(x), qw))
        rel, mx = assert_close(y[:, rows], oracle.gemm_ref(x, w_hat), f"INT4 {N}x{K} B={B}")
        say(f"  B={B}: rel L2 {rel:.2e} max {mx:.2e}")


def test_int8_over_2g_weights(q4, big):
    Wd, rows, idx, W = big
    say(f"INT8 {N}x{K} ({N * K} code bytes)")
    qw = q4.q8_quantize_pack(Wd)
    q_o, s_o = oracle.quantize_w8(W)
    c, s = q4.q8_to_canonical(qw)
    assert np.array_equal(to_np(c[idx]), q_o)
    assert np.array_equal(to_np(s[idx]).view(np.uint16), s_o.view(np.uint16))
    del c, s
    for B in (1, 32):
        x = synth.activation(B, K, seed=200 + B)
        y = to_np(q4.q8_gemm(to_gpu(x), qw))
        rel, mx = assert_close(y[:, rows], oracle.gemm_w8_rows(x, q_o, s_o, np.arange(len(rows))),
                               f"INT8 {N}x{K} B={B}")
        say(f"  B={B}: rel L2 {rel:.2e} max {mx:.2e}")


def test_kv_cache_over_2g_words(q4):
    """A KV cache of 128 sequences x 1048584 positions x 128 channels (2,147,500,032
    code words): three tokens appended at its last positions land past every 32-bit
    word and byte offset; codes, scales and their dequantization equal the oracle's,
    and the position before them keeps its sentinel."""
    import torch

    bh, max_seq, d, g = 128, (1 << 20) + 8, 128, 128
    n, pos = 3, max_seq - 3
    assert bh * max_seq * d // 8 > 2**31
    say(f"KV cache {bh}x{max_seq}x{d}, append {n} at {pos}")
    cache = q4.kv_cache_alloc(bh, max_seq, d, g)
    cache.codes[:, pos - 1:].fill_(0x5A)
    cache.scales[:, pos - 1:].view(torch.int16).fill_(0x1234)
    r = np.random.default_rng(13)
    K = (r.standard_normal((16, 8, n, d)) * r.lognormal(size=(1, 8, 1, 1))).astype(np.float16)
    q4.kv_quantize_pack(to_gpu(K), cache, pos)
    q_o, s_o = oracle.quantize_kv_int4(K, g)
    codes = to_np(cache.codes[:, pos - 1:]).reshape(16, 8, n + 1, d // 2)
    scales = to_np(cache.scales[:, pos - 1:]).reshape(16, 8, n + 1, d // g)
    assert np.array_equal(codes[:, :, 1:], oracle.pack_kv_int4(q_o))
    assert np.array_equal(scales[:, :, 1:].view(np.uint16), s_o.view(np.uint16))
    assert np.all(codes[:, :, 0] == 0x5A) and np.all(scales[:, :, 0].view(np.uint16) == 0x1234)
    deq = to_np(q4.kv_dequant(cache, pos, n)).reshape(K.shape)
    assert np.array_equal(deq.view(np.uint16), oracle.dequant_kv_int4(q_o, s_o, g).astype(np.float16).view(np.uint16))
    del cache
    torch.cuda.empty_cache()
