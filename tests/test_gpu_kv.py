"""INT4 KV-cache HIP path vs the oracle, through the C ABI (needs an MI355X).

Codes and scales must match the oracle bit for bit at the positions written, every
other position of the cache must keep its contents, and the dequantized values
must equal the oracle's float64 x_hat rounded once to float16.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import say, to_gpu, to_np

pytestmark = pytest.mark.gpu

SENT_CODE, SENT_SCALE = 0xA5, 0x1234


@pytest.fixture(scope="module")
def q4():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_decode_amd as q4mod

    say("libq4", q4mod.version())
    return q4mod


def _kv(b, h, s, d, seed, scale_heads=True):
    r = np.random.default_rng(seed)
    x = r.standard_normal((b, h, s, d)).astype(np.float32)
    if scale_heads:
        x *= r.lognormal(size=(1, h, 1, 1)).astype(np.float32)
    return x.astype(np.float16)


def _cache(q4, bh, max_seq, d, g):
    c = q4.kv_cache_alloc(bh, max_seq, d, g)
    c.codes.fill_(SENT_CODE)
    c.scales.view(dtype=__import__("torch").int16).fill_(SENT_SCALE)
    return c


def _check_written(cache, K, g, pos):
    b, h, n, d = K.shape
    q_o, s_o = oracle.quantize_kv_int4(K, g)
    codes = to_np(cache.codes).reshape(b, h, -1, d // 2)
    scales = to_np(cache.scales).reshape(b, h, -1, d // g)
    assert np.array_equal(codes[:, :, pos:pos + n], oracle.pack_kv_int4(q_o)), (K.shape, g, pos, "codes")
    assert np.array_equal(scales[:, :, pos:pos + n].view(np.uint16), s_o.view(np.uint16)), (K.shape, g, pos, "scales")
    return q_o, s_o


def _check_untouched(cache, written):
    codes = to_np(cache.codes)
    scales = to_np(cache.scales).view(np.uint16)
    mask = np.ones(codes.shape[1], dtype=bool)
    for p0, p1 in written:
        mask[p0:p1] = False
    assert np.all(codes[:, mask] == SENT_CODE) and np.all(scales[:, mask] == SENT_SCALE)


@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_kv_prefill_bit_exact(q4, d, g):
    if d % g:
        pytest.skip("head_dim must be a multiple of the group")
    say(f"kv prefill d={d} g={g}")
    K = _kv(2, 8, 37, d, seed=d + g)
    cache = _cache(q4, 16, 64, d, g)
    q4.kv_quantize_pack(to_gpu(K), cache, 0)
    q_o, s_o = _check_written(cache, K, g, 0)
    _check_untouched(cache, [(0, 37)])
    deq = to_np(q4.kv_dequant(cache, 0, 37)).reshape(K.shape)
    ref = oracle.dequant_kv_int4(q_o, s_o, g).astype(np.float16)
    assert np.array_equal(deq.view(np.uint16), ref.view(np.uint16))


def test_kv_append_matches_prefill(q4):
    """Decode steps (n = 1 at pos = t) write what one prefill of the same tokens writes."""
    d, g = 128, 128
    K = _kv(3, 8, 9, d, seed=1)
    pre = _cache(q4, 24, 16, d, g)
    q4.kv_quantize_pack(to_gpu(K[:, :, :4]), pre, 0)          # a prompt of 4
    for t in range(4, 9):                                      # 5 decode steps
        q4.kv_quantize_pack(to_gpu(np.ascontiguousarray(K[:, :, t:t + 1])), pre, t)
    _check_written(pre, K, g, 0)
    _check_untouched(pre, [(0, 9)])


def test_kv_offset_window(q4):
    d, g = 128, 64
    K = _kv(1, 4, 20, d, seed=2)
    cache = _cache(q4, 4, 40, d, g)
    q4.kv_quantize_pack(to_gpu(K), cache, 17)
    _check_written(cache, K, g, 17)
    _check_untouched(cache, [(17, 37)])
    deq = to_np(q4.kv_dequant(cache, 17, 20)).reshape(K.shape)
    q_o, s_o = oracle.quantize_kv_int4(K, g)
    assert np.array_equal(deq.view(np.uint16), oracle.dequant_kv_int4(q_o, s_o, g).astype(np.float16).view(np.uint16))


def test_kv_edge_values(q4):
    d, g = 128, 32
    r = np.random.default_rng(3)
    sink = _kv(1, 8, 16, d, seed=4)
    sink[:, :, :2] *= np.float16(100)                          # attention-sink tokens
    ties = (r.integers(-15, 16, size=(1, 8, 16, d)) * 0.5).astype(np.float16)
    ties[..., ::32] = np.float16(7)                            # scale exactly 1 per group: half-integer ties
    cases = {
        "zeros": np.zeros((1, 8, 16, d), dtype=np.float16),
        "subnormal": (r.integers(-3, 4, size=(1, 8, 16, d)) * 2.0 ** -24).astype(np.float16),
        "huge": np.clip(_kv(1, 8, 16, d, seed=5).astype(np.float32) * 2e4, -65504, 65504).astype(np.float16),
        "sink": sink,
        "ties": ties,
    }
    for name, K in cases.items():
        say(f"  kv {name}")
        cache = _cache(q4, 8, 16, d, g)
        q4.kv_quantize_pack(to_gpu(K), cache, 0)
        _check_written(cache, K, g, 0)


def test_kv_full_70b_layer_prefill(q4):
    """One Llama-3-70B layer's K for a 32768-token prompt (8 KV heads x 128), checked on
    sampled tokens (tokens are quantized independently)."""
    import torch

    say("kv 70B layer prefill 32768 tokens")
    b, h, s, d, g = 1, 8, 32768, 128, 128
    Kd = synth.device_activation(b * h * s, d, seed=7, layer=0, matrix=0, device="cuda").view(b, h, s, d)
    cache = q4.kv_cache_alloc(b * h, s, d, g)
    q4.kv_quantize_pack(Kd, cache, 0)
    toks = np.sort(np.random.default_rng(9).choice(s, 64, replace=False))
    K = to_np(Kd[:, :, torch.from_numpy(toks).cuda()])
    q_o, s_o = oracle.quantize_kv_int4(K, g)
    codes = to_np(cache.codes).reshape(b, h, s, d // 2)[:, :, toks]
    scales = to_np(cache.scales).reshape(b, h, s, d // g)[:, :, toks]
    assert np.array_equal(codes, oracle.pack_kv_int4(q_o))
    assert np.array_equal(scales.view(np.uint16), s_o.view(np.uint16))
