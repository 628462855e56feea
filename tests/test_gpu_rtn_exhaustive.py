"""The quantizers' division-free code decision on the device, for every float16 weight.

The kernels round w / s half to even from one hardware reciprocal per scale and a
tie check ("LLM 后训练量化深度实战…", www.ybb.press, section 二: q = round(w / scale)).
tests/test_rtn_decision.py proves on the host that this equals the IEEE quotient's
decision; here the device itself runs it: for each of ~170 float16 scales (all
binades, subnormals included) a matrix holds every finite float16 weight the scale's
group can contain, next to the element that fixes the scale, and the codes of every
quantizer that uses the decision -- symmetric INT4 (g = 32 and 128), asymmetric uint4
(scale, zero point, codes), the clipping search at p_min = 100, per-channel INT8 and
the INT4 KV cache -- must equal the oracle's bit for bit.

Also here: products of the bias-folded symmetric GEMV (the float16 magic-number
operands with a per-block float32 bias removed from each partial) on activations
that are not zero-mean, x = c + N(0, 1) for c in {1, 8, 64} and |N(0, 1)|, at the
stated tolerance.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, say, to_gpu, to_np
from test_rtn_decision import _all_finite_fp16, _scales

pytestmark = pytest.mark.gpu

ALL16 = _all_finite_fp16()


@pytest.fixture(scope="module")
def q4():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_decode_amd as q4mod

    say("libq4", q4mod.version())
    return q4mod


def _amax_for_scale(s16, d, scale_fn):
    """A float16 amax whose scale is exactly s16 (None if no float16 amax gives it)."""
    a = np.float16(min(float(s16) * d, 65504.0))
    with np.errstate(over="ignore"):
        cands = (a, np.nextafter(a, np.float16(0)), np.nextafter(a, np.float16(np.inf)))
    for cand in cands:
        if np.isfinite(cand) and cand > 0 and scale_fn(np.array([cand], dtype=np.float16))[0] == s16:
            return cand
    return None


def _groups(lead, pool, g, fill=0.0):
    """Rows of groups [lead, pool...] of size g: every value of pool once, the last group
    padded with `fill` (a value inside the pool's range)."""
    per = g - len(lead)
    n = -(-pool.size // per)
    body = np.full(n * per, fill, dtype=np.float16)
    body[:pool.size] = pool
    head = np.tile(np.asarray(lead, dtype=np.float16), (n, 1))
    return np.concatenate([head, body.reshape(n, per)], axis=1)


def _matrix(groups, K, g):
    """Stack groups of g into rows of K channels (zero groups pad the last row)."""
    per_row = K // g
    rows = -(-groups.shape[0] // per_row)
    out = np.zeros((rows * per_row, g), dtype=np.float16)
    out[:groups.shape[0]] = groups
    return out.reshape(rows, K)


def _sym_matrix(g):
    groups = []
    for s16 in _scales():
        amax = _amax_for_scale(s16, 7, oracle.sym_scale_fp16)
        if amax is None:
            continue
        pool = ALL16[np.abs(ALL16.astype(np.float64)) <= float(amax)]
        groups.append(_groups([amax], pool, g))
    return _matrix(np.concatenate(groups), 1024, g)


@pytest.mark.parametrize("g", [32, 128])
def test_sym_codes_every_fp16_weight(q4, g):
    W = _sym_matrix(g)
    say(f"symmetric INT4, every float16 weight per scale: W {W.shape}, g={g}")
    qw = q4.quantize_pack(to_gpu(W), g)
    codes, scales, _ = q4.to_canonical(qw)
    q_o, s_o = oracle.quantize_sym(W, g)
    assert np.array_equal(to_np(scales).view(np.uint16), s_o.view(np.uint16))
    assert np.array_equal(to_np(codes), oracle.pack_canonical(q_o))
    if g in (32, 128):
        qc = q4.quantize_pack_clip(to_gpu(W), g, 100)
        codes_c, scales_c, _ = q4.to_canonical(qc)
        q_c, s_c, _ = oracle.quantize_sym_clip(W, g, 100)
        assert np.array_equal(to_np(scales_c).view(np.uint16), s_c.view(np.uint16))
        assert np.array_equal(to_np(codes_c), oracle.pack_canonical(q_c))


def test_asym_codes_every_fp16_weight(q4):
    g = 64
    groups = []
    for i, s in enumerate(_scales()):
        z = (1, 8, 14, 0, 15)[i % 5]
        with np.errstate(over="ignore"):
            mn = np.float16(-z * float(s))
            mx = np.float16((15 - z) * float(s))
        if not (np.isfinite(mn) and np.isfinite(mx)) or mx == mn:
            continue
        v = ALL16.astype(np.float64)
        pool = ALL16[(v >= float(mn)) & (v <= float(mx))]
        groups.append(_groups([mn, mx], pool, g, fill=float(mn)))
    W = _matrix(np.concatenate(groups), 1024, g)
    say(f"asymmetric uint4, every float16 weight per (min, max): W {W.shape}, g={g}")
    qw = q4.quantize_pack(to_gpu(W), g, asym=True)
    codes, scales, zeros = q4.to_canonical(qw)
    q_o, s_o, z_o = oracle.quantize_asym(W, g)
    assert np.array_equal(to_np(scales).view(np.uint16), s_o.view(np.uint16))
    assert np.array_equal(to_np(zeros), z_o)
    assert np.array_equal(to_np(codes), oracle.pack_canonical(q_o))


def test_w8_codes_every_fp16_weight(q4):
    rows = []
    for s16 in _scales():
        amax = _amax_for_scale(s16, 127, oracle.w8_scale_fp16)
        if amax is None:
            continue
        rows.append(np.concatenate([[amax], ALL16[np.abs(ALL16.astype(np.float64)) <= float(amax)]]))
    K = -(-max(r.size for r in rows) // 128) * 128
    W = np.zeros((len(rows), K), dtype=np.float16)
    for i, r in enumerate(rows):
        W[i, :r.size] = r
    say(f"per-channel INT8, every float16 weight per row scale: W {W.shape}")
    qw = q4.q8_quantize_pack(to_gpu(W))
    codes, scales = q4.q8_to_canonical(qw)
    q_o, s_o = oracle.quantize_w8(W)
    assert np.array_equal(to_np(scales).view(np.uint16), s_o.view(np.uint16))
    assert np.array_equal(to_np(codes), q_o)


@pytest.mark.parametrize("g", [32, 128])
def test_kv_codes_every_fp16_value(q4, g):
    d = 128
    groups = _matrix(np.concatenate([_sym_matrix(g).reshape(-1, g)]), d, g)  # tokens of head_dim d
    n = groups.shape[0]
    src = groups.reshape(1, 1, n, d)
    say(f"INT4 KV cache, every float16 value per scale: {n} tokens x {d}, g={g}")
    cache = q4.kv_cache_alloc(1, n, d, g)
    q4.kv_quantize_pack(to_gpu(src), cache, 0)
    q_o, s_o = oracle.quantize_kv_int4(src, g)
    assert np.array_equal(to_np(cache.scales).view(np.uint16), s_o.reshape(1, n, d // g).view(np.uint16))
    assert np.array_equal(to_np(cache.codes), oracle.pack_kv_int4(q_o).reshape(1, n, d // 2))


def test_device_decision_every_fp16_pair(q4):
    """q4_rtn_check: the kernels' division-free decision against rint of the correctly
    rounded float32 quotient for every positive finite float16 scale and every finite
    float16 weight, on the device itself (the host proof in test_rtn_decision models
    v_rcp_f32 as within one ulp; this checks the hardware and the compiled code)."""
    checked, bad = q4.rtn_check()
    say(f"device decision: {checked} (w, s) pairs, {bad} mismatches")
    assert checked == 31743 * 63488
    assert bad == 0


OFFSET_SHAPES = [(4096, 4096), (1024, 8192), (8192, 8192), (2048, 28672)]


@pytest.mark.parametrize("B", [1, 4])
@pytest.mark.parametrize("N,K", OFFSET_SHAPES)
def test_gemv_offset_activations(q4, N, K, B):
    W = synth.weight(N, K, seed=N + K)
    qw = q4.quantize_pack(to_gpu(W), 128)
    q_o, s_o = oracle.quantize_sym(W, 128)
    rows = np.unique(np.concatenate([np.arange(0, N, max(1, N // 96)), [N - 1]]))
    z = synth.activation(B, K, seed=B + K).astype(np.float32)
    for name, x32 in (("c=1", z + 1), ("c=8", z + 8), ("c=64", z + 64), ("|z|", np.abs(z))):
        x = x32.astype(np.float16)
        say(f"GEMV offset activations N={N} K={K} B={B} x={name}")
        y = to_np(q4.gemm(to_gpu(x), qw))
        ref = oracle.gemm_ref_rows(x, q_o, s_o, 128, rows)
        assert_close(y[:, rows], ref, f"{N}x{K} B={B} x={name}")
