"""HIP path vs the oracle, through the C ABI (needs an MI355X).

Quantization must match bit for bit (codes, scales, zero points, padding);
products must meet relative L2 <= 1e-3 and max |dy| <= 1e-3 * max |y|.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, say, to_gpu, to_np

pytestmark = pytest.mark.gpu

SMALL_SHAPES = [  # (N, K, g): several tiles, ragged row and channel tails
    (1, 32, 32), (17, 96, 32), (33, 192, 64), (40, 352, 32), (48, 384, 128),
    (31, 512, 256), (16, 4096, 4096), (100, 1280, 128), (129, 640, 64), (64, 2048, 512),
]


@pytest.fixture(scope="module")
def q4():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_decode_amd as q4mod

    say("libq4", q4mod.version())
    return q4mod


def _oracle_quant(W, g, asym):
    if asym:
        return oracle.quantize_asym(W, g)
    q, s = oracle.quantize_sym(W, g)
    return q, s, None


def _check_quant_exact(q4, W, g, asym, device_layout=True):
    N, K = W.shape
    qw = q4.quantize_pack(to_gpu(W), g, asym=asym)
    q_o, s_o, z_o = _oracle_quant(W, g, asym)
    codes, scales, zeros = q4.to_canonical(qw)
    assert np.array_equal(to_np(codes), oracle.pack_canonical(q_o)), (N, K, g, asym, "canonical codes")
    assert np.array_equal(to_np(scales).view(np.uint16), s_o.view(np.uint16)), (N, K, g, asym, "scales")
    if asym:
        assert np.array_equal(to_np(zeros), z_o), (N, K, g, "zeros")
    if device_layout:
        assert np.array_equal(to_np(qw.packed), oracle.codes_to_device(q_o, symmetric=not asym)), "device codes"
        dev_s = oracle.groupwise_to_device(s_o, N, K, g).ravel()
        assert np.array_equal(to_np(qw.scales).view(np.uint16), dev_s.view(np.uint16)), "device scales"
        if asym:
            assert np.array_equal(to_np(qw.zeros), oracle.groupwise_to_device(z_o, N, K, g).ravel())
    return qw, q_o, s_o, z_o


@pytest.mark.parametrize("asym", [False, True], ids=["sym", "asym"])
@pytest.mark.parametrize("N,K,g", SMALL_SHAPES)
def test_quantize_small_bit_exact(q4, N, K, g, asym):
    say(f"quantize N={N} K={K} g={g} asym={asym}")
    W = synth.weight(N, K, seed=N * 7 + K)
    _check_quant_exact(q4, W, g, asym)


@pytest.mark.parametrize("asym", [False, True], ids=["sym", "asym"])
def test_quantize_edge_values(q4, asym):
    say(f"quantize edge values asym={asym}")
    N, K = 37, 384
    cases = {
        "ties_and_zero_groups": synth.uniform_codes_weight(N, K, seed=1),
        "all_zero": np.zeros((N, K), dtype=np.float16),
        "tiny": (synth.weight(N, K, seed=2).astype(np.float32) * np.float32(1e-4)).astype(np.float16),
        "subnormal": (np.arange(N * K) % 7 - 3).reshape(N, K).astype(np.float16) * np.float16(2.0 ** -24),
        "huge": (synth.weight(N, K, seed=3).astype(np.float32) * np.float32(2.0e4)).clip(-65504, 65504).astype(np.float16),
        "constant_rows": np.full((N, K), 0.5, dtype=np.float16),
        "one_sided": np.abs(synth.weight(N, K, seed=4)) + np.float16(0.01),
    }
    for name, W in cases.items():
        for g in (32, 128):
            say(f"  {name} g={g}")
            _check_quant_exact(q4, W, g, asym)


@pytest.mark.parametrize("asym", [False, True], ids=["sym", "asym"])
@pytest.mark.parametrize("g", [32, 64, 128])
def test_quantize_heavy_tailed_full(q4, g, asym):
    """The heavy-tailed 14336x4096 workload (Student-t df=3, 1% outlier columns x50)."""
    say(f"quantize heavy-tailed 14336x4096 g={g} asym={asym}")
    W, _ = synth.heavy_tailed_weight(14336, 4096, seed=5)
    _check_quant_exact(q4, W, g, asym, device_layout=False)


def _check_clip_exact(q4, W, g, pmin, rows=None):
    """q4_quantize_pack_clip against the oracle's clipping search: canonical codes and
    scales bit for bit (on `rows` only when given: rows are quantized independently)."""
    qw = q4.quantize_pack_clip(to_gpu(W), g, pmin)
    codes, scales, _ = q4.to_canonical(qw)
    Wo = W if rows is None else W[rows]
    q_o, s_o, _ = oracle.quantize_sym_clip(Wo, g, pmin)
    c = to_np(codes) if rows is None else to_np(codes)[rows]
    sc = to_np(scales) if rows is None else to_np(scales)[rows]
    assert np.array_equal(c, oracle.pack_canonical(q_o)), (W.shape, g, pmin, "codes")
    assert np.array_equal(sc.view(np.uint16), s_o.view(np.uint16)), (W.shape, g, pmin, "scales")
    return qw, q_o, s_o


@pytest.mark.parametrize("pmin", [80, 100, 1])
@pytest.mark.parametrize("N,K,g", [(17, 96, 32), (33, 192, 64), (40, 352, 32), (48, 384, 128), (129, 640, 64),
                                   (100, 1280, 128)])
def test_quantize_clip_bit_exact(q4, N, K, g, pmin):
    say(f"quantize clip N={N} K={K} g={g} pmin={pmin}")
    W = synth.weight(N, K, seed=N * 3 + K)
    qw, q_o, s_o = _check_clip_exact(q4, W, g, pmin)
    assert np.array_equal(to_np(qw.packed), oracle.codes_to_device(q_o, symmetric=True)), "device codes"
    if pmin == 100:
        q_r, s_r = oracle.quantize_sym(W, g)
        assert np.array_equal(q_o, q_r) and np.array_equal(s_o.view(np.uint16), s_r.view(np.uint16))


def test_quantize_clip_edge_values(q4):
    N, K = 37, 384
    cases = {
        "ties_and_zero_groups": synth.uniform_codes_weight(N, K, seed=1),
        "all_zero": np.zeros((N, K), dtype=np.float16),
        "tiny": (synth.weight(N, K, seed=2).astype(np.float32) * np.float32(1e-4)).astype(np.float16),
        "huge": (synth.weight(N, K, seed=3).astype(np.float32) * np.float32(2.0e4)).clip(-65504, 65504).astype(np.float16),
        "constant_rows": np.full((N, K), 0.5, dtype=np.float16),
        "heavy_tailed": synth.heavy_tailed_weight(N, K, seed=6)[0],
    }
    for name, W in cases.items():
        for g in (32, 128):
            say(f"  clip {name} g={g}")
            _check_clip_exact(q4, W, g, 80)


@pytest.mark.parametrize("g", [32, 64, 128])
def test_quantize_clip_heavy_tailed_full(q4, g):
    """The heavy-tailed 14336x4096 workload with the clipping search (alpha 0.80..1.00),
    checked bit for bit on 512 sampled rows (rows are quantized independently)."""
    say(f"quantize clip heavy-tailed 14336x4096 g={g}")
    W, _ = synth.heavy_tailed_weight(14336, 4096, seed=5)
    rows = np.sort(np.random.default_rng(g).choice(14336, 512, replace=False))
    _check_clip_exact(q4, W, g, 80, rows=rows)


def test_gemm_on_clip_weights(q4):
    """The product reads clip-searched codes (-7..7) like RTN ones."""
    for B, N, K, g in ((1, 300, 2048, 128), (4, 129, 640, 64), (40, 100, 1280, 32)):
        say(f"  gemm on clip weights B={B} N={N} K={K} g={g}")
        W = synth.weight(N, K, seed=B + N)
        x = synth.activation(B, K, seed=K)
        qw, q_o, s_o = _check_clip_exact(q4, W, g, 80)
        assert_close(to_np(q4.gemm(to_gpu(x), qw)), _ref_product(x, q_o, s_o, None, g), f"clip B={B}")


def test_quantize_single_layer_full(q4):
    """4096x4096, N(0, 0.02^2), g=128, seed 0: codes and scales bit-exact, layout included."""
    say("quantize 4096x4096 g=128")
    W = synth.weight(4096, 4096, seed=0)
    _check_quant_exact(q4, W, 128, False)


def test_canonical_round_trip(q4):
    for N, K, g, asym in ((40, 352, 32, False), (33, 192, 64, True), (100, 1280, 128, True)):
        W = synth.weight(N, K, seed=9)
        q_o, s_o, z_o = _oracle_quant(W, g, asym)
        qw = q4.from_canonical(to_gpu(oracle.pack_canonical(q_o)), to_gpu(s_o), g,
                               zeros=to_gpu(z_o) if asym else None)
        assert np.array_equal(to_np(qw.packed), oracle.codes_to_device(q_o, symmetric=not asym))
        assert np.array_equal(to_np(qw.scales).view(np.uint16),
                              oracle.groupwise_to_device(s_o, N, K, g).ravel().view(np.uint16))
        c, s, z = q4.to_canonical(qw)
        assert np.array_equal(to_np(c), oracle.pack_canonical(q_o))


def _ref_product(x, q_o, s_o, z_o, g):
    w_hat = oracle.dequant_asym(q_o, s_o, z_o, g) if z_o is not None else oracle.dequant_sym(q_o, s_o, g)
    return oracle.gemm_ref(x, w_hat)


GEMM_CASES = [  # (B, N, K, g, asym)
    (1, 1, 32, 32, False), (1, 17, 96, 32, False), (3, 40, 352, 32, True), (2, 33, 192, 64, False),
    (4, 48, 384, 128, True), (5, 31, 512, 256, False), (7, 100, 1280, 128, False), (8, 129, 640, 64, True),
    (9, 64, 2048, 128, False), (15, 47, 1024, 128, False), (16, 200, 1024, 128, True), (17, 100, 512, 128, False),
    (31, 48, 1024, 64, False), (33, 65, 768, 128, True), (64, 128, 2048, 128, False), (65, 40, 512, 32, False),
    (100, 300, 1024, 128, False), (256, 96, 1024, 128, True), (1, 16, 4096, 4096, False), (2, 4000, 256, 128, False),
    (48, 40, 4096, 4096, False), (20, 33, 1024, 512, True), (129, 17, 384, 64, True),
]


@pytest.mark.parametrize("B,N,K,g,asym", GEMM_CASES)
def test_gemm_small(q4, B, N, K, g, asym):
    say(f"gemm B={B} N={N} K={K} g={g} asym={asym}")
    W = synth.weight(N, K, seed=B + N)
    x = synth.activation(B, K, seed=K + B)
    qw, q_o, s_o, z_o = _check_quant_exact(q4, W, g, asym, device_layout=False)
    y = q4.gemm(to_gpu(x), qw)
    assert_close(to_np(y), _ref_product(x, q_o, s_o, z_o, g), f"B={B} N={N} K={K} g={g}")


def test_gemm_launch_shapes_agree(q4):
    """Every tuning shape of the same kernel meets the tolerance; each is deterministic."""
    B, N, K, g = 4, 300, 2048, 128
    W = synth.weight(N, K, seed=1)
    x = synth.activation(B, K, seed=2)
    qw, q_o, s_o, _ = _check_quant_exact(q4, W, g, False, device_layout=False)
    ref = _ref_product(x, q_o, s_o, None, g)
    xg = to_gpu(x)
    ran = 0
    for R in (1, 2, 4):
        for Wv in (1, 2, 4, 8, 16):
            for KS in (1, 3, 16):
                say(f"  config R={R} W={Wv} KS={KS}")
                try:
                    y1 = to_np(q4.gemm_config(xg, qw, R, Wv, KS))
                except q4.Q4Error as e:
                    # shapes the kernel cannot run: an activation slice larger than one
                    # workgroup copies (8 chunks of 16 bytes per thread)
                    nsb = -(-(K // 128) // KS)
                    assert e.status == 5 and B * nsb * 16 > 8 * Wv * 64, str(e)
                    continue
                y2 = to_np(q4.gemm_config(xg, qw, R, Wv, KS))
                assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16)), "non-deterministic"
                assert_close(y1, ref, f"R={R} W={Wv} KS={KS}")
                ran += 1
    assert ran >= 40


@pytest.mark.parametrize("asym", [False, True], ids=["sym", "asym"])
@pytest.mark.parametrize("g", [32, 64, 128, 256, 1024])
@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_gemv_streamed_x(q4, B, g, asym):
    """B <= 3 with two row tiles per wavefront streams x per unit of 1024 channels
    (register and LDS room for 1, 2 or 4 rows; B = 3 leaves one unused), and so does
    B = 4 for symmetric codes with g = 128 (the burst form; other codes stage); ragged rows
    (N = 300), several units per row block, wavefronts left without work (W = 8 on
    few units) and the staged-slice kernel (k_splits = 2) agree with the oracle."""
    N, K = 300, 3072
    W = synth.weight(N, K, seed=g)
    x = synth.activation(B, K, seed=g + 1)
    qw, q_o, s_o, z_o = _check_quant_exact(q4, W, g, asym, device_layout=False)
    ref = _ref_product(x, q_o, s_o, z_o, g)
    xg = to_gpu(x)
    streamed = B <= 3 or (g == 128 and not asym)
    # staged B = 4 needs 8 wavefronts to copy its activation slice
    for Wv, KS in ((1, 1), (2, 1), (8, 1), (8, 2)) if streamed else ((8, 1), (8, 2)):
        say(f"  streamed x B={B} g={g} asym={asym} W={Wv} KS={KS}")
        y1 = to_np(q4.gemm_config(xg, qw, 2, Wv, KS))
        y2 = to_np(q4.gemm_config(xg, qw, 2, Wv, KS))
        assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16)), "non-deterministic"
        assert_close(y1, ref, f"B={B} g={g} W={Wv} KS={KS}")


@pytest.mark.parametrize("asym", [False, True], ids=["sym", "asym"])
@pytest.mark.parametrize("B,g", [(40, 128), (100, 32), (200, 64)])
def test_gemm_mfma_shapes_agree(q4, B, g, asym):
    """Skinny GEMM (B > 16): every row-tile / column-tile shape the kernel builds
    meets the tolerance and is deterministic; ragged rows (N = 300), a ragged last
    column group and a channel count that is not a multiple of the prefetch depth."""
    N, K = 300, 1280
    W = synth.weight(N, K, seed=B)
    x = synth.activation(B, K, seed=B + 1)
    qw, q_o, s_o, z_o = _check_quant_exact(q4, W, g, asym, device_layout=False)
    ref = _ref_product(x, q_o, s_o, z_o, g)
    xg = to_gpu(x)
    gsub = max(1, 128 // g)
    ran = 0
    for R in (1, 2, 4):
        for CT in (2, 3, 4, 6, 8):
            say(f"  config B={B} g={g} R={R} CT={CT}")
            try:
                y1 = to_np(q4.gemm_config(xg, qw, R, 4, 1, col_tiles=CT))
            except q4.Q4Error as e:
                assert e.status == 5 and R * CT * gsub > 16, str(e)
                continue
            y2 = to_np(q4.gemm_config(xg, qw, R, 4, 1, col_tiles=CT))
            assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16)), "non-deterministic"
            assert_close(y1, ref, f"B={B} g={g} R={R} CT={CT}")
            ran += 1
    assert ran >= 3


@pytest.mark.parametrize("B,N,K", [(4, 1000, 28672), (32, 4096, 8192), (6, 998, 28672)])
def test_split_sum_any_output_alignment(q4, B, N, K):
    """Products whose channel range is split over workgroups (float32 partials added
    by a second kernel: 8 outputs per thread when y is 16-byte aligned and B * N a
    multiple of 8, one per thread otherwise) give the same bits into an aligned output
    and into one that is only 2-byte aligned, and match the oracle."""
    import torch

    W = synth.weight(N, K, seed=40)
    x = synth.activation(B, K, seed=41)
    qw = q4.quantize_pack(to_gpu(W), 128)
    assert q4.workspace_bytes(B, N, K, 128) > 0, "shape must take a channel split"
    y_al = q4.gemm(to_gpu(x), qw)
    buf = torch.empty(B * N + 8, dtype=torch.float16, device="cuda")
    y_un = buf[1:1 + B * N].view(B, N)
    assert y_un.data_ptr() % 16 == 2
    q4.gemm(to_gpu(x), qw, out=y_un)
    assert torch.equal(y_al.view(torch.int16), y_un.view(torch.int16))
    q_o, s_o = oracle.quantize_sym(W, 128)
    assert_close(to_np(y_al), _ref_product(x, q_o, s_o, None, 128), f"split sum B={B} N={N} K={K}")


def test_gemm_empty_batch(q4):
    import torch

    qw = q4.quantize_pack(to_gpu(synth.weight(32, 128)), 128)
    y = q4.gemm(torch.empty((0, 128), dtype=torch.float16, device="cuda"), qw)
    assert tuple(y.shape) == (0, 32)


def _sampled_rows(N, n, seed):
    r = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, N - 1], r.choice(N, size=min(n, N), replace=False)]))
    return rows


def _full_size_check(q4, N, K, g, Bs, asym=False, seed=0, heavy=False, nrows=96):
    import torch

    W = synth.heavy_tailed_weight(N, K, seed=seed)[0] if heavy else synth.weight(N, K, seed=seed)
    Wg = to_gpu(W)
    qw = q4.quantize_pack(Wg, g, asym=asym)
    del Wg
    rows = _sampled_rows(N, nrows, seed + 1)
    if asym:
        q_o, s_o, z_o = oracle.quantize_asym(W[rows], g)
    else:
        (q_o, s_o), z_o = oracle.quantize_sym(W[rows], g), None
    c, s, z = q4.to_canonical(qw)
    assert np.array_equal(to_np(c[torch.from_numpy(rows).cuda()]), oracle.pack_canonical(q_o))
    assert np.array_equal(to_np(s[torch.from_numpy(rows).cuda()]).view(np.uint16), s_o.view(np.uint16))
    for B in Bs:
        x = synth.activation(B, K, seed=seed + B)
        y = to_np(q4.gemm(to_gpu(x), qw))
        ref = _ref_product(x, q_o, s_o, z_o, g)
        rel, mx = assert_close(y[:, rows], ref, f"N={N} K={K} g={g} B={B}")
        say(f"  N={N} K={K} g={g} B={B} asym={asym}: rel L2 {rel:.2e} max {mx:.2e}")


def test_full_single_layer_b1(q4):
    """4096x4096, B = 1: every output checked."""
    W = synth.weight(4096, 4096, seed=0)
    x = synth.activation(1, 4096, seed=0)
    qw, q_o, s_o, _ = _check_quant_exact(q4, W, 128, False, device_layout=False)
    y = to_np(q4.gemm(to_gpu(x), qw))
    rel, mx = assert_close(y, _ref_product(x, q_o, s_o, None, 128), "4096x4096 B=1")
    say(f"4096x4096 B=1 rel L2 {rel:.2e} max {mx:.2e}")


@pytest.mark.parametrize("name", list(synth.LLAMA3_70B))
def test_full_70b_shapes(q4, name):
    N, K = synth.LLAMA3_70B[name]
    say(f"70B {name} {N}x{K}")
    _full_size_check(q4, N, K, 128, (1, 2, 4, 8), seed=3)


@pytest.mark.parametrize("name", ["q_proj", "k_proj", "gate_proj", "down_proj"])
def test_full_8b_shapes(q4, name):
    N, K = synth.LLAMA3_8B[name]
    say(f"8B {name} {N}x{K}")
    _full_size_check(q4, N, K, 128, (1,), seed=2)


def test_full_batch_sweep_28672x8192(q4):
    say("28672x8192 batch sweep")
    _full_size_check(q4, 28672, 8192, 128, (1, 4, 16, 32, 48, 64, 96, 128, 192, 256), seed=4, nrows=64)


@pytest.mark.parametrize("N,K,Bs", [(8192, 28672, (5, 12, 17, 48, 80, 192)), (8192, 8192, (16, 192)),
                                    (6144, 4096, (144, 256)), (4096, 14336, (6, 32, 64)),
                                    (28672, 8192, (40, 96, 144))])
def test_full_launch_rules(q4, N, K, Bs):
    """Full-size matrices at the batch sizes where the launch-shape choices take their
    less common branches: the GEMV cost model's 8-way channel splits (down at B = 5, 12),
    and the skinny-GEMM model's 8-way splits of long rows (B = 17-192), groups of 3 and
    6 column tiles (B = 40-192) and short rows on 2 column tiles in several groups
    (6144x4096 at 144 and 256)."""
    say(f"launch rules {N}x{K} B={Bs} shapes {[q4.gemm_shape(B, N, K, 128) for B in Bs]}")
    _full_size_check(q4, N, K, 128, Bs, seed=N % 97, nrows=64)


def test_full_fused_gate_up_batches(q4):
    """The fused 70B gate/up matrix (57344x8192, device-generated weights) at B = 16,
    64, 128 and 256: B = 128 takes the wider column groups that keep its skinny-GEMM
    grid within one round of workgroups; codes, scales and products on sampled rows."""
    import torch

    N, K, g = 57344, 8192, 128
    say(f"fused gate/up {N}x{K} batches")
    Wd = synth.device_weight(N, K, seed=6, layer=0, matrix=0)
    qw = q4.quantize_pack(Wd, g)
    rows = _sampled_rows(N, 64, 7)
    W = to_np(Wd[torch.from_numpy(rows).cuda()])
    del Wd
    q_o, s_o = oracle.quantize_sym(W, g)
    c, sc, _ = q4.to_canonical(qw)
    assert np.array_equal(to_np(c[torch.from_numpy(rows).cuda()]), oracle.pack_canonical(q_o))
    assert np.array_equal(to_np(sc[torch.from_numpy(rows).cuda()]).view(np.uint16), s_o.view(np.uint16))
    for B in (16, 64, 128, 256):
        x = synth.activation(B, K, seed=B)
        y = to_np(q4.gemm(to_gpu(x), qw))
        rel, mx = assert_close(y[:, rows], _ref_product(x, q_o, s_o, None, g), f"gate/up B={B}")
        say(f"  B={B}: rel L2 {rel:.2e} max {mx:.2e}")


@pytest.mark.parametrize("asym", [False, True], ids=["sym", "asym"])
@pytest.mark.parametrize("g", [32, 64, 128])
def test_full_heavy_tailed_gemv(q4, g, asym):
    say(f"heavy-tailed GEMV g={g} asym={asym}")
    _full_size_check(q4, 14336, 4096, g, (1,), asym=asym, seed=5, heavy=True)


# Burst GEMVs. Staged, one row tile per wavefront (gemv_burst_kernel): units of one
# 4-block burst (4096x4096 and 6144x4096 at B <= 2, 8 chunks of 32 blocks) and of
# several (14336x4096 at B = 4). Streamed, two row tiles per wavefront
# (gemv_stream_burst_kernel: 8192x8192 at B = 1 and 4, one workgroup per CU). Each
# wavefront's first units are fixed and the LDS unit counter is read only after the
# barrier that follows its initialisation; a product that took a unit from an
# uninitialised counter would skip or repeat units. The products run repeatedly with
# a skinny GEMM between them (other data left in LDS) and must all give the bits of
# the first, which must match the oracle.
@pytest.mark.parametrize("N,K,B,R", [(4096, 4096, 1, 1), (4096, 4096, 2, 1), (6144, 4096, 1, 1), (14336, 4096, 4, 1),
                                     (8192, 8192, 1, 2), (8192, 8192, 4, 2)])
def test_burst_gemv_units_repeatable(q4, N, K, B, R):
    import torch

    say(f"burst GEMV N={N} K={K} B={B}")
    got = q4.gemm_shape(B, N, K, 128)
    assert (got[0], got[2], got[3]) == (R, 1, 1), got  # one split: the staged (R = 1) or streamed (R = 2) launch
    W_ = synth.weight(N, K, seed=31)
    x = synth.activation(B, K, seed=31)
    qw = q4.quantize_pack(to_gpu(W_), 128)
    q_o, s_o = oracle.quantize_sym(W_, 128)
    ref = oracle.gemm_ref(x, oracle.dequant_sym(q_o, s_o, 128))
    xg = to_gpu(x)
    other = q4.quantize_pack(to_gpu(synth.weight(1024, 2048, seed=32)), 128)
    xo = to_gpu(-np.abs(synth.activation(64, 2048, seed=32)))
    first = q4.gemm(xg, qw)
    assert_close(to_np(first), ref, f"burst GEMV {N}x{K} B={B}")
    for _ in range(8):
        q4.gemm(xo, other)
        y = q4.gemm(xg, qw)
        assert torch.equal(y, first), f"burst GEMV {N}x{K} B={B}: a repeated product differs"
