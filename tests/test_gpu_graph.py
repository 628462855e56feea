"""The library's calls inside HIP graphs (needs an MI355X).

Every call only enqueues kernels on the caller's stream (no allocation, no
memset, no synchronisation), so it can be captured. Each captured graph is
replayed several times with eager work and new inputs in between; every replay
must equal, bit for bit, an eager call on the same inputs (the kernels are
deterministic).
"""

import numpy as np
import pytest

import synth
from gpu_util import say, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_decode_amd as q4mod

    return q4mod


def _replays_match(run, x, fill_seeds):
    """Capture run() (which reads x and returns its output tensor), then for each seed:
    refill x eagerly, replay, and compare with an eager run on the same x."""
    import torch

    run()  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_graph = run()
    for seed in fill_seeds:
        gen = torch.Generator(device=x.device)
        gen.manual_seed(seed)
        x.copy_(torch.randn(x.shape, generator=gen, device=x.device, dtype=torch.float32).to(x.dtype))
        g.replay()
        torch.cuda.synchronize()
        got = y_graph.clone()
        want = run()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"replay with seed {seed} differs"


@pytest.mark.parametrize("B,N,K", [(1, 8192, 8192), (2, 8192, 8192), (3, 8192, 28672), (4, 300, 2048), (40, 256, 4096),
                                   (1, 512, 28672)])
def test_graph_q4_gemm(q4, B, N, K):
    import torch

    say(f"graph q4_gemm B={B} N={N} K={K}")
    qw = q4.quantize_pack(to_gpu(synth.weight(N, K, seed=B)), 128)
    x = to_gpu(synth.activation(B, K, seed=K))
    y = torch.empty((B, N), dtype=torch.float16, device="cuda")
    ws = torch.empty(max(16, q4.workspace_bytes(B, N, K, 128)), dtype=torch.uint8, device="cuda")
    _replays_match(lambda: q4.gemm(x, qw, out=y, workspace=ws), x, (1, 2, 3))


@pytest.mark.parametrize("B", [1, 64])
def test_graph_q8_gemm(q4, B):
    import torch

    N, K = 512, 4096
    qw = q4.q8_quantize_pack(to_gpu(synth.weight(N, K, seed=3)))
    x = to_gpu(synth.activation(B, K, seed=4))
    y = torch.empty((B, N), dtype=torch.float16, device="cuda")
    ws = torch.empty(max(16, q4.q8_workspace_bytes(B, N, K)), dtype=torch.uint8, device="cuda")
    _replays_match(lambda: q4.q8_gemm(x, qw, out=y, workspace=ws), x, (5, 6, 7))


def test_graph_actorder_gemm(q4):
    import torch

    N, K, g = 384, 2048, 128
    perm = q4.actorder_perm(np.random.default_rng(1).permutation(np.arange(K) // g), g)
    aw = q4.quantize_pack_perm(to_gpu(synth.weight(N, K, seed=5)), g, to_gpu(perm))
    for B in (1, 20):
        x = to_gpu(synth.activation(B, K, seed=B))
        y = torch.empty((B, N), dtype=torch.float16, device="cuda")
        ws = torch.empty(max(16, q4.workspace_bytes_perm(B, N, K, g)), dtype=torch.uint8, device="cuda")
        _replays_match(lambda: q4.gemm_perm(x, aw, out=y, workspace=ws), x, (8, 9, 10))


def test_graph_kv_append(q4):
    """One decode step's append captured once, replayed for new tokens at the same position."""
    import torch

    d, g = 128, 128
    cache = q4.kv_cache_alloc(16, 64, d, g)
    tok = torch.empty((2, 8, 1, d), dtype=torch.float16, device="cuda")

    def run():
        q4.kv_quantize_pack(tok, cache, 7)
        return q4.kv_dequant(cache, 7, 1)

    tok.copy_(to_gpu(synth.activation(16, d, seed=1).reshape(2, 8, 1, d)))
    _replays_match(run, tok, (11, 12, 13))
