"""Concurrent use of the library (needs an MI355X).

The calls keep no device state between them (scratch comes in the caller's
workspace) and guard their host-side caches with locks, so products launched on
several streams at once, and from several host threads, must equal the same
products run one after another, bit for bit (the kernels are deterministic).
"""

import threading

import pytest

import synth
from gpu_util import say, to_gpu

pytestmark = pytest.mark.gpu

SHAPES = [(1, 8192, 8192), (2, 8192, 28672), (4, 10240, 8192), (40, 4096, 4096), (1, 300, 3072)]


@pytest.fixture(scope="module")
def q4():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_decode_amd as q4mod

    return q4mod


def _cases(q4):
    import torch

    cases = []
    for i, (B, N, K) in enumerate(SHAPES):
        qw = q4.quantize_pack(to_gpu(synth.weight(N, K, seed=20 + i)), 128)
        x = to_gpu(synth.activation(B, K, seed=30 + i))
        ws = torch.empty(max(16, q4.workspace_bytes(B, N, K, 128)), dtype=torch.uint8, device="cuda")
        cases.append((x, qw, ws))
    return cases


def test_streams_match_sequential(q4):
    import torch

    say("products on several streams at once")
    cases = _cases(q4)
    want = [q4.gemm(x, qw, workspace=ws) for x, qw, ws in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    outs = [torch.empty_like(w) for w in want]
    for _ in range(3):
        for (x, qw, ws), s, y in zip(cases, streams, outs):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                q4.gemm(x, qw, out=y, workspace=ws)
        torch.cuda.synchronize()
        for y, w in zip(outs, want):
            assert torch.equal(y.view(torch.int16), w.view(torch.int16))


def test_threads_match_sequential(q4):
    import torch

    say("products from several host threads")
    cases = _cases(q4)
    want = [q4.gemm(x, qw, workspace=ws) for x, qw, ws in cases]
    torch.cuda.synchronize()
    outs = [torch.empty_like(w) for w in want]
    errors = []

    def run(i):
        try:
            x, qw, ws = cases[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(4):
                    q4.gemm(x, qw, out=outs[i], workspace=ws)
            s.synchronize()
        except Exception as ex:  # reported below
            errors.append(repr(ex))

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    torch.cuda.synchronize()
    for y, w in zip(outs, want):
        assert torch.equal(y.view(torch.int16), w.view(torch.int16))
