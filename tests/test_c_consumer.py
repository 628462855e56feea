"""libq4 from a plain C99 program (tests/c/q4_consumer.c): no C++, no torch.

The host part runs here; the GPU part allocates its own device buffers and stream
with the HIP runtime, runs quantize + canonical export + product, and its output
is compared with the oracle (codes and scales bit for bit, y within the output
tolerance).
"""

import os
import subprocess
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c"))
import build_consumer  # noqa: E402

BIN = build_consumer.BIN


def _binary():
    lib = os.path.join(os.path.dirname(HERE), "w4a16_decode_amd", "libq4.so")
    if not os.path.exists(lib):
        from w4a16_decode_amd import build

        build.build()
    if not os.path.exists(BIN) or os.path.getmtime(BIN) < os.path.getmtime(lib):
        build_consumer.build()
    return BIN


def test_c_consumer_host():
    p = subprocess.run([_binary(), "host"], capture_output=True, text=True, timeout=60)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "host ok" in p.stdout


@pytest.mark.gpu
def test_c_consumer_gpu(tmp_path):
    import oracle
    import synth
    from gpu_util import assert_close

    assert os.path.exists(BIN), "tests/c/q4_consumer is built by __graft_entry__.build()"
    for N, K, B, g in ((300, 1024, 4, 128), (40, 352, 33, 32)):
        W = synth.weight(N, K, seed=N)
        x = synth.activation(B, K, seed=K)
        inp, out = tmp_path / f"in_{N}.bin", tmp_path / f"out_{N}.bin"
        with open(inp, "wb") as f:
            f.write(np.array([N, K, B, g], dtype=np.int32).tobytes())
            f.write(W.tobytes())
            f.write(x.tobytes())
        p = subprocess.run([BIN, "gpu", str(inp), str(out)], capture_output=True, text=True, timeout=120)
        assert p.returncode == 0, p.stdout + p.stderr
        raw = open(out, "rb").read()
        nc, ns = N * K // 2, N * (K // g) * 2
        codes = np.frombuffer(raw[:nc], dtype=np.uint8).reshape(N, K // 2)
        scales = np.frombuffer(raw[nc:nc + ns], dtype=np.float16).reshape(N, K // g)
        y = np.frombuffer(raw[nc + ns:], dtype=np.float16).reshape(B, N)
        q_o, s_o = oracle.quantize_sym(W, g)
        assert np.array_equal(codes, oracle.pack_canonical(q_o))
        assert np.array_equal(scales.view(np.uint16), s_o.view(np.uint16))
        assert_close(y, oracle.gemm_ref(x, oracle.dequant_sym(q_o, s_o, g)), f"C consumer N={N} B={B}")
