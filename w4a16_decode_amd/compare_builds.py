"""Time two builds of libq4.so against each other, interleaved (GPU).

    python -m w4a16_decode_amd.compare_builds LIB_A LIB_B --batches 1,4,8 \
        --shapes 57344x8192,8192x28672 [--rounds 8] [--group 128] [--q8]

Both libraries are opened in one process (each through its own handle; the product
calls of this package are pointed at one or the other in turn). For every matrix
shape and batch size the script quantizes a few copies of a seeded weight (enough to
stream past the last-level cache), captures one HIP graph per library that runs the
product over every copy, warms the GPU up, and then replays the two graphs in
alternating order (A B, B A, B A, A B, ...) for the given number of rounds. It prints
the median time per launch of each build and the median and interquartile range of
the per-round differences A - B, and flags outputs that differ by more than 1e-3
relative L2 (two builds that sum in a different order differ at rounding level only),
and says whether the two outputs are bit-identical.

Interleaving matters on this hardware: the first graph timed after the GPU idles runs
1-4 us slow, and one kernel's time differs by up to +-1 us from one board to the next,
so separate before/after runs cannot resolve changes below a microsecond.
"""

from __future__ import annotations

import argparse
import ctypes
import os
import statistics
import sys


def _open(path: str):
    from . import _lib

    lib = ctypes.CDLL(os.path.abspath(path))
    for name, (res, args) in _lib.SIGNATURES.items():
        fn = getattr(lib, name, None)
        if fn is not None:
            fn.restype = res
            fn.argtypes = args
    return lib


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("lib_a")
    ap.add_argument("lib_b")
    ap.add_argument("--batches", default="1")
    ap.add_argument("--shapes", default="57344x8192")
    ap.add_argument("--rounds", type=int, default=8)
    ap.add_argument("--group", type=int, default=128)
    ap.add_argument("--q8", action="store_true", help="per-row INT8 codes (q8_quantize_pack / q8_gemm)")
    args = ap.parse_args(argv)

    import torch

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import synth  # noqa: E402  (the seeded input generators, a package at the repository root)

    from . import _lib, ops

    libs = {"A": _open(args.lib_a), "B": _open(args.lib_b)}
    dev = torch.device("cuda", 0)

    def use(name):
        _lib._lib = libs[name]

    def graph_of(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        return g

    def replay_time(g, reps=3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3 / reps

    warmed = False
    for shape in args.shapes.split(","):
        N, K = map(int, shape.split("x"))
        copies = max(2, min(16, int(1.0e9 // (N * K * 0.52))))
        use("A")
        copies = max(2, copies // 2) if args.q8 else copies  # INT8 codes are twice the bytes
        quant = ops.q8_quantize_pack if args.q8 else (lambda W: ops.quantize_pack(W, args.group))
        product = ops.q8_gemm if args.q8 else ops.gemm
        qws = [quant(synth.device_weight(N, K, seed=4, layer=c, matrix=0, device=dev)) for c in range(copies)]
        for B in (int(b) for b in args.batches.split(",")):
            x = synth.device_activation(B, K, seed=4, layer=0, matrix=0, device=dev)
            ys = {n: torch.empty((B, N), dtype=torch.float16, device=dev) for n in libs}
            wss = {n: torch.zeros(max(256, 8 * B * N * 4), dtype=torch.uint8, device=dev) for n in libs}
            graphs = {}
            for n in libs:
                use(n)
                graphs[n] = graph_of(lambda: [product(x, qw, out=ys[n], workspace=wss[n]) for qw in qws])
            if not warmed:
                for _ in range(60):
                    for n in libs:
                        graphs[n].replay()
                torch.cuda.synchronize()
                warmed = True
            ya, yb = ys["A"].float(), ys["B"].float()
            err = ((ya - yb).norm() / ya.norm().clamp_min(1e-30)).item()
            same = bool(torch.equal(ys["A"], ys["B"]))
            t = {n: [] for n in libs}
            for r in range(args.rounds):
                order = ("A", "B") if r % 2 == 0 else ("B", "A")
                if r % 4 >= 2:
                    order = order[::-1]
                for n in order:
                    t[n].append(replay_time(graphs[n]) / copies)
            d = sorted(a - b for a, b in zip(t["A"], t["B"]))
            flag = f"  !! outputs differ: rel L2 {err:.1e}" if err > 1e-3 else (
                "  (outputs bit-identical)" if same else f"  (outputs differ at rounding level: rel L2 {err:.1e})")
            print(f"{N}x{K} B={B:3d}: A {statistics.median(t['A']) * 1e6:7.2f}  B {statistics.median(t['B']) * 1e6:7.2f}"
                  f"  A-B {statistics.median(d) * 1e6:+6.2f} [{d[len(d) // 4] * 1e6:+.2f}, "
                  f"{d[(3 * len(d)) // 4] * 1e6:+.2f}] us{flag}", flush=True)
            del graphs
        del qws
        torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
