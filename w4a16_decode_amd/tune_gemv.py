"""Launch-shape model of the LDS-staged GEMV at 4 <= B <= 16: measure, fit, check.

The host picks the GEMV launch shape (R row tiles per wavefront, W wavefronts per
workgroup, KS channel splits) for 4 <= B <= 16, symmetric INT4 codes and one scale
per block, as the lowest value of a linear model of the busiest CU's work
(gemv_model_us in csrc/q4_api.cpp). This module holds the same model in Python, the
least-squares fit of its coefficients and the measurement that feeds the fit:

    python -m w4a16_decode_amd.tune_gemv fit [grid.jsonl ...]     # CPU: coefficients + regret
    python -m w4a16_decode_amd.tune_gemv grid OUT.jsonl [--shapes 8192x8192,...] [--batches 4,8,16]

`grid` (GPU) times every shape R in {1, 2}, W in {8, 16}, KS in {1, 2, 3, 4, 6, 8}
through q4_gemm_config from graph replays over copies of the matrix (one line per
matrix and batch size: microseconds per launch shape "R:W:KS"); `fit` reads such
lines -- by default tuning/gemv_grid_mi355x.jsonl, measured on MI355X -- and fits
time = a*codes + b*staged + c*[KS > 1] + d*partials + e*codes/waves + f with
relative-error weights over KS in {1, 2, 4, 8}; regret is how much slower the
model's pick is than the fastest measured shape.
"""

from __future__ import annotations

import argparse
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
GRID = os.path.join(HERE, "tuning", "gemv_grid_mi355x.jsonl")
CANDIDATE_KS = (1, 2, 4, 8)
LDS_LIMIT = 160 * 1024
CUS = 256
ROW_PAD = 16  # halfs of padding per activation row in LDS


def gemv_lds(B: int, S: int, KS: int, R: int) -> int:
    """LDS bytes of one GEMV workgroup with one unit (gemv_lds in csrc/q4_api.cpp,
    symmetric codes, one scale per block)."""
    nsb = -(-S // KS)
    x = ((B * (nsb * 128 + ROW_PAD) + 128) * 2 + 15) & ~15
    beta = (B * nsb + 1 + 3) // 4 * 4 * 4
    return x + beta + R * 16 * B * 4 + 16


def features(N: int, K: int, B: int, R: int, W: int, KS: int, lds_limit: int = LDS_LIMIT, cus: int = CUS):
    """The model's terms for one launch shape: [codes KiB, staged KiB, split, partials
    MB, codes KiB per wavefront, 1] of the busiest CU."""
    T, S = -(-N // 16), -(-K // 128)
    nRB = (T + R - 1) // R
    nsb = -(-S // KS)
    per_cu = max(1, min(16 // W, lds_limit // gemv_lds(B, S, KS, R)))
    per_split = max(1, min(nRB, per_cu * cus // KS))
    n_rb = -(-nRB // per_split)
    wgs_cu = -(-(per_split * KS) // cus)
    codes = n_rb * R * nsb * wgs_cu
    staged = B * nsb / 4.0 * wgs_cu
    split = 1.0 if KS > 1 else 0.0
    partials = KS * B * 16 * T * 4 / 1e6 if KS > 1 else 0.0
    return [float(codes), staged, split, partials, codes / (W * wgs_cu), 1.0]


def shape_ok(B: int, S: int, KS: int, R: int, W: int, lds_limit: int = LDS_LIMIT) -> bool:
    """gemv_shape_ok in csrc/q4_api.cpp (symmetric codes, one scale per block)."""
    nsb = -(-S // KS)
    return KS <= S and gemv_lds(B, S, KS, R) <= lds_limit and B * nsb * 16 <= 8 * W * 64


def pick(N: int, K: int, B: int, coef, lds_limit: int = LDS_LIMIT, cus: int = CUS):
    """The launch shape (R, W, KS) of lowest modelled time, in the host's order (ties
    keep fewer splits), or None if no candidate fits."""
    import numpy as np

    S = -(-K // 128)
    best, out = None, None
    for ks in CANDIDATE_KS:
        for r in (1, 2):
            for w in (8, 16):
                if not shape_ok(B, S, ks, r, w, lds_limit):
                    continue
                t = float(np.dot(features(N, K, B, r, w, ks, lds_limit, cus), coef))
                if best is None or t < best:
                    best, out = t, (r, w, ks)
    return out


def load(paths):
    rows = []
    for p in paths:
        with open(p) as f:
            rows += [json.loads(line) for line in f if line.strip()]
    return rows


def samples(rows):
    out = []
    for r in rows:
        for shape, us in r["us"].items():
            R, W, KS = map(int, shape.split(":"))
            if KS in CANDIDATE_KS:
                out.append((r["N"], r["K"], r["B"], shape, us, features(r["N"], r["K"], r["B"], R, W, KS)))
    return out


def fit(rows):
    import numpy as np

    sm = samples(rows)
    A = np.array([s[5] for s in sm])
    y = np.array([s[4] for s in sm])
    coef, *_ = np.linalg.lstsq(A / y[:, None], np.ones_like(y), rcond=None)
    return coef


def regret(rows, coef):
    """Per (matrix, batch): (model's pick, its time / fastest measured time - 1)."""
    import numpy as np

    groups = {}
    for s in samples(rows):
        groups.setdefault((s[0], s[1], s[2]), []).append((float(np.dot(s[5], coef)), s[4], s[3]))
    out = {}
    for key, lst in groups.items():
        best = min(t for _, t, _ in lst)
        pick = min(lst)
        out[key] = (pick[2], pick[1] / best - 1.0)
    return out


def run_grid(out_path: str, shapes, batches) -> None:
    import torch

    sys.path.insert(0, os.path.dirname(HERE))
    import synth  # noqa: E402  (the seeded input generators, a package at the repository root)
    import w4a16_decode_amd as q4

    dev = torch.device("cuda", 0)

    def gtime(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3 / reps

    shapes_all = [(r, w, ks) for r in (1, 2) for w in (8, 16) for ks in (1, 2, 3, 4, 6, 8)]
    with open(out_path, "w") as out:
        for N, K in shapes:
            copies = max(2, min(16, int(1.0e9 // (N * K * 0.52))))
            qws = [q4.quantize_pack(synth.device_weight(N, K, seed=4, layer=c, matrix=0, device=dev), 128)
                   for c in range(copies)]
            for B in batches:
                x = synth.device_activation(B, K, seed=4, layer=0, matrix=0, device=dev)
                y = torch.empty((B, N), dtype=torch.float16, device=dev)
                ws = torch.zeros(max(256, 8 * B * N * 4), dtype=torch.uint8, device=dev)
                best = {}
                for _ in range(2):
                    for (r, w, ks) in shapes_all:
                        try:
                            t = gtime(lambda: [q4.gemm_config(x, qw, r, w, ks, 1, out=y, workspace=ws) for qw in qws])
                        except q4.Q4Error:
                            continue  # shape does not fit this matrix and batch
                        k = f"{r}:{w}:{ks}"
                        best[k] = min(best.get(k, 1e9), t / copies)
                out.write(json.dumps({"N": N, "K": K, "B": B, "us": {k: round(v * 1e6, 2) for k, v in best.items()}},
                                     separators=(",", ":")) + "\n")
                out.flush()
                print(f"{N}x{K} B={B}: {len(best)} shapes", flush=True)
            del qws
            torch.cuda.empty_cache()


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    f = sub.add_parser("fit")
    f.add_argument("grids", nargs="*", default=[GRID])
    g = sub.add_parser("grid")
    g.add_argument("out")
    g.add_argument("--shapes", default="10240x8192,8192x8192,8192x28672,57344x8192")
    g.add_argument("--batches", default="4,5,6,8,12,16")
    args = ap.parse_args(argv)
    if args.cmd == "grid":
        shapes = [tuple(map(int, s.split("x"))) for s in args.shapes.split(",")]
        run_grid(args.out, shapes, [int(b) for b in args.batches.split(",")])
        return 0
    rows = load(args.grids)
    coef = fit(rows)
    names = ["codes_kib", "staged_kib", "split", "partials_mb", "codes_kib_per_wave", "const"]
    for n, c in zip(names, coef):
        print(f"{n}: {c:.5g}")
    reg = regret(rows, coef)
    vals = [v for _, v in reg.values()]
    print(f"matrices x batches: {len(vals)}; regret mean {100 * sum(vals) / len(vals):.2f}%, "
          f"max {100 * max(vals):.1f}%")
    return 0


if __name__ == "__main__":
    sys.exit(main())
