"""Launch-shape model of the skinny GEMM (B > 16): measure, fit, check.

For symmetric INT4 codes with one scale per block the host picks the skinny GEMM's
launch shape -- R row tiles per wavefront (1 or 2), KS channel splits (1, 2, 3, 4, 6
or 8) and CT column tiles of 16 batch rows per workgroup (2, 3, 4, 6 or 8), always 8
wavefronts per workgroup -- as the lowest value of a linear model of the busiest CU's
work (skinny_model_us in csrc/q4_api.cpp). This module holds the same model in Python,
the least-squares fit of its coefficients and the measurement that feeds the fit:

    python -m w4a16_decode_amd.tune_skinny fit [grid.jsonl ...]     # CPU: coefficients + regret
    python -m w4a16_decode_amd.tune_skinny grid OUT.jsonl [--shapes 28672x8192,...] [--batches 17,...]

`grid` (GPU) times every launch shape through q4_gemm_config from graph replays over
copies of the matrix (enough to stream past the 256 MB last-level cache; one line per
matrix and batch size: microseconds per shape "R:8:KS:CT", plus the library's own pick
under "old_rules" when the grid was taken); `fit` reads such lines -- by default
tuning/skinny_grid_mi355x.jsonl, measured on MI355X over 9 matrices and 16 batch sizes
-- and fits

    time = a*codes + b*codes*CT + c*staged + d*[KS > 1] + e*partials + f*codes/waves + g

with relative-error weights: codes = KiB of codes the busiest CU streams and
dequantizes (its workgroups x 8 wavefronts x R tiles x blocks per split), codes*CT
its MFMA work, staged = activation tile-blocks it stages into LDS, partials = MB of
float32 split partials written and reduced, codes/waves = codes per wavefront the CU
holds at once (latency that fewer resident wavefronts leave exposed). Column-tile
counts that would leave two or more 16-row tiles of one group empty are not
candidates. Regret is how much slower the model's pick is than the fastest measured
shape.
"""

from __future__ import annotations

import argparse
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
GRID = os.path.join(HERE, "tuning", "skinny_grid_mi355x.jsonl")
CANDIDATE_CT = (2, 3, 4, 6, 8)
CANDIDATE_R = (1, 2)
CANDIDATE_KS = (1, 2, 3, 4, 6, 8)
WAVES = 8
LDS_LIMIT = 160 * 1024
CUS = 256
ROW_PAD = 16  # halfs of padding per activation row in LDS


def chunk_blocks(CT: int) -> int:
    """Blocks of 128 channels per activation chunk (q4::mfma_chunk_blocks)."""
    return 2 if CT >= 4 else 8 // CT


def lds_bytes(CT: int) -> int:
    """LDS of one workgroup: two activation tiles of CT * 16 rows by one chunk."""
    return 2 * CT * 16 * (chunk_blocks(CT) * 128 + ROW_PAD) * 2


def per_cu_mi355x(R: int, CT: int) -> int:
    """Workgroups one MI355X CU holds at once: the kernels with one row tile per
    wavefront and at most 4 column tiles take 90-104 VGPRs and <= 68 KiB of LDS, so two
    8-wavefront workgroups fit; every other shape takes 122-242 VGPRs or > 100 KiB of
    LDS and runs one. The library asks the runtime instead (mfma_resident_per_cu)."""
    return 2 if R == 1 and CT <= 4 else 1


def shape_ok(R: int, KS: int, CT: int, S: int, lds_limit: int = LDS_LIMIT) -> bool:
    """mfma_shape_ok in csrc/q4_api.cpp for 8 wavefronts and one scale per block."""
    chunks = -(-S // chunk_blocks(CT))
    return R in CANDIDATE_R and CT in CANDIDATE_CT and 1 <= KS <= chunks and R * CT <= 16 and \
        lds_bytes(CT) <= lds_limit


def features(N: int, K: int, B: int, R: int, KS: int, CT: int, per_cu: int, cus: int = CUS):
    """The model's terms for one launch shape: [codes KiB, codes KiB x CT, staged
    tile-blocks, split, partials MB, codes KiB per resident wavefront, 1]."""
    T, S, t = -(-N // 16), -(-K // 128), -(-B // 16)
    nb = chunk_blocks(CT)
    cps = -(-(-(-S // nb)) // KS)
    nsb = min(S, cps * nb)
    G = -(-T // (8 * R)) * -(-t // CT) * KS
    wg = -(-G // cus)
    conc = min(wg, per_cu)
    codes = float(wg * 8 * R * nsb)
    partials = KS * B * N * 4 / 1e6 if KS > 1 else 0.0
    return [codes, codes * CT, float(wg * CT * nsb), 1.0 if KS > 1 else 0.0, partials, codes / (8 * conc), 1.0]


def candidates(B: int):
    """Launch shapes (R, KS, CT) in the host's order: column tiles, then row tiles, then
    splits, ascending (ties keep the first)."""
    t = -(-B // 16)
    for ct in CANDIDATE_CT:
        if ct > 2 and ct > t + 1:
            continue
        for r in CANDIDATE_R:
            for ks in CANDIDATE_KS:
                yield r, ks, ct


def pick(N: int, K: int, B: int, coef, lds_limit: int = LDS_LIMIT, cus: int = CUS, per_cu=per_cu_mi355x):
    """(R, W, KS, CT) of lowest modelled time, or None if no candidate fits."""
    import numpy as np

    S = -(-K // 128)
    best, out = None, None
    for r, ks, ct in candidates(B):
        if not shape_ok(r, ks, ct, S, lds_limit):
            continue
        t = float(np.dot(features(N, K, B, r, ks, ct, per_cu(r, ct), cus), coef))
        if best is None or t < best:
            best, out = t, (r, WAVES, ks, ct)
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
            if shape == "old_rules":
                continue
            R, W, KS, CT = map(int, shape.split(":"))
            out.append((r["N"], r["K"], r["B"], shape, us,
                        features(r["N"], r["K"], r["B"], R, KS, CT, per_cu_mi355x(R, CT))))
    return out


def fit(rows):
    import numpy as np

    sm = samples(rows)
    A = np.array([s[5] for s in sm])
    y = np.array([s[4] for s in sm])
    coef, *_ = np.linalg.lstsq(A / y[:, None], np.ones_like(y), rcond=None)
    return coef


def regret(rows, coef):
    """Per (matrix, batch): (model's pick, its time / fastest measured time - 1, its
    time / the old rules' time - 1 or None)."""
    import numpy as np

    groups = {}
    for s in samples(rows):
        groups.setdefault((s[0], s[1], s[2]), []).append((float(np.dot(s[5], coef)), s[4], s[3]))
    old = {(r["N"], r["K"], r["B"]): r["us"].get("old_rules") for r in rows}
    out = {}
    for key, lst in groups.items():
        best = min(t for _, t, _ in lst)
        p = min(lst)
        out[key] = (p[2], p[1] / best - 1.0, p[1] / old[key] - 1.0 if old.get(key) else None)
    return out


def run_grid(out_path: str, shapes, batches, group: int = 128, asym: bool = False) -> None:
    import torch

    sys.path.insert(0, os.path.dirname(HERE))
    import synth  # noqa: E402  (the seeded input generators, a package at the repository root)
    import w4a16_decode_amd as q4

    dev = torch.device("cuda", 0)

    def graph(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        return g

    def gtime(g, reps=3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3 / reps

    with open(out_path, "w") as out:
        for N, K in shapes:
            copies = min(32, max(2, -(-int(0.6e9) // int(N * K * 0.515625))))
            qws = [q4.quantize_pack(synth.device_weight(N, K, seed=4, layer=c, matrix=0, device=dev), group, asym)
                   for c in range(copies)]
            for B in batches:
                x = synth.device_activation(B, K, seed=4, layer=0, matrix=0, device=dev)
                y = torch.empty((B, N), dtype=torch.float16, device=dev)
                ws = torch.zeros(max(256, 8 * B * N * 4), dtype=torch.uint8, device=dev)
                graphs = {"old_rules": graph(lambda: [q4.gemm(x, qw, out=y, workspace=ws) for qw in qws])}
                for r, ks, ct in candidates(B):
                    try:
                        graphs[f"{r}:8:{ks}:{ct}"] = graph(
                            lambda: [q4.gemm_config(x, qw, r, 8, ks, ct, out=y, workspace=ws) for qw in qws])
                    except q4.Q4Error:
                        continue  # shape does not fit this matrix
                for _ in range(10):
                    graphs["old_rules"].replay()
                best = {k: 1e9 for k in graphs}
                for rnd in range(3):
                    items = list(graphs.items())
                    for k, g in (items if rnd % 2 == 0 else items[::-1]):
                        best[k] = min(best[k], gtime(g) / copies)
                row = {"N": N, "K": K, "B": B, "us": {k: round(v * 1e6, 2) for k, v in best.items()}}
                if group != 128 or asym:
                    row.update(group=group, asym=asym)
                out.write(json.dumps(row, separators=(",", ":")) + "\n")
                out.flush()
                print(f"{N}x{K} B={B}: {len(best)} shapes", flush=True)
                del graphs
            del qws
            torch.cuda.empty_cache()


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    f = sub.add_parser("fit")
    f.add_argument("grids", nargs="*", default=[GRID])
    g = sub.add_parser("grid")
    g.add_argument("out")
    g.add_argument("--shapes", default="28672x8192,8192x28672,57344x8192,10240x8192,8192x8192,4096x14336,"
                                        "6144x4096,14336x4096,28672x4096")
    g.add_argument("--batches", default="17,24,32,40,48,56,64,80,96,112,128,144,160,192,224,256")
    g.add_argument("--group", type=int, default=128)
    g.add_argument("--asym", action="store_true")
    args = ap.parse_args(argv)
    if args.cmd == "grid":
        shapes = [tuple(map(int, s.split("x"))) for s in args.shapes.split(",")]
        run_grid(args.out, shapes, [int(b) for b in args.batches.split(",")], args.group, args.asym)
        return 0
    rows = load(args.grids)
    coef = fit(rows)
    names = ["codes_kib", "codes_kib_x_ct", "staged_tile_blocks", "split", "partials_mb", "codes_kib_per_wave", "const"]
    for n, c in zip(names, coef):
        print(f"{n}: {c:.5g}")
    reg = regret(rows, coef)
    vals = [v[1] for v in reg.values()]
    olds = [v[2] for v in reg.values() if v[2] is not None]
    print(f"matrices x batches: {len(vals)}; regret mean {100 * sum(vals) / len(vals):.2f}%, "
          f"max {100 * max(vals):.1f}%")
    if olds:
        print(f"against the old rules: mean {100 * sum(olds) / len(olds):+.2f}%, worst {100 * max(olds):+.1f}%, "
              f"best {100 * min(olds):+.1f}%")
    return 0


if __name__ == "__main__":
    sys.exit(main())
