"""Benchmark of the W4A16 decode hot path on one MI355X.

Headline (one JSON line on stdout): effective HBM GB/s of the B = 1 W4A16 GEMV
over a full Llama-3-70B-shaped decode step -- 80 resident layers of INT4 g128
weights (q/k/v fused, o, gate/up fused, down: 320 launches), captured once in a
HIP graph and replayed. A "step" is one such sweep. Bytes counted per step are
the algorithmic bytes: packed codes + float16 scales + float16 activations
(outputs not counted). Inputs are synthetic and already resident in HBM.

The same line carries:
  roofline      the dominant kernel (gate/up GEMV) against the 8 TB/s HBM peak,
                its average duration measured with HIP events on its stream;
  cpu_baseline  the CPU oracle timed on a bounded sample (layer 0), on this host;
  extras        us/layer vs B (1, 2, 4, 8), the Llama-3-8B sweep, the batch sweep
                on one 28672x8192 matrix with a dense bf16 torch.matmul beside it,
                and quantize+pack throughput on the heavy-tailed 14336x4096 weights.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMV effective HBM GB/s & % of peak (B=1); us/layer vs B"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_sweep(shapes: dict, layers: int, seed: int, group: int, device):
    """Quantize every layer's fused matrices on the GPU; returns [(name, N, K, qw)] per layer."""
    import torch

    import synth
    import w4a16_decode_amd as q4

    order = {name: i for i, name in enumerate(synth.MATRIX_ORDER)}
    model = []
    for layer in range(layers):
        mats = []
        for grp in synth.FUSED_GROUPS:
            parts = [synth.device_weight(*shapes[n], seed=seed, layer=layer, matrix=order[n], device=device)
                     for n in grp]
            W = parts[0] if len(parts) == 1 else torch.cat(parts, dim=0)
            del parts
            qw = q4.quantize_pack(W, group)
            mats.append(("+".join(grp), W.shape[0], W.shape[1], qw))
            del W
        model.append(mats)
    torch.cuda.synchronize()
    return model


class Sweep:
    """One decode step: every fused matrix of every layer, B rows, outputs preallocated."""

    def __init__(self, model, B: int, seed: int, device):
        import torch

        import synth

        import w4a16_decode_amd as q4

        self.model = model
        self.B = B
        self.xs, self.ys = [], []
        ws = 0
        for layer, mats in enumerate(model):
            for i, (_, N, K, qw) in enumerate(mats):
                self.xs.append(synth.device_activation(B, K, seed=seed, layer=layer, matrix=100 + i, device=device))
                self.ys.append(torch.empty((B, N), dtype=torch.float16, device=device))
                ws = max(ws, q4.workspace_bytes(B, N, K, qw.group))
        # one scratch buffer shared by the launches (they run in stream order)
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=device)
        self.graph = None

    def launches(self):
        i = 0
        for mats in self.model:
            for (name, N, K, qw) in mats:
                yield name, self.xs[i], qw, self.ys[i]
                i += 1

    def run_eager(self):
        import w4a16_decode_amd as q4

        for _, x, qw, y in self.launches():
            q4.gemm(x, qw, out=y, workspace=self.ws)

    def capture(self):
        import torch

        self.run_eager()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run_eager()
        torch.cuda.synchronize()
        self.graph = g

    def bytes_per_step(self) -> int:
        from w4a16_decode_amd import perfmodel

        return sum(perfmodel.gemm_read_bytes(self.B, qw.out_features, qw.in_features, qw.group)
                   for _, _, qw, _ in self.launches())

    def time_steps(self, steps: int, warmup: int) -> float:
        """Seconds per step over `steps` graph replays (after `warmup`)."""
        import torch

        for _ in range(warmup):
            self.graph.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            self.graph.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / 1e3 / steps

    def time_kernel(self, pick: str, reps: int = 2):
        """Per-launch duration of the launches named `pick`, HIP events on their stream."""
        import torch

        import w4a16_decode_amd as q4

        stream = torch.cuda.current_stream()
        durs = []
        for _ in range(reps):
            evs = []
            for name, x, qw, y in self.launches():
                if name == pick:
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    q4.gemm(x, qw, out=y, workspace=self.ws)
                    b.record(stream)
                    evs.append((a, b, qw))
                else:
                    q4.gemm(x, qw, out=y, workspace=self.ws)
            torch.cuda.synchronize()
            durs += [(a.elapsed_time(b) / 1e3, qw) for a, b, qw in evs]
        return durs


def cpu_baseline(layers_W, B: int, group: int) -> dict:
    """Oracle (numpy) W4A16 product on a bounded sample, timed on this host's cores."""
    import numpy as np

    import oracle
    import synth
    from w4a16_decode_amd import perfmodel

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    total_bytes = 0
    t_total = 0.0
    for (N, K, W) in layers_W:
        x = synth.activation(B, K, seed=11)
        q, s = oracle.quantize_sym(W, group)            # setup, not timed
        t0 = time.perf_counter()
        y = oracle.gemm_ref(x, oracle.dequant_sym(q, s, group))
        t_total += time.perf_counter() - t0
        assert y.shape == (B, N) and np.all(np.isfinite(y))
        total_bytes += perfmodel.gemm_read_bytes(B, N, K, group)
    return {"seconds": t_total, "bytes": total_bytes, "threads": threads}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=80)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported in this build "
              "(the kernel shards by output rows, see the design notes)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    import w4a16_decode_amd as q4
    from w4a16_decode_amd import perfmodel

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    group = 128
    log(f"[bench] {q4.version()} on {torch.cuda.get_device_name(0)}")

    t_setup = time.perf_counter()
    model = build_sweep(synth.LLAMA3_70B, args.layers, seed=3, group=group, device=dev)
    log(f"[bench] quantized {args.layers} layers in {time.perf_counter() - t_setup:.1f}s, "
        f"{sum(qw.nbytes() for m in model for *_, qw in m) / 1e9:.2f} GB resident")

    sweep = Sweep(model, 1, seed=3, device=dev)
    sweep.capture()
    step_s = sweep.time_steps(args.steps, args.warmup)
    bytes_step = sweep.bytes_per_step()
    gbs = bytes_step / step_s / 1e9
    log(f"[bench] B=1 sweep: {step_s * 1e3:.3f} ms/step, {gbs:.1f} GB/s ({gbs / perfmodel.HBM_PEAK_GBS:.1%} of 8 TB/s)")

    # dominant kernel: the fused gate/up GEMV (55% of the bytes)
    durs = sweep.time_kernel("gate_proj+up_proj")
    d_avg = float(np.mean([d for d, _ in durs]))
    qw0 = durs[0][1]
    kbytes = perfmodel.gemm_read_bytes(1, qw0.out_features, qw0.in_features, group)
    k_gbs = kbytes / d_avg / 1e9
    log(f"[bench] gate/up GEMV {qw0.out_features}x{qw0.in_features}: {d_avg * 1e6:.2f} us, {k_gbs:.1f} GB/s")
    roofline = {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": perfmodel.HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_gbs / perfmodel.HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": f"gemm_kernel gate/up {qw0.out_features}x{qw0.in_features} B=1",
                "avg_us": round(d_avg * 1e6, 3), "bytes_per_launch": kbytes}

    extras = {}
    if not args.no_extras:
        per_layer = {}
        for B in (1, 2, 4, 8):
            sw = sweep if B == 1 else Sweep(model, B, seed=3, device=dev)
            if B != 1:
                sw.capture()
            t = sw.time_steps(max(5, args.steps // 2), 2)
            per_layer[str(B)] = {"us_per_layer": round(t / args.layers * 1e6, 2),
                                 "GBps": round(sw.bytes_per_step() / t / 1e9, 1)}
            if B != 1:
                del sw
        extras["us_per_layer_vs_B_70b"] = per_layer
        log(f"[bench] us/layer vs B: {per_layer}")
    del sweep

    cpu = None
    if not args.no_cpu:
        # bounded sample: layer 0 of the sweep, regenerated on the GPU and copied to the host
        order = {name: i for i, name in enumerate(synth.MATRIX_ORDER)}
        sample = []
        for grp in synth.FUSED_GROUPS:
            parts = [synth.device_weight(*synth.LLAMA3_70B[n], seed=3, layer=0, matrix=order[n], device=dev)
                     for n in grp]
            W = torch.cat(parts, 0) if len(parts) > 1 else parts[0]
            sample.append((W.shape[0], W.shape[1], W.cpu().numpy()))
            del W, parts
        res = cpu_baseline(sample, 1, group)
        cpu_gbs = res["bytes"] / res["seconds"] / 1e9
        cpu = {"value": round(cpu_gbs, 3), "unit": "GB/s", "cores": res["threads"], "kind": "oracle",
               "sample": "layer 0 of the 70B sweep (q/k/v, o, gate/up, down), B=1: float64 dequantize + "
                         f"numpy matmul, {res['seconds']:.1f} s"}
        log(f"[bench] cpu oracle: {cpu_gbs:.3f} GB/s over {res['seconds']:.1f}s")

    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "llama3-70b decode GEMV sweep, INT4 g128 symmetric, B=1",
                   "layers": args.layers, "batch": 1, "group": group,
                   "launches_per_step": 4 * args.layers, "fusion": "q/k/v and gate/up row-concatenated",
                   "bytes_per_step": bytes_step, "pct_of_hbm_peak": round(gbs / perfmodel.HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
