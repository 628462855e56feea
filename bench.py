"""Benchmark of the W4A16 decode hot path on one MI355X.

Headline (one JSON line on stdout): effective HBM GB/s of the B = 1 W4A16 GEMV
over a full Llama-3-70B-shaped decode step -- 80 resident layers of INT4 g128
weights (q/k/v fused, o, gate/up fused, down: 320 launches), captured once in a
HIP graph and replayed. A "step" is one such sweep. Bytes counted per step are
the algorithmic bytes: packed codes + float16 scales + float16 activations
(outputs not counted). Inputs are synthetic and already resident in HBM.

The same line carries:
  roofline      the dominant kernel (the fused gate/up GEMV, 55% of the bytes)
                against the 8 TB/s HBM peak; its average duration is measured
                with HIP events on its stream inside this run (the 80 layers'
                gate/up launches back to back in a HIP graph). `traffic` comes
                from the rocprofv3 FETCH_SIZE/WRITE_SIZE summary under profiles/
                when that was taken on the current kernel sources, else null.
  cpu_baseline  the CPU oracle (numpy float64) timed on a bounded sample of the
                same sweep on this host.
  extras        us/layer vs B (1, 2, 4, 8); the Llama-3-8B sweep; one 4096x4096
                layer; the batch sweep on one 28672x8192 matrix with MFMA
                utilisation and a dense bf16 torch.mm beside it; quantize+pack
                throughput and the B = 1 GEMV on heavy-tailed 14336x4096 weights.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]
Profiling helpers: --only-kernel {gate_up,down,qkv,o} [--batch B] [--reps N] runs just
that GEMV kind of a few 70B layers; --only-batch B [--reps N] runs the product on one
28672x8192 matrix at batch B; --only-quantize, --only-w8, --only-actorder, --only-kv
run just that extra measurement; --copy-calibration runs a 256 MiB device copy.
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
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemv_gate_up_70b_b1_traffic.txt")
STATS_PROFILE = os.path.join(ROOT, "profiles", "gemv_70b_sweep_b1_kernel_stats.txt")
KIND_OF = {"q_proj+k_proj+v_proj": "qkv", "o_proj": "o", "gate_proj+up_proj": "gate_up", "down_proj": "down"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def events():
    import torch

    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def graph_time(fn, reps: int = 3) -> float:
    """Seconds per replay of a HIP graph holding the launches `fn` makes."""
    import torch

    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    a, b = events()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3 / reps


def build_model(shapes: dict, layers: int, seed: int, group: int, device):
    """Quantize every layer's fused matrices on the GPU; returns [[(name, qw)]] per layer."""
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
            mats.append(("+".join(grp), q4.quantize_pack(W, group)))
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

        self.model, self.B = model, B
        self.xs, self.ys = [], []
        ws = 0
        for layer, mats in enumerate(model):
            for i, (_, qw) in enumerate(mats):
                K, N = qw.in_features, qw.out_features
                self.xs.append(synth.device_activation(B, K, seed=seed, layer=layer, matrix=100 + i, device=device))
                self.ys.append(torch.empty((B, N), dtype=torch.float16, device=device))
                ws = max(ws, q4.workspace_bytes(B, N, K, qw.group))
        # one scratch buffer shared by the launches (they run in stream order)
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=device)
        self.graph = None

    def launches(self):
        i = 0
        for mats in self.model:
            for name, qw in mats:
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

    def time_steps(self, steps: int, warmup: int, per_step: list | None = None) -> float:
        """Seconds per step over `steps` graph replays (after `warmup`). If `per_step`
        is given, each replay's own duration (events between replays, no extra
        synchronisation) is appended to it in seconds."""
        import torch

        for _ in range(warmup):
            self.graph.replay()
        torch.cuda.synchronize()
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        marks[0].record()
        for i in range(steps):
            self.graph.replay()
            marks[i + 1].record()
        torch.cuda.synchronize()
        if per_step is not None:
            per_step.extend(marks[i].elapsed_time(marks[i + 1]) / 1e3 for i in range(steps))
        return marks[0].elapsed_time(marks[steps]) / 1e3 / steps

    def time_kernel(self, pick: str, reps: int = 5):
        """Average duration of the launches named `pick` (one per layer, back to back in a
        HIP graph, so every launch streams a different layer's weights from HBM), from
        HIP events on the stream they run on. Returns (seconds, a QuantizedWeight of
        that kind, launches timed)."""
        import w4a16_decode_amd as q4

        picked = [(x, qw, y) for name, x, qw, y in self.launches() if name == pick]
        t = graph_time(lambda: [q4.gemm(x, qw, out=y, workspace=self.ws) for x, qw, y in picked], reps)
        return t / len(picked), picked[0][1], len(picked) * reps


def measured_read_gbs(dev) -> float:
    """HBM read rate of the library's plain streaming read probe (q4_read_probe) on 8
    rotating 256 MiB buffers of random bytes (2 GiB, past the 256 MB last-level
    cache), timed over graph replays."""
    import torch

    import w4a16_decode_amd as q4

    bufs = [torch.randint(-2**31, 2**31 - 1, (64 * 1024 * 1024,), dtype=torch.int32, device=dev) for _ in range(8)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    t = graph_time(lambda: [q4.read_probe(b, sink) for b in bufs], 5) / len(bufs)
    nbytes = bufs[0].numel() * 4
    del bufs
    return nbytes / t / 1e9


def recorded_value(path: str, key: str):
    """A `key: value` line of a summary under profiles/, only if that summary was taken
    on the current kernel sources (its kernel_fingerprint line matches)."""
    from w4a16_decode_amd import profiling

    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_fingerprint") != profiling.kernel_fingerprint():
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def recorded_traffic():
    """Traffic per launch from profiles/, only if taken on the current kernel sources."""
    return recorded_value(TRAFFIC_PROFILE, "bytes")


SWEEP_B = (1, 4, 16, 32, 48, 64, 96, 128, 192, 256)  # batch sizes of the 28672x8192 sweep


def extras_batch_sweep(dev, group: int, log_prefix="[bench]"):
    """28672x8192: W4A16 at B in {1,4,16,32,48,64,96,128,192,256} vs dense bf16 torch.mm,
    with the launch shape the library picks at each B."""
    import torch

    import synth
    import w4a16_decode_amd as q4
    from w4a16_decode_amd import perfmodel

    N, K = 28672, 8192
    copies = 10  # 10 x 121 MB rotate past the 256 MB last-level cache
    qws = []
    for c in range(copies):
        W = synth.device_weight(N, K, seed=4, layer=c, matrix=0, device=dev)
        qws.append(q4.quantize_pack(W, group))
        del W
    dense = []
    for c in range(3):  # 3 x 470 MB bf16, stored [K, N] so torch.mm needs no transpose
        dense.append(synth.device_weight(N, K, seed=4, layer=c, matrix=0, device=dev).to(torch.bfloat16).t().contiguous())
    out = {}
    for B in SWEEP_B:
        x = synth.device_activation(B, K, seed=4, layer=0, matrix=0, device=dev)
        y = torch.empty((B, N), dtype=torch.float16, device=dev)
        ws = torch.empty(max(16, q4.workspace_bytes(B, N, K, group)), dtype=torch.uint8, device=dev)
        t = graph_time(lambda: [q4.gemm(x, qw, out=y, workspace=ws) for qw in qws]) / copies
        xb = x.to(torch.bfloat16)
        for Wd in dense:
            torch.mm(xb, Wd)
        torch.cuda.synchronize()
        a, b = events()
        a.record()
        reps = 4
        for _ in range(reps):
            for Wd in dense:
                torch.mm(xb, Wd)
        b.record()
        torch.cuda.synchronize()
        td = a.elapsed_time(b) / 1e3 / (reps * len(dense))
        flops = perfmodel.gemm_flops(B, N, K)
        nbytes = perfmodel.gemm_read_bytes(B, N, K, group)
        out[str(B)] = {"us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1),
                       "pct_of_hbm_peak": round(nbytes / t / 1e9 / perfmodel.HBM_PEAK_GBS, 4),
                       "TFLOPs": round(flops / t / 1e12, 2),
                       "mfma_util": round(flops / t / 1e12 / perfmodel.MFMA_FP16_DENSE_TFLOPS, 4),
                       "bf16_dense_us": round(td * 1e6, 2), "speedup_vs_bf16": round(td / t, 3),
                       "launch_shape_R_W_KS_CT": list(q4.gemm_shape(B, N, K, group))}
        log(f"{log_prefix} 28672x8192 B={B}: {t * 1e6:.1f} us ({nbytes / t / 1e9:.0f} GB/s, "
            f"{flops / t / 1e12:.1f} TFLOP/s) vs bf16 mm {td * 1e6:.1f} us")
    crossover = next((int(b) for b, v in out.items() if v["speedup_vs_bf16"] < 1.0), None)
    return {"per_B": out, "first_B_slower_than_bf16": crossover}


def extras_quantize(dev):
    """Heavy-tailed 14336x4096: quantize+pack throughput and the B = 1 GEMV, g in {32, 64, 128};
    the clipping search's time and weight error against RTN."""
    import numpy as np
    import torch

    import synth
    import w4a16_decode_amd as q4
    from w4a16_decode_amd import perfmodel

    N, K = 14336, 4096
    Wh, _ = synth.heavy_tailed_weight(N, K, seed=5)
    base = torch.from_numpy(Wh).to(dev)
    Ws = [base] + [base.clone() for _ in range(7)]  # 8 x 117 MB rotate past the last-level cache
    x = synth.device_activation(1, K, seed=5, layer=0, matrix=0, device=dev)
    y = torch.empty((1, N), dtype=torch.float16, device=dev)
    out = {}
    for g in (32, 64, 128):
        for asym in (False, True):
            qws = [q4.quantize_pack(W, g, asym=asym) for W in Ws]
            torch.cuda.synchronize()
            # the quantizer's launches captured in a HIP graph (into the buffers of qws)
            tq = graph_time(lambda: [q4.quantize_pack_into(W, qw) for W, qw in zip(Ws, qws)], 3) / len(Ws)
            ws = torch.empty(max(16, q4.workspace_bytes(1, N, K, g)), dtype=torch.uint8, device=dev)
            tg = graph_time(lambda: [q4.gemm(x, qw, out=y, workspace=ws) for qw in qws]) / len(qws)
            qb = perfmodel.quantize_bytes(N, K, g, asym)
            gb = perfmodel.gemm_read_bytes(1, N, K, g, asym)
            out[f"g{g}_{'asym' if asym else 'sym'}"] = {
                "quantize_us": round(tq * 1e6, 2), "quantize_GBps": round(qb / tq / 1e9, 1),
                "gemv_us": round(tg * 1e6, 2), "gemv_GBps": round(gb / tg / 1e9, 1)}
            del qws
        # clipping search (alpha = 0.80 .. 1.00 of the group amax): time, and the weight
        # reconstruction error against RTN's (dequantized from the library's own codes)
        qcs = [q4.quantize_pack_clip(W, g, 80) for W in Ws[:4]]
        tc = graph_time(lambda: [q4.quantize_pack_clip_into(W, qc, 80) for W, qc in zip(Ws[:4], qcs)], 2) / 4
        qc = qcs[0]
        qr = q4.quantize_pack(base, g)
        mse = {}
        for name, qw in (("rtn", qr), ("clip", qc)):
            codes, scales, _ = q4.to_canonical(qw)
            c = codes.cpu().numpy()
            lo = (c & 0xF).astype(np.int8)
            hi = (c >> 4).astype(np.int8)
            q = np.empty((N, K), dtype=np.int8)
            q[:, 0::2] = np.where(lo > 7, lo - 16, lo)
            q[:, 1::2] = np.where(hi > 7, hi - 16, hi)
            w_hat = q.astype(np.float32) * np.repeat(scales.cpu().numpy().astype(np.float32), g, axis=1)
            mse[name] = float(np.mean((w_hat - Wh.astype(np.float32)) ** 2))
        out[f"g{g}_sym_clip80"] = {"quantize_us": round(tc * 1e6, 2),
                                   "quantize_GBps": round(perfmodel.quantize_bytes(N, K, g, False) / tc / 1e9, 1),
                                   "weight_mse": mse["clip"], "weight_mse_rtn": mse["rtn"],
                                   "mse_ratio": round(mse["clip"] / mse["rtn"], 4)}
    return out


def extras_w8(dev, int4_us_per_layer: float | None):
    """W8A16 (per-channel INT8) product on the 70B layer's fused matrices at B in {1, 4, 8, 64}:
    per-launch time and GB/s (copies of each matrix rotate past the 256 MB last-level
    cache), the layer total against the INT4 layer, and the INT8 quantizer's time."""
    import torch

    import synth
    import w4a16_decode_amd as q4
    from w4a16_decode_amd import perfmodel

    order = {name: i for i, name in enumerate(synth.MATRIX_ORDER)}
    out = {}
    per_layer = {}
    for grp in synth.FUSED_GROUPS:
        N = sum(synth.LLAMA3_70B[n][0] for n in grp)
        K = synth.LLAMA3_70B[grp[0]][1]
        copies = max(2, -(-600_000_000 // (N * K)))
        qws = []
        for c in range(copies):
            parts = [synth.device_weight(*synth.LLAMA3_70B[n], seed=3, layer=c, matrix=order[n], device=dev)
                     for n in grp]
            W = parts[0] if len(parts) == 1 else torch.cat(parts, dim=0)
            del parts
            if c == 0:  # the quantizer's time on this matrix
                q4.q8_quantize_pack(W)
                torch.cuda.synchronize()
                a, b = events()
                a.record()
                for _ in range(3):
                    q4.q8_quantize_pack(W)
                b.record()
                torch.cuda.synchronize()
                tq = a.elapsed_time(b) / 1e3 / 3
            qws.append(q4.q8_quantize_pack(W))
            del W
        kind = KIND_OF["+".join(grp)]
        res = {"shape": [N, K], "quantize_us": round(tq * 1e6, 2),
               "quantize_GBps": round((2 * N * K + perfmodel.w8_weight_bytes(N, K)) / tq / 1e9, 1)}
        for B in (1, 4, 8, 64):
            x = synth.device_activation(B, K, seed=3, layer=0, matrix=100, device=dev)
            y = torch.empty((B, N), dtype=torch.float16, device=dev)
            ws = torch.empty(max(16, q4.q8_workspace_bytes(B, N, K)), dtype=torch.uint8, device=dev)
            t = graph_time(lambda: [q4.q8_gemm(x, qw, out=y, workspace=ws) for qw in qws], 5) / copies
            nb = perfmodel.w8_gemm_read_bytes(B, N, K)
            res[f"B{B}"] = {"us": round(t * 1e6, 2), "GBps": round(nb / t / 1e9, 1)}
            per_layer[B] = per_layer.get(B, 0.0) + t
        out[kind] = res
        log(f"[bench] W8A16 {kind} {N}x{K}: {res}")
        del qws
        torch.cuda.empty_cache()
    out["us_per_layer"] = {str(B): round(t * 1e6, 2) for B, t in per_layer.items()}
    if int4_us_per_layer:
        out["vs_int4_layer_b1"] = round(per_layer[1] * 1e6 / int4_us_per_layer, 3)
    return out


def extras_actorder(dev, group: int):
    """Act-order (g_idx) INT4 weights on the 70B layer's fused matrices: the product with
    x gathered through perm against the plain product on the same shape, B in {1, 4, 32},
    and the quantizer reading the columns through perm."""
    import numpy as np
    import torch

    import synth
    import w4a16_decode_amd as q4
    from w4a16_decode_amd import perfmodel

    order = {name: i for i, name in enumerate(synth.MATRIX_ORDER)}
    out = {}
    for grp in synth.FUSED_GROUPS:
        N = sum(synth.LLAMA3_70B[n][0] for n in grp)
        K = synth.LLAMA3_70B[grp[0]][1]
        copies = max(2, -(-300_000_000 // perfmodel.gemm_read_bytes(1, N, K, group)))
        # a synthetic g_idx: every group gets `group` channels drawn at random
        g_idx = np.random.default_rng(K).permutation(np.arange(K) // group).astype(np.int32)
        perm = torch.from_numpy(q4.actorder_perm(g_idx, group)).to(dev)
        plain, ao = [], []
        for c in range(copies):
            parts = [synth.device_weight(*synth.LLAMA3_70B[n], seed=3, layer=c, matrix=order[n], device=dev)
                     for n in grp]
            W = parts[0] if len(parts) == 1 else torch.cat(parts, dim=0)
            del parts
            plain.append(q4.quantize_pack(W, group))
            if c == 0:
                q4.quantize_pack_perm(W, group, perm)
                torch.cuda.synchronize()
                a, b = events()
                a.record()
                for _ in range(3):
                    q4.quantize_pack_perm(W, group, perm)
                b.record()
                torch.cuda.synchronize()
                tq = a.elapsed_time(b) / 1e3 / 3
            ao.append(q4.quantize_pack_perm(W, group, perm))
            del W
        kind = KIND_OF["+".join(grp)]
        res = {"shape": [N, K], "quantize_perm_us": round(tq * 1e6, 2)}
        for B in (1, 4, 32):
            x = synth.device_activation(B, K, seed=3, layer=0, matrix=100, device=dev)
            y = torch.empty((B, N), dtype=torch.float16, device=dev)
            ws = torch.empty(max(16, q4.workspace_bytes(B, N, K, group)), dtype=torch.uint8, device=dev)
            wsp = torch.empty(max(16, q4.workspace_bytes_perm(B, N, K, group)), dtype=torch.uint8, device=dev)
            t0 = graph_time(lambda: [q4.gemm(x, qw, out=y, workspace=ws) for qw in plain], 5) / copies
            t1 = graph_time(lambda: [q4.gemm_perm(x, aw, out=y, workspace=wsp) for aw in ao], 5) / copies
            res[f"B{B}"] = {"plain_us": round(t0 * 1e6, 2), "actorder_us": round(t1 * 1e6, 2),
                            "gather_cost_us": round((t1 - t0) * 1e6, 2)}
        out[kind] = res
        log(f"[bench] act-order {kind} {N}x{K}: {res}")
        del plain, ao
        torch.cuda.empty_cache()
    return out


def extras_kv(dev):
    """INT4 KV cache (group 128 = head_dim): one Llama-3-70B layer's K (8 KV heads x 128)
    quantized for a 32768-token prompt, and one decode step's append at B in {1, 16}."""
    import torch

    import synth
    import w4a16_decode_amd as q4

    h, d, g, S = 8, 128, 128, 32768
    out = {}
    src = synth.device_activation(h * S, d, seed=7, layer=0, matrix=0, device=dev).view(1, h, S, d)
    caches = [q4.kv_cache_alloc(h, S, d, g, device=dev) for _ in range(4)]
    t = graph_time(lambda: [q4.kv_quantize_pack(src, c, 0) for c in caches], 5) / len(caches)
    elems = h * S * d
    nbytes = elems * 2 + elems // 2 + (elems // g) * 2
    out["prefill_32k_one_layer_K"] = {"us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1)}
    for B in (1, 16):
        tok = synth.device_activation(B * h, d, seed=8, layer=0, matrix=0, device=dev).view(B, h, 1, d)
        cs = [q4.kv_cache_alloc(B * h, 4096, d, g, device=dev) for _ in range(8)]
        t = graph_time(lambda: [q4.kv_quantize_pack(tok, c, 4000) for c in cs], 5) / len(cs)
        out[f"append_B{B}_one_layer_K"] = {"us": round(t * 1e6, 2)}
    log(f"[bench] INT4 KV cache: {out}")
    return out


def cpu_baseline(dev, group: int, target_s: float = 8.0, max_layers: int = 12) -> dict:
    """Oracle (numpy) W4A16 product on whole layers of the 70B sweep, until ~target_s of CPU time."""
    import numpy as np
    import torch

    import oracle
    import synth
    from w4a16_decode_amd import perfmodel

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    order = {name: i for i, name in enumerate(synth.MATRIX_ORDER)}
    total_bytes, t_total, t_deq, t_mm, layers = 0, 0.0, 0.0, 0.0, 0
    t_q, q_bytes = 0.0, 0
    while t_total < target_s and layers < max_layers:
        for gi, grp in enumerate(synth.FUSED_GROUPS):
            parts = [synth.device_weight(*synth.LLAMA3_70B[n], seed=3, layer=layers, matrix=order[n], device=dev)
                     for n in grp]
            W = (torch.cat(parts, 0) if len(parts) > 1 else parts[0]).cpu().numpy()
            del parts
            N, K = W.shape
            x = synth.activation(1, K, seed=11, layer=layers)
            t0 = time.perf_counter()
            q, s = oracle.quantize_sym(W, group)  # timed on the first layer's q/k/v only
            if layers == 0 and gi == 0:
                t_q = time.perf_counter() - t0
                q_bytes = perfmodel.quantize_bytes(N, K, group)
            del W
            t0 = time.perf_counter()
            wh = oracle.dequant_sym(q, s, group)
            t1 = time.perf_counter()
            yy = oracle.gemm_ref(x, wh)
            t2 = time.perf_counter()
            t_deq += t1 - t0
            t_mm += t2 - t1
            t_total += t2 - t0
            assert yy.shape == (1, N) and np.all(np.isfinite(yy))
            total_bytes += perfmodel.gemm_read_bytes(1, N, K, group)
        layers += 1
    return {"seconds": t_total, "bytes": total_bytes, "threads": threads, "layers": layers,
            "dequant_s": t_deq, "matmul_s": t_mm, "quantize_s": t_q, "quantize_bytes": q_bytes}


def cpu_configs(dev, group: int) -> dict:
    """The oracle on the other workloads, in full: the 4096x4096 layer at B=1, the 28672x8192
    batch sweep (one float64 dequantization, then the matmul at every B) and the heavy-tailed
    14336x4096 quantizer at g = 32/64/128, symmetric and asymmetric. Seconds and GB/s on the
    same byte formulas as the GPU figures."""
    import numpy as np

    import oracle
    import synth
    from w4a16_decode_amd import perfmodel

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    out = {}
    W1 = synth.weight(4096, 4096, seed=0)
    x1 = synth.activation(1, 4096, seed=0)
    (q, s), tq = timed(lambda: oracle.quantize_sym(W1, group))
    wh, td = timed(lambda: oracle.dequant_sym(q, s, group))
    _, tm = timed(lambda: oracle.gemm_ref(x1, wh))
    nb = perfmodel.gemm_read_bytes(1, 4096, 4096, group)
    out["single_layer_4096_b1"] = {"quantize_s": round(tq, 3), "dequant_s": round(td, 3), "matmul_s": round(tm, 4),
                                   "gemv_GBps": round(nb / (td + tm) / 1e9, 3)}
    N, K = 28672, 8192
    W4 = synth.device_weight(N, K, seed=4, layer=0, matrix=0, device=dev).cpu().numpy()
    (q, s), tq = timed(lambda: oracle.quantize_sym(W4, group))
    del W4
    wh, td = timed(lambda: oracle.dequant_sym(q, s, group))
    del q, s
    per_b = {}
    for B in SWEEP_B:
        x = synth.activation(B, K, seed=4)
        y, tm = timed(lambda: oracle.gemm_ref(x, wh))
        assert np.all(np.isfinite(y))
        per_b[str(B)] = {"matmul_s": round(tm, 4),
                         "GBps_with_dequant": round(perfmodel.gemm_read_bytes(B, N, K, group) / (td + tm) / 1e9, 3),
                         "GFLOPs_matmul": round(perfmodel.gemm_flops(B, N, K) / tm / 1e9, 1)}
    del wh
    out["batch_sweep_28672x8192"] = {"quantize_s": round(tq, 2), "dequant_s": round(td, 2), "per_B": per_b}
    Wh, _ = synth.heavy_tailed_weight(14336, 4096, seed=5)
    hq = {}
    for g in (32, 64, 128):
        for asym in (False, True):
            _, tq = timed(lambda: oracle.quantize_asym(Wh, g) if asym else oracle.quantize_sym(Wh, g))
            hq[f"g{g}_{'asym' if asym else 'sym'}"] = {
                "quantize_s": round(tq, 3),
                "quantize_GBps": round(perfmodel.quantize_bytes(14336, 4096, g, asym) / tq / 1e9, 3)}
    out["heavy_tailed_14336x4096_quantize"] = hq
    return out


def only_kernel(kind: str, reps: int, layers: int, dev, group: int, batch: int = 1):
    """Run just one GEMV kind of a few 70B layers at `batch` rows, for counter collection."""
    import torch

    import synth
    import w4a16_decode_amd as q4

    model = build_model(synth.LLAMA3_70B, layers, seed=3, group=group, device=dev)
    sweep = Sweep(model, batch, seed=3, device=dev)
    picked = [(x, qw, y) for name, x, qw, y in sweep.launches() if KIND_OF[name] == kind]
    for _ in range(reps):
        for x, qw, y in picked:
            q4.gemm(x, qw, out=y, workspace=sweep.ws)
    torch.cuda.synchronize()
    log(f"[bench] ran {kind} B={batch} x {reps * len(picked)}")


def only_batch(B: int, reps: int, dev, group: int):
    """Run the W4A16 product on one 28672x8192 matrix at batch B, for counter collection."""
    import torch

    import synth
    import w4a16_decode_amd as q4

    N, K = 28672, 8192
    qw = q4.quantize_pack(synth.device_weight(N, K, seed=4, layer=0, matrix=0, device=dev), group)
    x = synth.device_activation(B, K, seed=4, layer=0, matrix=0, device=dev)
    y = torch.empty((B, N), dtype=torch.float16, device=dev)
    ws = torch.empty(max(16, q4.workspace_bytes(B, N, K, group)), dtype=torch.uint8, device=dev)
    for _ in range(reps):
        q4.gemm(x, qw, out=y, workspace=ws)
    torch.cuda.synchronize()
    log(f"[bench] ran 28672x8192 B={B} x {reps}")


def copy_calibration(dev):
    import torch

    a = torch.ones(128 * 1024 * 1024, dtype=torch.float16, device=dev)  # 256 MiB
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("[bench] copied 3 x 256 MiB (268435456 bytes read and written per copy)")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=80)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only-kernel", choices=["gate_up", "down", "qkv", "o"])
    ap.add_argument("--only-batch", type=int, default=0)
    ap.add_argument("--batch", type=int, default=1, help="batch rows for --only-kernel")
    ap.add_argument("--only-w8", action="store_true", help="only the W8A16 layer measurement")
    ap.add_argument("--only-actorder", action="store_true", help="only the act-order layer measurement")
    ap.add_argument("--only-kv", action="store_true", help="only the INT4 KV-cache measurement")
    ap.add_argument("--only-quantize", action="store_true", help="only the heavy-tailed quantizer measurement")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the library has no "
              "multi-GPU path (the GEMV would shard by output rows)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    import w4a16_decode_amd as q4
    from w4a16_decode_amd import perfmodel

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    group = 128
    if args.copy_calibration:
        copy_calibration(dev)
        return 0
    if args.only_kernel:
        only_kernel(args.only_kernel, args.reps, min(args.layers, 4), dev, group, args.batch)
        return 0
    if args.only_batch:
        only_batch(args.only_batch, args.reps, dev, group)
        return 0
    if args.only_w8:
        log(f"[bench] W8A16: {json.dumps(extras_w8(dev, None))}")
        return 0
    if args.only_actorder:
        log(f"[bench] act-order: {json.dumps(extras_actorder(dev, group))}")
        return 0
    if args.only_kv:
        extras_kv(dev)
        return 0
    if args.only_quantize:
        log(f"[bench] quantize: {json.dumps(extras_quantize(dev))}")
        return 0

    log(f"[bench] {q4.version()} on {torch.cuda.get_device_name(0)}")
    t_setup = time.perf_counter()
    model = build_model(synth.LLAMA3_70B, args.layers, seed=3, group=group, device=dev)
    log(f"[bench] quantized {args.layers} layers in {time.perf_counter() - t_setup:.1f}s, "
        f"{sum(qw.nbytes() for m in model for _, qw in m) / 1e9:.2f} GB resident")

    sweep = Sweep(model, 1, seed=3, device=dev)
    sweep.capture()
    per_step = []
    step_s = sweep.time_steps(args.steps, args.warmup, per_step)
    pct = np.percentile(np.array(per_step) * 1e3, [10, 50, 90])
    bytes_step = sweep.bytes_per_step()
    gbs = bytes_step / step_s / 1e9
    log(f"[bench] B=1 sweep: {step_s * 1e3:.3f} ms/step, {gbs:.1f} GB/s ({gbs / perfmodel.HBM_PEAK_GBS:.1%} of 8 TB/s)")

    # dominant kernel: the fused gate/up GEMV (55% of the bytes), HIP events on its stream
    d_avg, qw0, n_timed = sweep.time_kernel("gate_proj+up_proj")
    kbytes = perfmodel.gemm_read_bytes(1, qw0.out_features, qw0.in_features, group)
    k_gbs = kbytes / d_avg / 1e9
    log(f"[bench] gate/up GEMV {qw0.out_features}x{qw0.in_features}: {d_avg * 1e6:.2f} us, {k_gbs:.1f} GB/s")
    traffic = recorded_traffic()
    read_gbs = measured_read_gbs(dev)
    log(f"[bench] read probe: {read_gbs:.1f} GB/s; gate/up at {k_gbs / read_gbs:.1%} of it")
    roofline = {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": perfmodel.HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_gbs / perfmodel.HBM_PEAK_GBS, 4),
                "traffic": round(traffic) if traffic is not None else None,
                "measured_read_GBps": round(read_gbs, 1), "frac_of_measured_read": round(k_gbs / read_gbs, 4),
                "kernel": f"gemv_burst_kernel, fused gate/up {qw0.out_features}x{qw0.in_features}, B=1, g=128",
                "avg_us": round(d_avg * 1e6, 3), "bytes_per_launch": kbytes, "launches_timed": n_timed}
    # the same kernel's average duration in the committed rocprofv3 kernel trace of this command
    # (its summary under profiles/, while the kernel sources match): the two must agree
    prof_us = recorded_value(STATS_PROFILE, "gate_up_avg_us_rocprof")
    roofline["avg_us_rocprof"] = prof_us
    roofline["rocprof_over_events"] = round(prof_us / (d_avg * 1e6), 4) if prof_us else None

    extras = {}
    if not args.no_extras:
        # every matrix kind of the layer at B = 1, timed like the roofline kernel (its 80
        # launches back to back in a HIP graph), each against the 8 TB/s peak and the read probe
        per_matrix = {}
        for name, kind in KIND_OF.items():
            d, qwk, _ = sweep.time_kernel(name)
            nb = perfmodel.gemm_read_bytes(1, qwk.out_features, qwk.in_features, group)
            per_matrix[kind] = {"shape": [qwk.out_features, qwk.in_features], "us": round(d * 1e6, 2),
                                "GBps": round(nb / d / 1e9, 1),
                                "pct_of_hbm_peak": round(nb / d / 1e9 / perfmodel.HBM_PEAK_GBS, 4),
                                "frac_of_measured_read": round(nb / d / 1e9 / read_gbs, 4)}
        extras["per_matrix_b1_70b"] = per_matrix
        log(f"[bench] per matrix at B=1: {per_matrix}")
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
    del sweep, model
    torch.cuda.empty_cache()

    if not args.no_extras:
        m8 = build_model(synth.LLAMA3_8B, 32, seed=2, group=group, device=dev)
        s8 = Sweep(m8, 1, seed=2, device=dev)
        s8.capture()
        t8 = s8.time_steps(args.steps, args.warmup)
        per_matrix8 = {}
        for name, kind in KIND_OF.items():
            d, qwk, _ = s8.time_kernel(name)
            nb = perfmodel.gemm_read_bytes(1, qwk.out_features, qwk.in_features, group)
            per_matrix8[kind] = {"shape": [qwk.out_features, qwk.in_features], "us": round(d * 1e6, 2),
                                 "GBps": round(nb / d / 1e9, 1),
                                 "pct_of_hbm_peak": round(nb / d / 1e9 / perfmodel.HBM_PEAK_GBS, 4)}
        extras["sweep_8b_b1"] = {"ms_per_step": round(t8 * 1e3, 4), "GBps": round(s8.bytes_per_step() / t8 / 1e9, 1),
                                 "pct_of_hbm_peak": round(s8.bytes_per_step() / t8 / 1e9 / perfmodel.HBM_PEAK_GBS, 4),
                                 "us_per_layer": round(t8 / 32 * 1e6, 2), "per_matrix": per_matrix8}
        log(f"[bench] 8B sweep: {extras['sweep_8b_b1']}")
        del s8, m8

        W1 = synth.device_weight(4096, 4096, seed=0, layer=0, matrix=0, device=dev)
        qws = [q4.quantize_pack(W1, group)] + [q4.quantize_pack(synth.device_weight(4096, 4096, seed=0, layer=c,
                                                                                  matrix=0, device=dev), group)
                                              for c in range(1, 128)]
        x1 = synth.device_activation(1, 4096, seed=0, layer=0, matrix=0, device=dev)
        y1 = torch.empty((1, 4096), dtype=torch.float16, device=dev)
        t1 = graph_time(lambda: [q4.gemm(x1, qw, out=y1) for qw in qws]) / len(qws)
        b1 = perfmodel.gemm_read_bytes(1, 4096, 4096, group)
        extras["single_layer_4096_b1"] = {"us": round(t1 * 1e6, 3), "GBps": round(b1 / t1 / 1e9, 1)}
        log(f"[bench] 4096x4096 B=1: {extras['single_layer_4096_b1']}")
        del qws, W1
        torch.cuda.empty_cache()

        extras["batch_sweep_28672x8192"] = extras_batch_sweep(dev, group)
        torch.cuda.empty_cache()
        extras["heavy_tailed_14336x4096"] = extras_quantize(dev)
        log(f"[bench] heavy-tailed: {extras['heavy_tailed_14336x4096']}")
        torch.cuda.empty_cache()
        int4_layer = extras.get("us_per_layer_vs_B_70b", {}).get("1", {}).get("us_per_layer")
        extras["w8a16_70b_layer"] = extras_w8(dev, int4_layer)
        torch.cuda.empty_cache()
        extras["actorder_70b_layer"] = extras_actorder(dev, group)
        torch.cuda.empty_cache()
        extras["kv_int4_70b"] = extras_kv(dev)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        res = cpu_baseline(dev, group)
        cpu_gbs = res["bytes"] / res["seconds"] / 1e9
        cpu = {"value": round(cpu_gbs, 3), "unit": "GB/s", "cores": res["threads"], "kind": "oracle",
               "sample": f"the first {res['layers']} layers of the 70B sweep (q/k/v, o, gate/up, down), B=1: "
                         f"float64 dequantize + numpy matmul, {res['seconds']:.1f} s of oracle time",
               "stages": {"dequant_s": round(res["dequant_s"], 2), "dequant_cores": 1,
                          "matmul_s": round(res["matmul_s"], 2), "matmul_cores": res["threads"],
                          "quantize_GBps": round(res["quantize_bytes"] / res["quantize_s"] / 1e9, 3),
                          "quantize_sample": "layer 0's fused q/k/v (10240x8192), numpy on 1 core",
                          "host_cpus": os.cpu_count()}}
        t0 = time.perf_counter()
        cpu["stages"]["configs"] = cpu_configs(dev, group)
        cpu["stages"]["configs_seconds"] = round(time.perf_counter() - t0, 1)
        log(f"[bench] cpu oracle: {cpu_gbs:.3f} GB/s over {res['seconds']:.1f}s ({res['layers']} layers); "
            f"other configs {cpu['stages']['configs_seconds']} s")

    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "ms_per_step_p10_p50_p90": [round(float(v), 4) for v in pct],
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
