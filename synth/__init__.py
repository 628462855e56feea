"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module holds random-number plumbing and workload shapes only: it computes
no scales, codes or products. Both the oracle (CPU) and the
HIP path receive the same arrays from here, so a parity test compares the two
implementations on bit-identical inputs.

Weights are drawn as N(0, 1) in float32, multiplied by 0.02 and cast to
float16 with round-to-nearest-even; activations are N(0, 1) cast to float16.
Host streams come from ``numpy.random.default_rng(SeedSequence([seed, layer,
matrix, stream]))`` (stream 0 = weights, 1 = activations, 2 = outlier column
choice, 3 = per-channel energies ordering act-order groups). Large sweeps generate weights on the device with a seeded
``torch.Generator``; :func:`device_weight` documents that recipe.
"""

from __future__ import annotations

import numpy as np

# Workload shapes (out_features, in_features) of the decoder layers the source
# pages use as their running examples (Llama-3 8B and 70B).
LLAMA3_8B = {
    "q_proj": (4096, 4096),
    "k_proj": (1024, 4096),
    "v_proj": (1024, 4096),
    "o_proj": (4096, 4096),
    "gate_proj": (14336, 4096),
    "up_proj": (14336, 4096),
    "down_proj": (4096, 14336),
}
LLAMA3_70B = {
    "q_proj": (8192, 8192),
    "k_proj": (1024, 8192),
    "v_proj": (1024, 8192),
    "o_proj": (8192, 8192),
    "gate_proj": (28672, 8192),
    "up_proj": (28672, 8192),
    "down_proj": (8192, 28672),
}
MATRIX_ORDER = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")
# Matrices that read the same activation vector and are stored row-concatenated
# (one launch each), the way serving engines lay them out.
FUSED_GROUPS = (("q_proj", "k_proj", "v_proj"), ("o_proj",), ("gate_proj", "up_proj"), ("down_proj",))


def _rng(seed: int, layer: int, matrix: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(layer), int(matrix), int(stream)]))


def weight(out_features: int, in_features: int, seed: int = 0, layer: int = 0, matrix: int = 0,
           std: float = 0.02) -> np.ndarray:
    """W ~ N(0, std^2) as float16 [out, in] (sampled in float32, RNE cast)."""
    r = _rng(seed, layer, matrix, 0)
    w = r.standard_normal((out_features, in_features), dtype=np.float32) * np.float32(std)
    return w.astype(np.float16)


def heavy_tailed_weight(out_features: int, in_features: int, seed: int = 5, df: float = 3.0,
                        std: float = 0.02, outlier_frac: float = 0.01, outlier_gain: float = 50.0,
                        layer: int = 0, matrix: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Student-t(df) * std with round(outlier_frac * in) input columns scaled by outlier_gain.

    Returns (W float16 [out, in], sorted outlier column indices). The columns are
    drawn without replacement from their own stream; the gain is applied in
    float32 before the float16 cast.
    """
    r = _rng(seed, layer, matrix, 0)
    w = (r.standard_t(df, size=(out_features, in_features)).astype(np.float32) * np.float32(std))
    n_out = int(round(outlier_frac * in_features))
    cols = np.sort(_rng(seed, layer, matrix, 2).choice(in_features, size=n_out, replace=False))
    w[:, cols] *= np.float32(outlier_gain)
    return w.astype(np.float16), cols


def channel_energy(in_features: int, seed: int = 0, layer: int = 0, matrix: int = 0) -> np.ndarray:
    """Synthetic stand-in for a calibration statistic per input channel (the Hessian
    diagonal that orders the act-order groups): log-normal(0, 1) float64 values
    from stream 3. No calibration data is involved."""
    return _rng(seed, layer, matrix, 3).lognormal(0.0, 1.0, size=in_features)


def activation(batch: int, in_features: int, seed: int = 0, layer: int = 0, matrix: int = 0) -> np.ndarray:
    """x ~ N(0, 1) as float16 [batch, in]."""
    r = _rng(seed, layer, matrix, 1)
    return r.standard_normal((batch, in_features), dtype=np.float32).astype(np.float16)


def uniform_codes_weight(out_features: int, in_features: int, seed: int = 0) -> np.ndarray:
    """W with a few exact ties and zero groups mixed in: used by edge-case tests.

    Values are small multiples of 2^-6 in [-1, 1] so that many quotients land
    exactly on half-integers; every fourth row-block of 32 columns is zeroed.
    """
    r = _rng(seed, 0, 99, 0)
    w = r.integers(-64, 65, size=(out_features, in_features)).astype(np.float32) / np.float32(64.0)
    w[::4, : min(32, in_features)] = 0.0
    return w.astype(np.float16)


def device_weight(out_features: int, in_features: int, seed: int, layer: int, matrix: int,
                  device="cuda", std: float = 0.02):
    """Device-side recipe for large sweeps: torch.Generator seeded with
    seed*1_000_003 + layer*1009 + matrix, N(0,1) float32 * std, RNE cast to float16.
    (Host generation of tens of billions of values would take minutes.)
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(layer) * 1009 + int(matrix))
    w = torch.randn((out_features, in_features), generator=g, device=device, dtype=torch.float32)
    return (w * std).to(torch.float16)


def device_activation(batch: int, in_features: int, seed: int, layer: int, matrix: int, device="cuda"):
    """Device-side N(0,1) float16 activations; generator seed offset by 7 from the weights'."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(layer) * 1009 + int(matrix) + 7)
    return torch.randn((batch, in_features), generator=g, device=device, dtype=torch.float32).to(torch.float16)
