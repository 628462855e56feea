"""The W4A16 product, written as its plain definition.

Test infrastructure only (see the package docstring).

A linear layer stores W as [out_features, in_features] and computes
y = x . W^T, a [B, k] x [k, n] product ([YBB] section 一, the decode GEMV of
q_proj; [ARG] section 二.1, the [B, k] x [k, n] weight GEMM). Under W4A16 the
weights are replaced by their dequantized values w_hat = s * (q - z) and the
activations stay 16-bit ([ARG] section 二.3). The result here is that
definition computed in float64: the dequantized weights are exact in float64
and the only rounding is the float64 accumulation, far below the float16
output's resolution.
"""

from __future__ import annotations

import numpy as np

from .rtn import dequant_asym, dequant_sym


def gemm_ref(x16, w_hat) -> np.ndarray:
    """y[b, n] = sum_k x[b, k] * w_hat[n, k] in float64. x float16 [B, K], w_hat [N, K]."""
    x = np.asarray(x16, dtype=np.float64)
    w = np.asarray(w_hat, dtype=np.float64)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("shapes must be x [B, K] and w_hat [N, K]")
    return x @ w.T


def gemm_ref_rows(x16, q, s16, g: int, rows, z=None) -> np.ndarray:
    """y[:, rows] only: dequantize the chosen output rows, then gemm_ref.

    Used to check full-size matrices on sampled outputs.
    """
    rows = np.asarray(rows, dtype=np.int64)
    qr = np.asarray(q)[rows]
    sr = np.asarray(s16)[rows]
    if z is None:
        w_hat = dequant_sym(qr, sr, g)
    else:
        w_hat = dequant_asym(qr, sr, np.asarray(z)[rows], g)
    return gemm_ref(x16, w_hat)
