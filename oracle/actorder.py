"""Act-order (desc_act) grouping with a per-channel group index g_idx, written out from the pages.

Test infrastructure only (see the package docstring for who may import it).

[ARG] section 五.3: GPTQ may quantize the input channels in descending order of
the Hessian diagonal H_ii (the channels' input variance), so that the channels
that matter most are quantized first; the cost is that the quantized column
order is shuffled and the kernel needs a reorder index, g_idx. Section 十一.2:
that reorder is a gather. Groups of g are formed along the quantization order,
so the channels sharing a scale are no longer contiguous in the weight matrix:
channel k uses the scale of group g_idx[k].

Steps (this module quantizes with RTN inside each act-order group; GPTQ's
Hessian-based error compensation needs calibration data and is not part of the
kernel-visible path):
  1. order = the channels sorted by descending h (h standing in for H_ii),
     equal h in ascending channel index;
  2. g_idx[order[i]] = i // g: group j holds order[j*g : (j+1)*g];
  3. per row n and group j: amax = max |W[n, k]| over the channels k of group j,
     s16[n, j] = fp16(fp32(amax) / 7), and q[n, k] = clamp(rint(fp32(w) / fp32(s16)),
     -8, 7) with the scale of the channel's own group (readings R1-R4 of rtn.py);
  4. w_hat[n, k] = s16[n, g_idx[k]] * q[n, k] (the per-channel scale gather), and
     y = x . w_hat^T.

Readings (where the pages are silent, ambiguous or disagree):
  A1 Ties in h keep ascending channel order (a stable sort of -h).
  A2 Groups are consecutive runs of g channels in quantization order; in % g == 0.
  A3 Inside a group the codes and the scale are plain RTN: act-order changes which
     channels share a scale, not the rounding.
"""

from __future__ import annotations

import numpy as np

from .rtn import QMAX_SYM, QMIN_SYM, _check_fp16_matrix, sym_scale_fp16


def actorder_order(h) -> np.ndarray:
    """Channels by descending h, ties in ascending channel index (step 1, A1)."""
    h = np.asarray(h, dtype=np.float64)
    if h.ndim != 1 or not np.all(np.isfinite(h)):
        raise ValueError("h must be a finite 1-D array, one value per input channel")
    return np.argsort(-h, kind="stable")


def actorder_gidx(h, g: int) -> np.ndarray:
    """g_idx[k] = (position of channel k in the quantization order) // g (step 2, A2)."""
    order = actorder_order(h)
    K = order.size
    if g <= 0 or K % g != 0:
        raise ValueError(f"in_features {K} is not a multiple of group size {g}")
    g_idx = np.empty(K, dtype=np.int64)
    g_idx[order] = np.arange(K) // g
    return g_idx


def quantize_sym_actorder(W16, g: int, h):
    """Symmetric INT4 RTN over act-order groups (steps 1-3).

    Returns (q int8 [N, K] in the original channel order, s16 float16 [N, K/g]
    indexed by group, g_idx int64 [K])."""
    W = _check_fp16_matrix(W16)
    N, K = W.shape
    if np.asarray(h).shape != (K,):
        raise ValueError("h must hold one value per input channel")
    g_idx = actorder_gidx(h, g)
    G = K // g
    s16 = np.zeros((N, G), dtype=np.float16)
    for j in range(G):
        members = np.flatnonzero(g_idx == j)
        s16[:, j] = sym_scale_fp16(np.abs(W[:, members]).max(axis=1))
    s32 = s16.astype(np.float32)[:, g_idx]              # each channel's own group scale
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = W.astype(np.float32) / s32
    q = np.clip(np.rint(quot), QMIN_SYM, QMAX_SYM)
    q = np.where(s32 == 0, 0.0, q)
    return q.astype(np.int8), s16, g_idx


def dequant_gidx(q, s16, g_idx) -> np.ndarray:
    """w_hat[n, k] = s16[n, g_idx[k]] * q[n, k], exact in float64 (step 4)."""
    q = np.asarray(q, dtype=np.float64)
    s = np.asarray(s16, dtype=np.float64)
    return q * s[:, np.asarray(g_idx, dtype=np.int64)]


def gemm_gidx_rows(x16, q, s16, g_idx, rows) -> np.ndarray:
    """y[:, rows] = x . w_hat[rows]^T in float64, w_hat by the g_idx gather."""
    rows = np.asarray(rows, dtype=np.int64)
    w = dequant_gidx(np.asarray(q)[rows], np.asarray(s16)[rows], g_idx)
    x = np.asarray(x16, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("shapes must be x [B, K] and q [N, K]")
    return x @ w.T
