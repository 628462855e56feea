"""Byte and FLOP accounting used to report achieved bandwidth and MFMA rate.

Algorithmic bytes are what the method must move, not what a kernel happens to
fetch: 4 bits per code, plus the per-group metadata, plus the activations.
bits/weight = b + (b_scale + b_zero)/g ("Post-training quantization: GPTQ,
AWQ and rotation", arganzheng.life, section 二.2 and the group-size table of
section 四.2). The decode time model T(m) = max(W_bytes / BW, 2 N m / F)
comes from section 二.1 of the same page.

MI355X figures are AMD's published datasheet peaks (dense, no sparsity).
"""

from __future__ import annotations

HBM_PEAK_GBS = 8000.0            # HBM3E, 8 TB/s
MFMA_FP16_DENSE_TFLOPS = 2500.0  # dense fp16/bf16 matrix peak
VALU_FP32_TFLOPS = 157.3


def bits_per_weight(group: int, bits: int = 4, scale_bits: int = 16, zero_bits: int = 0) -> float:
    return bits + (scale_bits + zero_bits) / group


def weight_bytes(out_features: int, in_features: int, group: int, asym: bool = False) -> int:
    """Packed codes (4 bits each) + float16 scales (+ uint8 zeros) of one matrix."""
    n = out_features * in_features // 2 + 2 * out_features * (in_features // group)
    if asym:
        n += out_features * (in_features // group)
    return n


def gemm_read_bytes(B: int, out_features: int, in_features: int, group: int, asym: bool = False) -> int:
    """Bytes the product must read: quantized weights + float16 activations (outputs not counted)."""
    return weight_bytes(out_features, in_features, group, asym) + 2 * B * in_features


def gemm_flops(B: int, out_features: int, in_features: int) -> int:
    return 2 * B * out_features * in_features


def quantize_bytes(out_features: int, in_features: int, group: int, asym: bool = False) -> int:
    """float16 weights read + quantized weights written."""
    return 2 * out_features * in_features + weight_bytes(out_features, in_features, group, asym)


def w8_weight_bytes(out_features: int, in_features: int) -> int:
    """Per-channel INT8 codes (1 byte each) + one float16 scale per row."""
    return out_features * in_features + 2 * out_features


def w8_gemm_read_bytes(B: int, out_features: int, in_features: int) -> int:
    """Bytes the W8A16 product must read: INT8 weights, row scales, float16 activations."""
    return w8_weight_bytes(out_features, in_features) + 2 * B * in_features


def time_model_s(w_bytes: float, n_params: float, m: int, bw_bytes_s: float, flops_s: float) -> float:
    """T(m) = max(W_bytes / BW, 2 N m / F): lower bound of one forward over m token rows."""
    return max(w_bytes / bw_bytes_s, 2.0 * n_params * m / flops_s)
