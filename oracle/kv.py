"""INT4 group-wise quantization of a KV cache [batch, heads, seq, head_dim], from the pages.

Test infrastructure only (see the package docstring for who may import it).

[WIKI] section 7.4.1.2 (quantize_kv_cache_int4): the head_dim axis of K (or V)
[batch, heads, seq_len, head_dim] is cut into groups of group_size channels; each
group's scale is its amax / 7, codes are round(x / scale) clamped to [-8, 7], and
two INT4 codes are packed per byte (pack_int4, which the page leaves undefined).
[YBB] section 七: K and V of Llama-3-70B (80 layers, 8 KV heads, head_dim 128) take
2 * 80 * 8 * 128 * 2 = 327,680 bytes per token in BF16; scales must follow the
tokens they belong to (one per token and head at group_size = head_dim).

Readings (where the pages are silent, ambiguous or disagree):
  K1 The rounding is that of the weight quantizer (readings R1-R4 of rtn.py): a
     float16 scale fp16(fp32(amax) / 7), the IEEE float32 quotient, round half to
     even, codes 0 where the scale is 0.
  K2 pack_int4: the canonical packing of layout.py (low nibble = even element,
     4-bit two's complement), codes [b, h, s, head_dim / 2] bytes; scales
     [b, h, s, head_dim / group] float16, i.e. per token, head and group.
  K3 head_dim must be a multiple of group_size (the page's reshape needs it).
"""

from __future__ import annotations

import numpy as np

from .layout import pack_canonical
from .rtn import QMAX_SYM, QMIN_SYM, sym_scale_fp16


def quantize_kv_int4(K16, group: int):
    """Codes int8 [b, h, s, d] and scales float16 [b, h, s, d/group] (the page's steps)."""
    K = np.asarray(K16)
    if K.dtype != np.float16 or K.ndim != 4:
        raise TypeError("K must be a 4-D float16 array [batch, heads, seq_len, head_dim]")
    if not np.all(np.isfinite(K)):
        raise ValueError("K holds non-finite values")
    b, h, s, d = K.shape
    if group <= 0 or d % group != 0:
        raise ValueError(f"head_dim {d} is not a multiple of group_size {group}")   # K3
    Kr = K.reshape(b, h, s, d // group, group)                  # [..., num_groups, group_size]
    amax = np.abs(Kr).max(axis=-1)                              # per group
    s16 = sym_scale_fp16(amax)                                  # amax / 7 (K1)
    s32 = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.clip(np.rint(Kr.astype(np.float32) / s32), QMIN_SYM, QMAX_SYM)
    q = np.where(s32 == 0, 0.0, q)
    return q.astype(np.int8).reshape(b, h, s, d), s16


def pack_kv_int4(q) -> np.ndarray:
    """Two codes per byte along head_dim (K2): uint8 [b, h, s, d/2]."""
    q = np.asarray(q)
    b, h, s, d = q.shape
    return pack_canonical(q.reshape(-1, d)).reshape(b, h, s, d // 2)


def dequant_kv_int4(q, s16, group: int) -> np.ndarray:
    """x_hat = q * scale of its group, exact in float64."""
    q = np.asarray(q, dtype=np.float64)
    s = np.asarray(s16, dtype=np.float64)
    return q * np.repeat(s, group, axis=-1)


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bits: int = 16, group: int | None = None,
                       scale_bits: int = 16) -> float:
    """K and V bytes per token: 2 * layers * kv_heads * head_dim * bits / 8, plus one
    scale of scale_bits per group when `group` is given ([YBB] section 七)."""
    per_head = head_dim * bits / 8
    if group is not None:
        per_head += (head_dim // group) * scale_bits / 8
    return 2 * layers * kv_heads * per_head
