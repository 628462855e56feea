"""w4a16_decode_amd: INT4 group-wise RTN weight quantization and the fused
W4A16 GEMV / skinny GEMM for AMD MI355X (gfx950), plus per-channel INT8
weights with the W8A16 GEMV.

Every computation runs in the HIP kernels of ``libq4.so`` behind the C ABI
declared in ``include/q4.h``, ``include/q8.h`` and ``include/q4_kv.h``; this package only marshals torch tensors
(device memory, the current HIP stream) into those calls. There is no CPU
fallback: without the built library or a GPU the calls raise.
"""

from .ops import (  # noqa: F401
    ActOrderWeight,
    KVCache4,
    Q4Error,
    QuantizedWeight,
    QuantizedWeight8,
    actorder_perm,
    from_canonical,
    gemm,
    gemm_config,
    gemm_noalloc,
    gemm_perm,
    gemm_shape,
    groups_count,
    kv_cache_alloc,
    kv_dequant,
    kv_quantize_pack,
    packed_bytes,
    q8_from_canonical,
    q8_gemm,
    q8_gemm_config,
    q8_packed_bytes,
    q8_quantize_pack,
    q8_to_canonical,
    q8_workspace_bytes,
    quantize_pack,
    quantize_pack_clip,
    quantize_pack_clip_into,
    quantize_pack_into,
    quantize_pack_perm,
    read_probe,
    rtn_check,
    status_str,
    to_canonical,
    version,
    workspace_bytes,
    workspace_bytes_perm,
)

__all__ = [
    "Q4Error", "QuantizedWeight", "quantize_pack", "quantize_pack_into", "quantize_pack_clip", "quantize_pack_clip_into", "gemm", "gemm_noalloc", "gemm_config", "to_canonical",
    "from_canonical", "packed_bytes", "groups_count", "workspace_bytes", "gemm_shape", "status_str", "version",
    "QuantizedWeight8", "q8_quantize_pack", "q8_gemm", "q8_gemm_config", "q8_to_canonical", "q8_from_canonical",
    "q8_packed_bytes", "q8_workspace_bytes",
    "ActOrderWeight", "actorder_perm", "quantize_pack_perm", "gemm_perm", "workspace_bytes_perm",
    "KVCache4", "kv_cache_alloc", "kv_quantize_pack", "kv_dequant", "read_probe", "rtn_check",
]
