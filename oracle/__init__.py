"""CPU oracle for group-wise INT4 round-to-nearest quantization and the W4A16 product.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product
path (``w4a16_decode_amd`` and its HIP library) never imports, calls or
links it, and this package imports nothing from the product: the two share
no code. Inputs for both come from ``synth``.

Plain numpy, written for a reader to check against the source pages by eye:
no blocking, fusion or reordering beyond what the formulas state.

Sources, cited by page title and section throughout:

[YBB]  "LLM 后训练量化深度实战：从 GPTQ/AWQ 到 FP8 与 KV Cache 量化的显存-带宽极限工程"
       (www.ybb.press) -- section 二 (group-wise symmetric quantize_per_group and
       its MSE demo), section 一 (roofline of the decode GEMV).
[ARG]  "Post-training quantization: GPTQ, AWQ and rotation" (arganzheng.life,
       part 03 of the efficient-inference series) -- section 二.2 (quantization
       form, granularity, bits per weight), 二.3 (W4A16 dataflow), 三.1 (step
       alpha/7 and the Delta^2/12 noise model), 三.2 (clipping vs rounding, the
       range search), 四.3 (INT8 per-channel RTN as the W8A16 default), 五.3
       (act-order and g_idx), 六.2 (the four-weight RTN/AWQ table), 七.1 and 七.5
       (the INT8 step and its error), 八.2 (41.86 -> scale 5.9805), 十一.2 (the
       g_idx reorder is a gather).
[WIKI] "压缩算法" (cs-knowledge-wiki.pages.dev) -- section 7.4.1.1 (asymmetric
       s = (max-min)/(2^b-1), z = round(-min/s)), 7.4.1.2 (INT4 group code,
       clamp [-8, 7], two INT4 codes packed into one byte).
[IOC]  "模型量化技术工程实践：GPTQ/AWQ/QLoRA深度解析" (www.iopencloud.com) --
       section 1.2 (worked rounding example 3.14159 at scale 0.01; clipping 1000
       to the INT8 range), 2.1 (symmetric INT8, scale max/127).
[CH]   "量化：PTQ、GPTQ、AWQ 与 SmoothQuant" (charles2530.github.io) --
       section 1 (unified affine form, 4-bit symmetric range {-8..7}); the
       closing quick code example (per-channel INT8).

Readings taken where the pages are silent or inconsistent are listed in the
docstrings of the functions that take them.

Every function here is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, exhaustive checks or exact brute force; none is
"parity unpinned".
"""

from .rtn import (  # noqa: F401
    rtn_scalar,
    sym_scale_fp16,
    asym_scale_fp16,
    quantize_sym,
    quantize_sym_exact,
    quantize_asym,
    dequant_sym,
    dequant_asym,
    quant_mse,
)
from .layout import (  # noqa: F401
    pack_canonical,
    unpack_canonical,
    device_shapes,
    codes_to_device,
    codes_from_device,
    groupwise_to_device,
    groupwise_from_device,
)
from .gemm import gemm_ref, gemm_ref_rows  # noqa: F401
from .clip import clip_scale_fp16, clip_codes, clip_errors, quantize_sym_clip  # noqa: F401
from .actorder import actorder_order, actorder_gidx, quantize_sym_actorder, dequant_gidx, gemm_gidx_rows  # noqa: F401
from .kv import quantize_kv_int4, pack_kv_int4, dequant_kv_int4, kv_bytes_per_token  # noqa: F401
from .w8 import (  # noqa: F401
    w8_scale_fp16,
    w8_codes,
    quantize_w8,
    dequant_w8,
    gemm_w8_rows,
    w8_device_shapes,
    w8_codes_to_device,
    w8_codes_from_device,
    w8_scales_to_device,
)
