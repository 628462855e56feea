"""ctypes loader for libq4.so: argument marshalling only, no computation.

torch is imported before the library is opened: libq4.so links the
libamdhip64.so.7 soname, and with torch's HIP runtime already loaded the
dynamic loader binds the library to that same runtime, so torch's streams and
device pointers are valid inside it.
"""

from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libq4.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HEADERS = tuple(sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")))

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); mirrors the headers under include/
SIGNATURES = {
    "q4_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "q4_last_error": (ctypes.c_char_p, []),
    "q4_version": (ctypes.c_char_p, []),
    "q4_group_supported": (_I32, [_I32]),
    "q4_packed_bytes": (_SZ, [_I64, _I64]),
    "q4_groups_count": (_SZ, [_I64, _I64, _I32]),
    "q4_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I32]),
    "q4_gemm_shape": (ctypes.c_int, [_I64, _I64, _I64, _I32, _P]),
    "q4_quantize_pack": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "q4_quantize_pack_asym": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _P, _P, _P]),
    "q4_quantize_pack_clip": (ctypes.c_int, [_P, _I64, _I64, _I32, _I32, _P, _P, _P]),
    "q4_gemm": (ctypes.c_int, [_P, _I64, _P, _P, _I64, _I64, _I32, _P, _P, _SZ, _P]),
    "q4_gemm_asym": (ctypes.c_int, [_P, _I64, _P, _P, _P, _I64, _I64, _I32, _P, _P, _SZ, _P]),
    "q4_gemm_noalloc": (ctypes.c_int, [_P, _I64, _P, _P, _I64, _I64, _I32, _P, _P]),
    "q4_gemm_config": (ctypes.c_int, [_P, _I64, _P, _P, _P, _I32, _I64, _I64, _I32, _P, _I32, _I32, _I32, _I32, _P, _SZ,
                                      _P]),
    "q4_to_canonical": (ctypes.c_int, [_P, _P, _P, _I32, _I64, _I64, _I32, _P, _P, _P, _P]),
    "q4_from_canonical": (ctypes.c_int, [_P, _P, _P, _I32, _I64, _I64, _I32, _P, _P, _P, _P]),
    "q4_actorder_perm": (ctypes.c_int, [_P, _I64, _I32, _P]),
    "q4_quantize_pack_perm": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _P, _P, _P]),
    "q4_workspace_bytes_perm": (_SZ, [_I64, _I64, _I64, _I32]),
    "q4_gemm_perm": (ctypes.c_int, [_P, _I64, _P, _P, _P, _I64, _I64, _I32, _P, _P, _SZ, _P]),
    "q4_read_probe": (ctypes.c_int, [_P, _SZ, _P, _P]),
    "q4_rtn_check": (ctypes.c_int, [_P, _P]),
    "q4_kv_quantize_pack": (ctypes.c_int, [_P, _I64, _I64, _I64, _I32, _P, _P, _I64, _I64, _P]),
    "q4_kv_dequant": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _I32, _I64, _I64, _P, _P]),
    "q8_packed_bytes": (_SZ, [_I64, _I64]),
    "q8_scales_count": (_SZ, [_I64]),
    "q8_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "q8_quantize_pack": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "q8_gemm": (ctypes.c_int, [_P, _I64, _P, _P, _I64, _I64, _P, _P, _SZ, _P]),
    "q8_gemm_config": (ctypes.c_int, [_P, _I64, _P, _P, _I64, _I64, _P, _I32, _I32, _I32, _P, _SZ, _P]),
    "q8_to_canonical": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P]),
    "q8_from_canonical": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P]),
}

_lib = None


def header_functions(paths=HEADERS) -> list[str]:
    """Names of the functions the headers under include/ declare."""
    names = set()
    for path in paths:
        src = open(path, encoding="utf-8").read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(q[48]_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def load() -> ctypes.CDLL:
    """Open libq4.so once. Raises if it has not been built, or was built from sources
    other than the ones in this tree."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (binds the library to torch's HIP runtime)

    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m w4a16_decode_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    from .build import source_hash

    built = lib.q4_version().decode().rsplit(" ", 1)[-1]
    if built != source_hash():
        raise RuntimeError(f"{LIB_PATH} was built from other sources (library {built}, tree {source_hash()}): "
                           "rebuild it with `python -m w4a16_decode_amd.build`")
    _lib = lib
    return lib
