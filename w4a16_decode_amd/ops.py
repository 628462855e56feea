"""torch-facing wrappers over the libq4 C ABI (same names as the C calls).

These functions check tensor dtypes, devices and shapes, allocate outputs with
torch on the tensors' device, and pass raw pointers plus torch's current HIP
stream to libq4. They do no arithmetic of their own.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

from . import _lib

SUPPORTED_GROUPS_NOTE = "32, 64 or a multiple of 128"


class Q4Error(RuntimeError):
    """A libq4 call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{status_str(status)} ({status}): {message}")
        self.status = status


def _check(status: int) -> None:
    if status != 0:
        raise Q4Error(status, _lib.load().q4_last_error().decode())


def status_str(status: int) -> str:
    return _lib.load().q4_status_str(int(status)).decode()


def version() -> str:
    return _lib.load().q4_version().decode()


def packed_bytes(out_features: int, in_features: int) -> int:
    return int(_lib.load().q4_packed_bytes(out_features, in_features))


def groups_count(out_features: int, in_features: int, group: int) -> int:
    return int(_lib.load().q4_groups_count(out_features, in_features, group))


def workspace_bytes(batch: int, out_features: int, in_features: int, group: int) -> int:
    return int(_lib.load().q4_workspace_bytes(batch, out_features, in_features, group))


def gemm_shape(batch: int, out_features: int, in_features: int, group: int) -> tuple:
    """q4_gemm_shape (host): the launch shape q4_gemm picks on the current device, as
    (rows_per_wave, waves_per_group, k_splits, col_tiles) -- gemm_config's arguments."""
    shape = (ctypes.c_int32 * 4)()
    _check(_lib.load().q4_gemm_shape(batch, out_features, in_features, group, shape))
    return tuple(int(v) for v in shape)


def _stream(t) -> int:
    import torch

    return torch.cuda.current_stream(t.device).cuda_stream


def _require_gpu(t, name: str, dtype) -> None:
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a GPU (got {t.device}); libq4 has no CPU path")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class QuantizedWeight:
    """Device-layout INT4 weights of an [out_features, in_features] matrix."""

    packed: object          # uint8 [packed_bytes(out, in)]
    scales: object          # float16 [groups_count(out, in, group)]
    zeros: object | None    # uint8 [groups_count(...)] for asymmetric weights
    out_features: int
    in_features: int
    group: int
    asym: bool = False

    @property
    def device(self):
        return self.packed.device

    def nbytes(self) -> int:
        n = self.packed.numel() + 2 * self.scales.numel()
        if self.zeros is not None:
            n += self.zeros.numel()
        return n


def _alloc_qw(out_features: int, in_features: int, group: int, asym: bool, device) -> QuantizedWeight:
    import torch

    nb = packed_bytes(out_features, in_features)
    ng = groups_count(out_features, in_features, group)
    if nb == 0 or ng == 0:
        lib = _lib.load()
        raise Q4Error(3 if nb else 2, lib.q4_last_error().decode() or
                      f"invalid shape [{out_features}, {in_features}] / group {group} ({SUPPORTED_GROUPS_NOTE})")
    packed = torch.empty(nb, dtype=torch.uint8, device=device)
    scales = torch.empty(ng, dtype=torch.float16, device=device)
    zeros = torch.empty(ng, dtype=torch.uint8, device=device) if asym else None
    return QuantizedWeight(packed, scales, zeros, out_features, in_features, group, asym)


def quantize_pack(W, group: int = 128, asym: bool = False) -> QuantizedWeight:
    """q4_quantize_pack / q4_quantize_pack_asym on a float16 [out, in] GPU tensor."""
    import torch

    _require_gpu(W, "W", torch.float16)
    if W.dim() != 2:
        raise ValueError("W must be 2-D [out_features, in_features]")
    out_features, in_features = W.shape
    qw = _alloc_qw(out_features, in_features, group, asym, W.device)
    return quantize_pack_into(W, qw)


def quantize_pack_into(W, qw: QuantizedWeight) -> QuantizedWeight:
    """q4_quantize_pack / q4_quantize_pack_asym into the buffers of an existing
    QuantizedWeight of the same shape, group and kind (allocates nothing)."""
    import torch

    _require_gpu(W, "W", torch.float16)
    if tuple(W.shape) != (qw.out_features, qw.in_features):
        raise ValueError("W does not match the QuantizedWeight's shape")
    lib = _lib.load()
    if qw.asym:
        st = lib.q4_quantize_pack_asym(W.data_ptr(), qw.out_features, qw.in_features, qw.group, qw.packed.data_ptr(),
                                       qw.scales.data_ptr(), qw.zeros.data_ptr(), _stream(W))
    else:
        st = lib.q4_quantize_pack(W.data_ptr(), qw.out_features, qw.in_features, qw.group, qw.packed.data_ptr(),
                                  qw.scales.data_ptr(), _stream(W))
    _check(st)
    return qw


def quantize_pack_clip(W, group: int = 128, min_percent: int = 80) -> QuantizedWeight:
    """q4_quantize_pack_clip: symmetric INT4 with the per-group clipping search
    (alpha = p/100, p = min_percent..100); same packed format as quantize_pack."""
    import torch

    _require_gpu(W, "W", torch.float16)
    if W.dim() != 2:
        raise ValueError("W must be 2-D [out_features, in_features]")
    out_features, in_features = W.shape
    qw = _alloc_qw(out_features, in_features, group, False, W.device)
    return quantize_pack_clip_into(W, qw, min_percent)


def quantize_pack_clip_into(W, qw: QuantizedWeight, min_percent: int = 80) -> QuantizedWeight:
    """q4_quantize_pack_clip into the buffers of an existing symmetric QuantizedWeight."""
    import torch

    _require_gpu(W, "W", torch.float16)
    if tuple(W.shape) != (qw.out_features, qw.in_features) or qw.asym:
        raise ValueError("W does not match the symmetric QuantizedWeight's shape")
    st = _lib.load().q4_quantize_pack_clip(W.data_ptr(), qw.out_features, qw.in_features, qw.group, min_percent,
                                           qw.packed.data_ptr(), qw.scales.data_ptr(), _stream(W))
    _check(st)
    return qw


def _prep_gemm(x, qw: QuantizedWeight, out):
    import torch

    _require_gpu(x, "x", torch.float16)
    if x.dim() != 2 or x.shape[1] != qw.in_features:
        raise ValueError(f"x must be [B, {qw.in_features}]")
    if qw.packed.device != x.device or qw.scales.device != x.device:
        raise ValueError(f"x ({x.device}) and the weights ({qw.packed.device}) must be on the same GPU")
    B = x.shape[0]
    if out is None:
        out = torch.empty((B, qw.out_features), dtype=torch.float16, device=x.device)
    else:
        _require_gpu(out, "out", torch.float16)
        if tuple(out.shape) != (B, qw.out_features):
            raise ValueError(f"out must be [{B}, {qw.out_features}]")
        if out.device != x.device:
            raise ValueError(f"out ({out.device}) must be on x's GPU ({x.device})")
    return B, out


def _workspace(x, need: int, workspace):
    """The caller's workspace tensor, or a fresh one when the shape needs it and none was given."""
    import torch

    if need == 0 and workspace is None:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    elif workspace.device != x.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on x's device")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def gemm(x, qw: QuantizedWeight, out=None, workspace=None):
    """q4_gemm / q4_gemm_asym: y = x . W_hat^T, float16 [B, out_features].

    `workspace`: optional device tensor of at least workspace_bytes(B, out, in, group)
    bytes (allocated here when needed and not given)."""
    B, out = _prep_gemm(x, qw, out)
    lib = _lib.load()
    need = int(lib.q4_workspace_bytes(B, qw.out_features, qw.in_features, qw.group)) if B > 0 else 0
    ws_ptr, ws_bytes = _workspace(x, need, workspace)
    if qw.asym:
        st = lib.q4_gemm_asym(x.data_ptr(), B, qw.packed.data_ptr(), qw.scales.data_ptr(), qw.zeros.data_ptr(),
                              qw.out_features, qw.in_features, qw.group, out.data_ptr(), ws_ptr, ws_bytes,
                              _stream(x))
    else:
        st = lib.q4_gemm(x.data_ptr(), B, qw.packed.data_ptr(), qw.scales.data_ptr(), qw.out_features,
                         qw.in_features, qw.group, out.data_ptr(), ws_ptr, ws_bytes, _stream(x))
    _check(st)
    return out


def gemm_noalloc(x, qw: QuantizedWeight, out=None):
    """q4_gemm_noalloc: q4_gemm with the library's own device scratch in place of a
    workspace (symmetric weights). Allocates nothing when `out` is given; calls that
    overlap on one GPU race on that scratch."""
    if qw.asym:
        raise ValueError("q4_gemm_noalloc takes symmetric weights")
    B, out = _prep_gemm(x, qw, out)
    _check(_lib.load().q4_gemm_noalloc(x.data_ptr(), B, qw.packed.data_ptr(), qw.scales.data_ptr(), qw.out_features,
                                       qw.in_features, qw.group, out.data_ptr(), _stream(x)))
    return out


def gemm_config(x, qw: QuantizedWeight, rows_per_wave: int, waves_per_group: int, k_splits: int = 1,
                col_tiles: int | None = None, out=None, workspace=None):
    """q4_gemm_config: q4_gemm with an explicit launch shape (tuning).

    col_tiles defaults to 1 for B <= 16 (GEMV) and, for the skinny GEMM, to the power of
    two (2, 4 or 8) of 16-row tiles that covers B; 3 and 6 are accepted too."""
    B, out = _prep_gemm(x, qw, out)
    lib = _lib.load()
    if col_tiles is None:
        col_tiles = 1 if B <= 16 else min(8, max(2, 1 << ((B + 15) // 16 - 1).bit_length()))
    need = 4 * k_splits * B * qw.out_features if k_splits > 1 else 0
    ws_ptr, ws_bytes = _workspace(x, need, workspace)
    st = lib.q4_gemm_config(x.data_ptr(), B, qw.packed.data_ptr(), qw.scales.data_ptr(),
                            qw.zeros.data_ptr() if qw.zeros is not None else None, int(qw.asym),
                            qw.out_features, qw.in_features, qw.group, out.data_ptr(), rows_per_wave,
                            waves_per_group, k_splits, col_tiles, ws_ptr, ws_bytes, _stream(x))
    _check(st)
    return out


def to_canonical(qw: QuantizedWeight):
    """q4_to_canonical: (codes uint8 [out, in/2], scales float16 [out, in/g], zeros uint8 or None)."""
    import torch

    N, K, g = qw.out_features, qw.in_features, qw.group
    dev = qw.packed.device
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, K // g), dtype=torch.float16, device=dev)
    zeros = torch.empty((N, K // g), dtype=torch.uint8, device=dev) if qw.asym else None
    lib = _lib.load()
    st = lib.q4_to_canonical(qw.packed.data_ptr(), qw.scales.data_ptr(),
                             qw.zeros.data_ptr() if qw.asym else None, int(qw.asym), N, K, g, codes.data_ptr(),
                             scales.data_ptr(), zeros.data_ptr() if qw.asym else None, _stream(qw.packed))
    _check(st)
    return codes, scales, zeros


def from_canonical(codes, scales, group: int, zeros=None) -> QuantizedWeight:
    """q4_from_canonical: canonical codes/scales(/zeros) on the GPU -> device layout."""
    import torch

    _require_gpu(codes, "codes", torch.uint8)
    _require_gpu(scales, "scales", torch.float16)
    asym = zeros is not None
    if asym:
        _require_gpu(zeros, "zeros", torch.uint8)
    N, K = codes.shape[0], codes.shape[1] * 2
    if tuple(scales.shape) != (N, K // group) or (asym and tuple(zeros.shape) != (N, K // group)):
        raise ValueError("scales/zeros must be [out, in/group]")
    qw = _alloc_qw(N, K, group, asym, codes.device)
    lib = _lib.load()
    st = lib.q4_from_canonical(codes.data_ptr(), scales.data_ptr(), zeros.data_ptr() if asym else None, int(asym),
                               N, K, group, qw.packed.data_ptr(), qw.scales.data_ptr(),
                               qw.zeros.data_ptr() if asym else None, _stream(codes))
    _check(st)
    return qw


# ---- act-order (g_idx) weights, include/q4.h -------------------------------------


@dataclass
class ActOrderWeight:
    """INT4 act-order weights: codes and scales of the column-permuted matrix, and the
    permutation (device int32 [in]) the product gathers x through."""

    qw: QuantizedWeight
    perm: object            # int32 [in_features] on the device

    @property
    def out_features(self) -> int:
        return self.qw.out_features

    @property
    def in_features(self) -> int:
        return self.qw.in_features

    @property
    def group(self) -> int:
        return self.qw.group


def read_probe(buf, sink) -> None:
    """q4_read_probe: read all of `buf` (a contiguous device tensor of a multiple of 8 KiB)
    with the plain streaming read kernel; `sink` is a device int32 tensor."""
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.load().q4_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), _stream(buf)))


def rtn_check(device=None) -> tuple[int, int]:
    """q4_rtn_check: (pairs checked, mismatches) of the quantizers' division-free code
    decision against the correctly rounded quotient, every float16 scale and weight."""
    import torch

    counts = torch.zeros(2, dtype=torch.int64, device=device or "cuda")
    _check(_lib.load().q4_rtn_check(counts.data_ptr(), _stream(counts)))
    c = counts.cpu().tolist()
    return int(c[0]), int(c[1])


def workspace_bytes_perm(batch: int, out_features: int, in_features: int, group: int) -> int:
    return int(_lib.load().q4_workspace_bytes_perm(batch, out_features, in_features, group))


def actorder_perm(g_idx, group: int):
    """q4_actorder_perm (host): channels of group 0 ascending, then group 1, ...
    g_idx: a sequence / numpy array of in_features ints. Returns a numpy int32 array."""
    import numpy as np

    gi = np.ascontiguousarray(np.asarray(g_idx), dtype=np.int32)
    if gi.ndim != 1:
        raise ValueError("g_idx must be 1-D")
    perm = np.empty_like(gi)
    _check(_lib.load().q4_actorder_perm(gi.ctypes.data, gi.size, group, perm.ctypes.data))
    return perm


def quantize_pack_perm(W, group: int, perm) -> ActOrderWeight:
    """q4_quantize_pack_perm: symmetric INT4 of W[:, perm] (perm: int32 tensor on W's device)."""
    import torch

    _require_gpu(W, "W", torch.float16)
    _require_gpu(perm, "perm", torch.int32)
    if W.dim() != 2 or perm.shape != (W.shape[1],):
        raise ValueError("W must be [out, in] and perm [in]")
    out_features, in_features = W.shape
    qw = _alloc_qw(out_features, in_features, group, False, W.device)
    _check(_lib.load().q4_quantize_pack_perm(W.data_ptr(), out_features, in_features, group, perm.data_ptr(),
                                             qw.packed.data_ptr(), qw.scales.data_ptr(), _stream(W)))
    return ActOrderWeight(qw, perm)


def gemm_perm(x, aw: ActOrderWeight, out=None, workspace=None):
    """q4_gemm_perm: y = x . W_hat^T for act-order weights (x gathered through perm)."""
    qw = aw.qw
    B, out = _prep_gemm(x, qw, out)
    if aw.perm.device != x.device:
        raise ValueError(f"perm ({aw.perm.device}) must be on x's GPU ({x.device})")
    lib = _lib.load()
    need = int(lib.q4_workspace_bytes_perm(B, qw.out_features, qw.in_features, qw.group)) if B > 0 else 0
    ws_ptr, ws_bytes = _workspace(x, need, workspace)
    _check(lib.q4_gemm_perm(x.data_ptr(), B, qw.packed.data_ptr(), qw.scales.data_ptr(), aw.perm.data_ptr(),
                            qw.out_features, qw.in_features, qw.group, out.data_ptr(), ws_ptr, ws_bytes, _stream(x)))
    return out


# ---- INT4 KV cache, include/q4_kv.h ------------------------------------------------


@dataclass
class KVCache4:
    """INT4 KV-cache storage for bh = batch * kv_heads sequences of max_seq positions:
    codes uint8 [bh, max_seq, head_dim / 2], scales float16 [bh, max_seq, head_dim / group]."""

    codes: object
    scales: object
    group: int

    @property
    def head_dim(self) -> int:
        return self.codes.shape[2] * 2

    @property
    def max_seq(self) -> int:
        return self.codes.shape[1]


def kv_cache_alloc(bh: int, max_seq: int, head_dim: int, group: int = 128, device="cuda") -> KVCache4:
    import torch

    if head_dim % group or group not in (32, 64, 128):
        raise ValueError("group must be 32, 64 or 128 and divide head_dim")
    return KVCache4(torch.zeros((bh, max_seq, head_dim // 2), dtype=torch.uint8, device=device),
                    torch.zeros((bh, max_seq, head_dim // group), dtype=torch.float16, device=device), group)


def kv_quantize_pack(src, cache: KVCache4, pos: int) -> None:
    """q4_kv_quantize_pack: src float16 [batch, heads, n, head_dim] (or [bh, n, head_dim])
    into positions pos .. pos + n - 1 of the cache."""
    import torch

    _require_gpu(src, "src", torch.float16)
    if src.dim() == 4:
        bh, n, d = src.shape[0] * src.shape[1], src.shape[2], src.shape[3]
    elif src.dim() == 3:
        bh, n, d = src.shape
    else:
        raise ValueError("src must be [batch, heads, n, head_dim] or [bh, n, head_dim]")
    if bh != cache.codes.shape[0] or d != cache.head_dim:
        raise ValueError("src does not match the cache's sequences or head_dim")
    if src.device != cache.codes.device:
        raise ValueError(f"src ({src.device}) and the cache ({cache.codes.device}) must be on the same GPU")
    _check(_lib.load().q4_kv_quantize_pack(src.data_ptr(), bh, n, d, cache.group, cache.codes.data_ptr(),
                                           cache.scales.data_ptr(), cache.max_seq, pos, _stream(src)))


def kv_dequant(cache: KVCache4, pos: int, n: int):
    """q4_kv_dequant: float16 [bh, n, head_dim] of positions pos .. pos + n - 1."""
    import torch

    bh = cache.codes.shape[0]
    dst = torch.empty((bh, n, cache.head_dim), dtype=torch.float16, device=cache.codes.device)
    _check(_lib.load().q4_kv_dequant(cache.codes.data_ptr(), cache.scales.data_ptr(), bh, n, cache.head_dim,
                                     cache.group, cache.max_seq, pos, dst.data_ptr(), _stream(dst)))
    return dst


# ---- per-channel INT8 weights (W8A16), include/q8.h ------------------------------


@dataclass
class QuantizedWeight8:
    """Device-layout per-channel INT8 weights of an [out_features, in_features] matrix."""

    packed: object          # uint8 [q8_packed_bytes(out, in)]
    scales: object          # float16 [q8_scales_count(out)]
    out_features: int
    in_features: int

    @property
    def device(self):
        return self.packed.device

    def nbytes(self) -> int:
        return self.packed.numel() + 2 * self.scales.numel()


def q8_packed_bytes(out_features: int, in_features: int) -> int:
    return int(_lib.load().q8_packed_bytes(out_features, in_features))


def q8_workspace_bytes(batch: int, out_features: int, in_features: int) -> int:
    return int(_lib.load().q8_workspace_bytes(batch, out_features, in_features))


def _alloc_qw8(out_features: int, in_features: int, device) -> QuantizedWeight8:
    import torch

    lib = _lib.load()
    nb = int(lib.q8_packed_bytes(out_features, in_features))
    ns = int(lib.q8_scales_count(out_features))
    if nb == 0 or ns == 0:
        raise Q4Error(2, f"invalid shape [{out_features}, {in_features}] (in must be a positive multiple of 8)")
    return QuantizedWeight8(torch.empty(nb, dtype=torch.uint8, device=device),
                            torch.empty(ns, dtype=torch.float16, device=device), out_features, in_features)


def q8_quantize_pack(W) -> QuantizedWeight8:
    """q8_quantize_pack: per-row symmetric INT8 of a float16 [out, in] GPU tensor."""
    import torch

    _require_gpu(W, "W", torch.float16)
    if W.dim() != 2:
        raise ValueError("W must be 2-D [out_features, in_features]")
    out_features, in_features = W.shape
    qw = _alloc_qw8(out_features, in_features, W.device)
    _check(_lib.load().q8_quantize_pack(W.data_ptr(), out_features, in_features, qw.packed.data_ptr(),
                                        qw.scales.data_ptr(), _stream(W)))
    return qw


def q8_gemm(x, qw: QuantizedWeight8, out=None, workspace=None):
    """q8_gemm: y = x . (q * s)^T, float16 [B, out_features]."""
    B, out = _prep_gemm(x, qw, out)
    lib = _lib.load()
    need = int(lib.q8_workspace_bytes(B, qw.out_features, qw.in_features)) if B > 0 else 0
    ws_ptr, ws_bytes = _workspace(x, need, workspace)
    _check(lib.q8_gemm(x.data_ptr(), B, qw.packed.data_ptr(), qw.scales.data_ptr(), qw.out_features,
                       qw.in_features, out.data_ptr(), ws_ptr, ws_bytes, _stream(x)))
    return out


def q8_gemm_config(x, qw: QuantizedWeight8, rows_per_wave: int, waves_per_group: int, k_splits: int = 1, out=None,
                   workspace=None):
    """q8_gemm_config: q8_gemm with an explicit GEMV launch shape (B <= 16, tuning)."""
    B, out = _prep_gemm(x, qw, out)
    need = 4 * k_splits * B * qw.out_features if k_splits > 1 else 0
    ws_ptr, ws_bytes = _workspace(x, need, workspace)
    _check(_lib.load().q8_gemm_config(x.data_ptr(), B, qw.packed.data_ptr(), qw.scales.data_ptr(), qw.out_features,
                                      qw.in_features, out.data_ptr(), rows_per_wave, waves_per_group, k_splits,
                                      ws_ptr, ws_bytes, _stream(x)))
    return out


def q8_to_canonical(qw: QuantizedWeight8):
    """q8_to_canonical: (codes int8 [out, in], scales float16 [out])."""
    import torch

    N, K = qw.out_features, qw.in_features
    codes = torch.empty((N, K), dtype=torch.int8, device=qw.device)
    scales = torch.empty(N, dtype=torch.float16, device=qw.device)
    _check(_lib.load().q8_to_canonical(qw.packed.data_ptr(), qw.scales.data_ptr(), N, K, codes.data_ptr(),
                                       scales.data_ptr(), _stream(qw.packed)))
    return codes, scales


def q8_from_canonical(codes, scales) -> QuantizedWeight8:
    """q8_from_canonical: canonical int8 codes [out, in] and float16 scales [out] -> device layout."""
    import torch

    _require_gpu(codes, "codes", torch.int8)
    _require_gpu(scales, "scales", torch.float16)
    N, K = codes.shape
    if tuple(scales.shape) != (N,):
        raise ValueError("scales must be [out]")
    qw = _alloc_qw8(N, K, codes.device)
    _check(_lib.load().q8_from_canonical(codes.data_ptr(), scales.data_ptr(), N, K, qw.packed.data_ptr(),
                                         qw.scales.data_ptr(), _stream(codes)))
    return qw
