"""Plant plausible mistakes into the oracle (CPU only) and check the pins catch each.

A pin set that passes on a broken oracle proves nothing; these tests show
that every mistake below makes at least one pin fail.
"""

import numpy as np
import pytest

import oracle
import oracle.gemm
import oracle.layout
import oracle.rtn
import oracle.clip
import oracle.w8
import oracle.actorder
import oracle.kv
from pins import ALL_PINS


class _NumpyWith:
    """numpy with a few functions replaced (planted into one oracle module)."""

    def __init__(self, **over):
        self.__dict__.update(over)

    def __getattr__(self, name):
        return getattr(np, name)


def _caught():
    failures = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception as e:  # AssertionError or a crash both count as caught
            failures.append((pin.__name__, type(e).__name__))
    return failures


def _scale_div8(monkeypatch):
    orig = oracle.rtn.sym_scale_fp16
    f = lambda a, qmax=7: orig(a, 8)  # noqa: E731
    monkeypatch.setattr(oracle.rtn, "sym_scale_fp16", f)
    monkeypatch.setattr(oracle, "sym_scale_fp16", f)


def _scale_two_alpha_over_15(monkeypatch):
    orig = oracle.rtn.sym_scale_fp16
    f = lambda a, qmax=7: orig(a, 7.5)  # noqa: E731
    monkeypatch.setattr(oracle.rtn, "sym_scale_fp16", f)
    monkeypatch.setattr(oracle, "sym_scale_fp16", f)


def _truncate(monkeypatch):
    monkeypatch.setattr(oracle.rtn, "np", _NumpyWith(rint=np.trunc))


def _half_away(monkeypatch):
    monkeypatch.setattr(oracle.rtn, "np", _NumpyWith(rint=lambda a: np.sign(a) * np.floor(np.abs(a) + 0.5)))


def _fp16_quotient(monkeypatch):
    monkeypatch.setattr(oracle.rtn, "np",
                        _NumpyWith(rint=lambda a: np.rint(np.asarray(a).astype(np.float16).astype(np.float64))))


def _nibbles_swapped(monkeypatch):
    def pack(c):
        c = np.asarray(c).astype(np.int64)
        return ((c[:, 1::2] & 0xF) | ((c[:, 0::2] & 0xF) << 4)).astype(np.uint8)

    monkeypatch.setattr(oracle, "pack_canonical", pack)


def _device_nibble_order(monkeypatch):
    monkeypatch.setattr(oracle.layout, "_nibble_index", lambda e: e)


def _device_lane_order(monkeypatch):
    # rows and k-quarters swapped in the lane index
    orig = oracle.layout._device_position

    def pos(N, K):
        byte, shift, Np, Kp = orig(N, K)
        return byte, shift, Np, Kp

    def pos_bad(N, K):
        Kp = -(-K // 128) * 128
        Np = -(-N // 16) * 16
        S = Kp // 128
        n = np.arange(Np)[:, None]
        k = np.arange(Kp)[None, :]
        t, r = n // 16, n % 16
        s, m = k // 128, (k % 128) // 32
        c, e = (k % 32) // 8, k % 8
        p = oracle.layout._nibble_index(e)
        byte = ((t * S + s) * 64 + (4 * r + c)) * 16 + 4 * m + p // 2
        return byte, np.broadcast_to(4 * (p % 2), byte.shape), Np, Kp

    monkeypatch.setattr(oracle.layout, "_device_position", pos_bad)


def _dequant_wrong_group(monkeypatch):
    def dq(q, s, g):
        q = np.asarray(q, dtype=np.float64)
        s = np.asarray(s, dtype=np.float64)
        return q * np.tile(s, (1, g))

    monkeypatch.setattr(oracle, "dequant_sym", dq)
    monkeypatch.setattr(oracle.gemm, "dequant_sym", dq)


def _gemm_rows_reversed(monkeypatch):
    def g(x16, w_hat):
        return np.asarray(x16, dtype=np.float64) @ np.asarray(w_hat, dtype=np.float64)[::-1].T

    monkeypatch.setattr(oracle, "gemm_ref", g)
    monkeypatch.setattr(oracle.gemm, "gemm_ref", g)


def _gemm_fp16_accumulate(monkeypatch):
    def g(x16, w_hat):
        return (np.asarray(x16, dtype=np.float16) @ np.asarray(w_hat).astype(np.float16).T).astype(np.float64)

    monkeypatch.setattr(oracle, "gemm_ref", g)
    monkeypatch.setattr(oracle.gemm, "gemm_ref", g)


def _asym_zero_sign(monkeypatch):
    orig = oracle.rtn.asym_scale_fp16

    def quant(W16, g):
        W = np.asarray(W16)
        Wg = W.reshape(W.shape[0], -1, g)
        mn, mx = Wg.min(axis=2), Wg.max(axis=2)
        s16 = orig(mn, mx)
        s32 = s16.astype(np.float32)
        with np.errstate(all="ignore"):
            z = np.where(s32 == 0, 0, np.clip(np.rint(mn.astype(np.float32) / s32), 0, 15))
            q = np.clip(np.rint(Wg.astype(np.float32) / s32[..., None]) + z[..., None], 0, 15)
        q = np.where(s32[..., None] == 0, 0, q)
        return q.astype(np.uint8).reshape(W.shape), s16, z.astype(np.uint8)

    monkeypatch.setattr(oracle, "quantize_asym", quant)


def _asym_dequant_plus(monkeypatch):
    def dq(q, s, z, g):
        return (np.asarray(q, np.float64) + np.repeat(np.asarray(z, np.float64), g, axis=1)) * np.repeat(
            np.asarray(s, np.float64), g, axis=1)

    monkeypatch.setattr(oracle, "dequant_asym", dq)
    monkeypatch.setattr(oracle.gemm, "dequant_asym", dq)


def _asym_levels16(monkeypatch):
    orig = oracle.rtn.asym_scale_fp16
    monkeypatch.setattr(oracle.rtn, "asym_scale_fp16", lambda mn, mx, levels=15: orig(mn, mx, 16))


def _asym_range_fp16(monkeypatch):
    def sc(mn16, mx16, levels=15):                                   # range formed in float16 (an fp16 tensor's max - min)
        with np.errstate(over="ignore"):
            rng16 = (np.asarray(mx16, dtype=np.float16) - np.asarray(mn16, dtype=np.float16)).astype(np.float16)
            return (rng16.astype(np.float32) / np.float32(levels)).astype(np.float16)

    monkeypatch.setattr(oracle.rtn, "asym_scale_fp16", sc)
    monkeypatch.setattr(oracle, "asym_scale_fp16", sc)


def _clip_scale_one_rounding(monkeypatch):
    def sc(amax16, percent):                                         # p/100 * amax / 7 in float64, one rounding
        a = np.maximum(np.asarray(amax16, dtype=np.float16).astype(np.float64) * percent / 100.0, 1e-12)
        return (a / 7.0).astype(np.float16)

    monkeypatch.setattr(oracle.clip, "clip_scale_fp16", sc)
    monkeypatch.setattr(oracle, "clip_scale_fp16", sc)


def _clip_ties_to_smaller(monkeypatch):
    orig = oracle.clip.clip_errors

    def quant(W16, g, min_percent=80):
        W = np.asarray(W16)
        Wg = W.reshape(W.shape[0], -1, g)
        errs = orig(W, g, min_percent)
        percent = np.argmin(errs, axis=0) + min_percent        # first (smallest) percent wins ties
        amax = np.abs(Wg).max(axis=2)
        s16 = np.zeros(amax.shape, dtype=np.float16)
        for p in np.unique(percent):
            s16[percent == p] = oracle.clip.clip_scale_fp16(amax[percent == p], int(p))
        return oracle.clip.clip_codes(Wg, s16).astype(np.int8).reshape(W.shape), s16, percent

    monkeypatch.setattr(oracle, "quantize_sym_clip", quant)


def _clip_qmin8(monkeypatch):
    def codes(Wg16, s16):
        s32 = np.asarray(s16, dtype=np.float16).astype(np.float32)[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.clip(np.rint(Wg16.astype(np.float32) / s32), -8, 7)
        return np.where(s32 == 0, 0.0, q)

    monkeypatch.setattr(oracle.clip, "clip_codes", codes)
    monkeypatch.setattr(oracle, "clip_codes", codes)


def _clip_error_on_codes(monkeypatch):
    def errs(W16, g, min_percent=80):
        W = np.asarray(W16)
        Wg = W.reshape(W.shape[0], -1, g)
        amax = np.abs(Wg).max(axis=2)
        out = []
        for p in range(min_percent, 101):
            s16 = oracle.clip.clip_scale_fp16(amax, p)
            q = oracle.clip.clip_codes(Wg, s16)
            d = q - Wg.astype(np.float64)                      # forgot the scale
            out.append((d * d).sum(axis=2))
        return np.stack(out)

    monkeypatch.setattr(oracle.clip, "clip_errors", errs)


def _clip_without_100(monkeypatch):
    orig = oracle.clip.clip_scale_fp16
    monkeypatch.setattr(oracle.clip, "clip_scale_fp16", lambda a, p: orig(a, min(p, 99)))


def _w8_div128(monkeypatch):
    def sc(a, eps=None):
        return (np.asarray(a, dtype=np.float16).astype(np.float32) / np.float32(128)).astype(np.float16)

    monkeypatch.setattr(oracle.w8, "w8_scale_fp16", sc)
    monkeypatch.setattr(oracle, "w8_scale_fp16", sc)


def _w8_clamp_m128(monkeypatch):
    monkeypatch.setattr(oracle.w8, "np", _NumpyWith(clip=lambda a, lo, hi: np.clip(a, -128 if lo == -127 else lo, hi)))


def _w8_truncate(monkeypatch):
    monkeypatch.setattr(oracle.w8, "np", _NumpyWith(rint=np.trunc))


def _w8_half_away(monkeypatch):
    monkeypatch.setattr(oracle.w8, "np", _NumpyWith(rint=lambda a: np.sign(a) * np.floor(np.abs(a) + 0.5)))


def _w8_fp16_quotient(monkeypatch):
    monkeypatch.setattr(oracle.w8, "np",
                        _NumpyWith(rint=lambda a: np.rint(np.asarray(a).astype(np.float16).astype(np.float64))))


def _w8_scale_per_column(monkeypatch):
    def quant(W16):
        W = np.asarray(W16)
        amax = np.abs(W).max(axis=0)                         # over rows instead of channels
        s16 = oracle.w8.w8_scale_fp16(amax)
        s32 = s16.astype(np.float32)[None, :]
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(s32 == 0, 0, np.clip(np.rint(W.astype(np.float32) / s32), -127, 127))
        return q.astype(np.int8), s16[: W.shape[0]] if s16.size >= W.shape[0] else np.resize(s16, W.shape[0])

    monkeypatch.setattr(oracle, "quantize_w8", quant)


def _w8_layout_h_m_swapped(monkeypatch):
    def pos(N, K):
        sh = oracle.w8.w8_device_shapes(N, K)
        n = np.arange(sh["Np"])[:, None]
        k = np.arange(sh["Kp"])[None, :]
        t, r = n // 16, n % 16
        s, m = k // 128, (k % 128) // 64                     # 64-channel halves and 32-channel steps swapped
        h, c, e = (k % 64) // 32, (k % 32) // 8, k % 8
        return ((t * sh["S"] + s) * 2 + h) * 1024 + (r + 16 * c) * 16 + 8 * m + e, sh

    monkeypatch.setattr(oracle.w8, "_w8_device_position", pos)


def _w8_offset127(monkeypatch):
    orig_to = oracle.w8.w8_codes_to_device

    def to(q):
        return (orig_to(q).astype(np.int64) - 1).astype(np.uint8)

    monkeypatch.setattr(oracle, "w8_codes_to_device", to)


def _w8_dequant_rows_shifted(monkeypatch):
    def dq(q, s16):
        return np.asarray(q, dtype=np.float64) * np.roll(np.asarray(s16, dtype=np.float64), 1)[:, None]

    monkeypatch.setattr(oracle.w8, "dequant_w8", dq)
    monkeypatch.setattr(oracle, "dequant_w8", dq)


def _actorder_ascending(monkeypatch):
    monkeypatch.setattr(oracle.actorder, "actorder_order",
                        lambda h: np.argsort(np.asarray(h, dtype=np.float64), kind="stable"))
    monkeypatch.setattr(oracle, "actorder_order", oracle.actorder.actorder_order)


def _actorder_gidx_inverted(monkeypatch):
    def gidx(h, g):
        order = oracle.actorder.actorder_order(h)
        return order // g                                   # position -> group, not channel -> group

    monkeypatch.setattr(oracle.actorder, "actorder_gidx", gidx)
    monkeypatch.setattr(oracle, "actorder_gidx", gidx)


def _actorder_ties_reversed(monkeypatch):
    def order(h):
        h = np.asarray(h, dtype=np.float64)
        return np.lexsort((-np.arange(h.size), -h))                 # descending, ties by descending channel

    monkeypatch.setattr(oracle.actorder, "actorder_order", order)
    monkeypatch.setattr(oracle, "actorder_order", order)


def _actorder_dequant_by_position(monkeypatch):
    def dq(q, s16, g_idx):
        q = np.asarray(q, dtype=np.float64)
        g = q.shape[1] // np.asarray(s16).shape[1]
        return q * np.repeat(np.asarray(s16, dtype=np.float64), g, axis=1)

    monkeypatch.setattr(oracle.actorder, "dequant_gidx", dq)
    monkeypatch.setattr(oracle, "dequant_gidx", dq)


def _kv_scale_per_head(monkeypatch):
    def quant(K16, group):
        K = np.asarray(K16)
        b, h, sq, d = K.shape
        amax = np.abs(K).max(axis=(2, 3), keepdims=True)                 # one scale per head, over all tokens
        s16 = oracle.rtn.sym_scale_fp16(np.broadcast_to(amax, (b, h, sq, 1)))
        s16 = np.repeat(s16, d // group, axis=-1)
        with np.errstate(all="ignore"):
            q = np.clip(np.rint(K.astype(np.float32) / np.repeat(s16, group, axis=-1).astype(np.float32)), -8, 7)
        return np.where(np.repeat(s16, group, axis=-1) == 0, 0, q).astype(np.int8), s16

    monkeypatch.setattr(oracle, "quantize_kv_int4", quant)


def _kv_groups_strided(monkeypatch):
    def quant(K16, group):
        K = np.asarray(K16)
        b, h, sq, d = K.shape
        Kr = K.reshape(b, h, sq, group, d // group)                      # groups taken with stride d/group
        s16 = oracle.rtn.sym_scale_fp16(np.abs(Kr).max(axis=-2))
        with np.errstate(all="ignore"):
            q = np.clip(np.rint(Kr.astype(np.float32) / s16.astype(np.float32)[..., None, :]), -8, 7)
        q = np.where(s16[..., None, :] == 0, 0, q)
        return q.astype(np.int8).reshape(b, h, sq, d), s16

    monkeypatch.setattr(oracle, "quantize_kv_int4", quant)


def _kv_pack_high_first(monkeypatch):
    def pack(q):
        q = np.asarray(q).astype(np.int64)
        return (((q[..., 0::2] & 0xF) << 4) | (q[..., 1::2] & 0xF)).astype(np.uint8)

    monkeypatch.setattr(oracle, "pack_kv_int4", pack)


def _kv_bytes_no_factor_two(monkeypatch):
    def kvb(layers, kv_heads, head_dim, bits=16, group=None, scale_bits=16):
        per_head = head_dim * bits / 8 + ((head_dim // group) * scale_bits / 8 if group else 0)
        return layers * kv_heads * per_head                              # K only

    monkeypatch.setattr(oracle, "kv_bytes_per_token", kvb)


MUTATIONS = [
    _scale_div8, _scale_two_alpha_over_15, _truncate, _half_away, _fp16_quotient, _nibbles_swapped,
    _device_nibble_order, _device_lane_order, _dequant_wrong_group, _gemm_rows_reversed,
    _gemm_fp16_accumulate, _asym_zero_sign, _asym_dequant_plus, _asym_levels16, _asym_range_fp16,
    _clip_ties_to_smaller, _clip_scale_one_rounding, _clip_qmin8, _clip_error_on_codes, _clip_without_100,
    _w8_div128, _w8_clamp_m128, _w8_truncate, _w8_half_away, _w8_fp16_quotient, _w8_scale_per_column,
    _w8_layout_h_m_swapped, _w8_offset127, _w8_dequant_rows_shifted,
    _actorder_ascending, _actorder_gidx_inverted, _actorder_ties_reversed, _actorder_dequant_by_position,
    _kv_scale_per_head, _kv_groups_strided, _kv_pack_high_first, _kv_bytes_no_factor_two,
]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m.__name__.lstrip("_") for m in MUTATIONS])
def test_planted_mistake_is_caught(mutation, monkeypatch):
    mutation(monkeypatch)
    caught = _caught()
    assert caught, f"no pin caught the planted mistake {mutation.__name__}"
