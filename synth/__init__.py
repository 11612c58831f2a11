"""Seeded synthetic inputs for the MoE layer (ctypes over synth.c).

This module draws numbers and encodes them into the byte formats the layer
reads; it holds none of the layer's own arithmetic. The HIP path and the
CPU oracle both consume exactly the bytes produced here.

Host arrays use: float32 for binary32, uint16 for bfloat16 bit patterns,
uint8 for OCP E4M3 bytes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

SEED_BASE = 0x4D6F45000000


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-ffp-contract=off", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                  ctypes.c_void_p)
        L.synth_u64.argtypes = [u64, u64]
        L.synth_u64.restype = u64
        L.synth_normal_f32.argtypes = [u64, i64, dbl, dbl, vp, i32]
        L.synth_normal_bf16.argtypes = [u64, i64, dbl, dbl, vp, i32]
        L.synth_int_f32.argtypes = [u64, i64, i32, i32, vp, i32]
        L.synth_int_bf16.argtypes = [u64, i64, i32, i32, vp, i32]
        L.synth_f32_to_bf16.argtypes = [vp, i64, vp, i32]
        L.synth_f32_to_e4m3.argtypes = [vp, i64, ctypes.c_float, vp, i32]
        L.synth_amax_f32.argtypes = [vp, i64]
        L.synth_amax_f32.restype = ctypes.c_float
        L.synth_random_routing.argtypes = [u64, i32, i32, i32, vp]
        L.synth_random_routing.restype = i32
        _lib = L
    return _lib


def threads() -> int:
    """Worker threads for generation: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def seed_for(config: int, tensor_id: int) -> int:
    return SEED_BASE + 256 * int(config) + int(tensor_id)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def normal(seed: int, shape, std: float = 1.0, mean: float = 0.0, dtype: str = "f32") -> np.ndarray:
    n = int(np.prod(shape))
    if dtype == "f32":
        out = np.empty(n, np.float32)
        lib().synth_normal_f32(seed, n, mean, std, _ptr(out), threads())
    elif dtype == "bf16":
        out = np.empty(n, np.uint16)
        lib().synth_normal_bf16(seed, n, mean, std, _ptr(out), threads())
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def ints(seed: int, shape, lo: int, hi: int, dtype: str = "f32") -> np.ndarray:
    n = int(np.prod(shape))
    if dtype == "f32":
        out = np.empty(n, np.float32)
        lib().synth_int_f32(seed, n, lo, hi, _ptr(out), threads())
    elif dtype == "bf16":
        out = np.empty(n, np.uint16)
        lib().synth_int_bf16(seed, n, lo, hi, _ptr(out), threads())
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().synth_f32_to_bf16(_ptr(a), a.size, _ptr(out), threads())
    return out


def to_e4m3(a: np.ndarray, scale: float) -> np.ndarray:
    """E4M3(a / scale), round to nearest even, saturating at +-448."""
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().synth_f32_to_e4m3(_ptr(a), a.size, float(scale), _ptr(out), threads())
    return out


def amax(a: np.ndarray) -> float:
    a = np.ascontiguousarray(a, np.float32)
    return float(lib().synth_amax_f32(_ptr(a), a.size))


def quantize_e4m3(a: np.ndarray):
    """Per-tensor quantisation input recipe: scale = amax / 448, bytes = E4M3(a / scale)."""
    s = amax(a) / 448.0
    if s == 0.0:
        s = 1.0
    return to_e4m3(a, s), np.float32(s)


def quantize_mx(a: np.ndarray, axis: int):
    """MX input recipe (OCP microscaling, E4M3 elements): blocks of 32 along
    `axis` share the power-of-two scale 2^(floor(log2 amax) - 8) (8 = E4M3's
    largest exponent), stored as an E8M0 byte (exponent + 127); elements are
    E4M3(a / scale). Returns (E4M3 bytes, same shape; scale bytes, `axis`
    divided by 32)."""
    a = np.moveaxis(np.asarray(a, np.float32), axis, -1)
    shp = a.shape
    if shp[-1] % 32:
        raise ValueError("quantize_mx: axis length must be a multiple of 32")
    blocks = a.reshape(shp[:-1] + (shp[-1] // 32, 32))
    am = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        ex = np.where(am > 0, np.floor(np.log2(np.where(am > 0, am, 1.0))) - 8, 0).astype(np.int32)
    ex = np.clip(ex, -127, 127)
    scaled = blocks / np.ldexp(np.float32(1.0), ex)[..., None].astype(np.float32)
    q = to_e4m3(scaled.reshape(shp), 1.0)
    sb = (ex + 127).astype(np.uint8)
    return (np.ascontiguousarray(np.moveaxis(q, -1, axis)), np.ascontiguousarray(np.moveaxis(sb, -1, axis)))


_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # OCP FP4 magnitudes, codes 0..7


def to_e2m1(a: np.ndarray) -> np.ndarray:
    """E2M1 codes (0..15, sign in bit 3) of a: nearest magnitude on the FP4
    grid, ties to the even code, saturating at 6."""
    a = np.asarray(a, np.float64)
    mag = np.abs(a)
    mids = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) / 2  # 0.25 0.75 1.25 1.75 2.5 3.5 5
    code = np.searchsorted(mids, mag, side="right").astype(np.uint8)  # a midpoint goes up ...
    down = (mag == 0.25) | (mag == 1.25) | (mag == 2.5) | (mag == 5.0)  # ... unless the even code is below
    code -= down.astype(np.uint8)
    return code | (np.signbit(a).astype(np.uint8) << 3)


def pack_e2m1(codes: np.ndarray, axis: int) -> np.ndarray:
    """Two E2M1 codes per byte along `axis` (even index in the low nibble)."""
    c = np.moveaxis(np.asarray(codes, np.uint8), axis, -1)
    if c.shape[-1] % 2:
        raise ValueError("pack_e2m1: axis length must be even")
    packed = (c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4)
    return np.ascontiguousarray(np.moveaxis(packed.astype(np.uint8), -1, axis))


def quantize_mx4(a: np.ndarray, axis: int):
    """MX input recipe with E2M1 elements (OCP microscaling): blocks of 32
    along `axis` share the scale 2^(floor(log2 amax) - 2) (2 = E2M1's largest
    exponent), stored as an E8M0 byte; elements E2M1(a / scale), packed two
    per byte along `axis`. Returns (packed bytes, scale bytes)."""
    a = np.moveaxis(np.asarray(a, np.float32), axis, -1)
    shp = a.shape
    if shp[-1] % 32:
        raise ValueError("quantize_mx4: axis length must be a multiple of 32")
    blocks = a.reshape(shp[:-1] + (shp[-1] // 32, 32))
    am = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        ex = np.where(am > 0, np.floor(np.log2(np.where(am > 0, am, 1.0))) - 2, 0).astype(np.int32)
    ex = np.clip(ex, -127, 127)
    scaled = blocks / np.ldexp(np.float32(1.0), ex)[..., None].astype(np.float32)
    codes = to_e2m1(scaled.reshape(shp))
    packed = pack_e2m1(codes, -1)
    sb = (ex + 127).astype(np.uint8)
    return (np.ascontiguousarray(np.moveaxis(packed, -1, axis)), np.ascontiguousarray(np.moveaxis(sb, -1, axis)))


def mx_scales_slice_major(sa: np.ndarray, per_slice: int) -> np.ndarray:
    """Rearrange activation block scales (A, nb) into the slice-major order the
    MX grouped GEMMs read: (nb/per_slice, A, per_slice), every row's scales of
    one reduction slice adjacent and rows consecutive."""
    A, nb = sa.shape
    if nb % per_slice:
        raise ValueError("mx_scales_slice_major: blocks per row must be a multiple of the slice")
    return np.ascontiguousarray(np.asarray(sa, np.uint8).reshape(A, nb // per_slice, per_slice).transpose(1, 0, 2))


def mx_weight_scales_interleaved(sw: np.ndarray) -> np.ndarray:
    """Rearrange weight block scales (e, nb, N) into the order the MX grouped
    GEMMs read: N padded to N64 (a multiple of 64) and, within each group of
    64 columns, column 16j + c stored at position 4c + j."""
    e, nb, N = sw.shape
    n64 = (N + 63) // 64 * 64
    pad = np.zeros((e, nb, n64), np.uint8)
    pad[:, :, :N] = sw
    g = pad.reshape(e, nb, n64 // 64, 4, 16)           # [.., group, j, c]
    return np.ascontiguousarray(g.transpose(0, 1, 2, 4, 3).reshape(e, nb, n64))  # position 4c + j


def random_routing(seed: int, T: int, E: int, K: int) -> np.ndarray:
    out = np.empty((T, K), np.int32)
    if lib().synth_random_routing(seed, T, E, K, _ptr(out)) != 0:
        raise ValueError("bad routing shape")
    return out


def u64(seed: int, j: int) -> int:
    return int(lib().synth_u64(seed, j))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to binary32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
