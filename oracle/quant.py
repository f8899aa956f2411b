"""Oracle INT4 quantizer for keys and values. Test infrastructure only.

[AFS] "How It Works", item 3: everything outside the vertical lines and the
local window is quantized to 4 bits, for keys and for values alike. The pages
fix nothing else about the format; the reading used here (and by the whole
build) is:

* one scale/zero pair per token and per group of 32 consecutive channels;
* asymmetric min-max: s = (max - min) / 15 and z = min, both stored as fp16;
* codes c = clamp(rint((x - z) / s), 0, 15), round half to even, evaluated in
  float32 with the fp16-rounded s and z (fp16 rounding may push the quotient
  slightly outside [0, 15], hence the clamp);
* a constant group (max == min) stores s = 0 and codes 0;
* signed zeros: the pages say nothing; a zero scale or a zero minimum is
  stored as +0 (s and z are formed as ``value + 0.0`` in float32);
* dequantized value x_hat = c * s + z;
* packing: two codes per byte, the even channel in the low nibble.

Float32 steps use NumPy's IEEE float32 arithmetic (correctly rounded
subtract and divide, no contraction); np.rint rounds half to even and
float32 -> float16 conversion rounds to nearest even.
"""
from __future__ import annotations

import numpy as np

LEVELS = 15  # codes 0 .. 15


def quantize_groups(x: np.ndarray, group: int = 32):
    """Quantize rows along the last axis.

    x: float array [..., D] whose values are exact in float32 (inputs are
    fp32, bf16 or fp16). Returns (codes uint8 [..., D] with values 0..15,
    scale float16 [..., D/group], zero float16 [..., D/group]).
    """
    x = np.asarray(x)
    D = x.shape[-1]
    assert D % group == 0, "head_dim must be a multiple of the group size"
    xf = x.astype(np.float32)
    if not np.array_equal(xf.astype(np.float64), np.asarray(x, dtype=np.float64)):
        raise ValueError("quantizer input must be exactly representable in float32")
    if not np.all(np.isfinite(xf)):
        raise ValueError("quantizer input must be finite")
    g = xf.reshape(x.shape[:-1] + (D // group, group))
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    s32 = (mx - mn) / np.float32(LEVELS) + np.float32(0)   # float32 ops; -0 -> +0
    mn0 = mn + np.float32(0)                               # -0 -> +0
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
        z16 = mn0.astype(np.float16)
    if not (np.all(np.isfinite(s16)) and np.all(np.isfinite(z16))):
        raise ValueError("group range or minimum outside the fp16 range")
    s = s16.astype(np.float32)[..., None]
    z = z16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g - z) / s                            # float32 subtract, float32 divide
    c = np.clip(np.rint(t), 0, LEVELS)
    c = np.where(s == 0, 0, c)
    codes = c.astype(np.uint8).reshape(x.shape)
    return codes, s16, z16


def dequantize_groups(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray,
                      group: int = 32) -> np.ndarray:
    """x_hat = c * s + z in float64, [..., D]."""
    codes = np.asarray(codes)
    D = codes.shape[-1]
    c = codes.astype(np.float64).reshape(codes.shape[:-1] + (D // group, group))
    s = np.asarray(scale).astype(np.float64)[..., None]
    z = np.asarray(zero).astype(np.float64)[..., None]
    return (c * s + z).reshape(codes.shape)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., D] codes 0..15 -> [..., D/2] bytes, even channel in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[-1] % 2 == 0
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[..., D/2] bytes -> [..., D] codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def interleave_scale_zero(scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """[..., n_groups] fp16 scale and zero -> [..., n_groups, 2] fp16 bit
    patterns (uint16) in the storage order {scale, zero}."""
    s = np.asarray(scale, dtype=np.float16).view(np.uint16)
    z = np.asarray(zero, dtype=np.float16).view(np.uint16)
    return np.stack([s, z], axis=-1)


def split_scale_zero(sz: np.ndarray):
    """Inverse of interleave_scale_zero: returns (scale fp16, zero fp16)."""
    sz = np.asarray(sz, dtype=np.uint16)
    return sz[..., 0].view(np.float16), sz[..., 1].view(np.float16)


def quantize_rows(x: np.ndarray, group: int = 32):
    """Storage form used by the library: (packed codes uint8 [..., D/2],
    scale/zero uint16 [..., D/group, 2])."""
    codes, s, z = quantize_groups(x, group)
    return pack_nibbles(codes), interleave_scale_zero(s, z)


def dequantize_rows(packed: np.ndarray, sz: np.ndarray, group: int = 32) -> np.ndarray:
    s, z = split_scale_zero(sz)
    return dequantize_groups(unpack_nibbles(packed), s, z, group)
