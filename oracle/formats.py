"""Decoding of the storage formats the GDPA inputs arrive in, to fp64.

Test infrastructure (see the package docstring).

* bf16: the upper 16 bits of an IEEE-754 binary32 value.
* fp16: IEEE-754 binary16: 1 sign bit, 5 exponent bits with bias 15, 10
  mantissa bits; exponent field 0 is subnormal (m/1024 * 2^-14); field 31 is
  infinity (m = 0) or NaN.
* FP8 E4M3: the OCP 8-bit floating point format ("OCP 8-bit Floating Point
  Specification (OFP8)", E4M3 encoding): 1 sign bit, 4 exponent bits with bias
  7, 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is
  NaN; there are no infinities; the largest finite magnitude is 448.
  The GDPA README ("Features": "FP8 (E4M3) forward") names the format; it does
  not state the scaling.  Reading: one fp32 scale per tensor, so the value a
  code stands for is decode(code) * scale.
* E8M0: the scale type of the OCP Microscaling Formats (MX) specification:
  8 exponent bits, no sign or mantissa, value 2^(code - 127); code 255 is NaN.
* MXFP8 (E4M3): the OCP MX format built on E4M3 elements: every block of 32
  consecutive elements shares one E8M0 scale, and an element stands for
  decode_e4m3(code) * 2^(scale - 127).  The GDPA README ("Features") lists
  MXFP8 among its coming formats without a layout; reading: blocks run along
  the head dim (the contraction axis of Q K^T), scales stored [..., D / 32].
* FP4 E2M1: the element type of the OCP MX specification's MXFP4: 1 sign bit,
  2 exponent bits with bias 1, 1 mantissa bit; exponent field 0 is subnormal
  (m/2 * 2^0); no infinities or NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* MXFP4: E2M1 elements, one E8M0 scale per block of 32.  Two elements share a
  byte; reading (the pages give no layout): element 2 i sits in the low nibble
  of byte i of a row, element 2 i + 1 in the high nibble, rows [..., D / 2]
  bytes, scales [..., D / 32] as for MXFP8.
"""
from __future__ import annotations

import numpy as np


def decode_bf16(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_f16(bits) -> np.ndarray:
    c = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(c & 0x8000, -1.0, 1.0)
    e = (c >> 10) & 0x1F
    m = (c & 0x3FF).astype(np.float64)
    normal = (1.0 + m / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    sub = (m / 1024.0) * 2.0 ** -14
    mag = np.where(e == 0, sub, normal)
    mag = np.where(e == 0x1F, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


def decode_e4m3(codes, scale: float = 1.0) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag * float(scale)


def decode_e8m0(codes) -> np.ndarray:
    """E8M0 scale codes -> 2^(code - 127) (fp64); code 255 -> NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2(c.astype(np.float64) - 127.0))


def decode_mxfp8(codes, scales, block: int = 32) -> np.ndarray:
    """MXFP8 E4M3 values (fp64): codes [..., D] (uint8 E4M3), scales
    [..., D / block] (uint8 E8M0); element d takes the scale of block d // block."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    assert codes.shape[-1] == scales.shape[-1] * block and codes.shape[:-1] == scales.shape[:-1]
    return decode_e4m3(codes) * np.repeat(decode_e8m0(scales), block, axis=-1)


def decode_e2m1(codes) -> np.ndarray:
    """FP4 E2M1 codes (low 4 bits of each value) -> fp64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    normal = (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0)
    sub = m / 2.0
    return sign * np.where(e == 0, sub, normal)


def unpack_fp4(packed) -> np.ndarray:
    """Bytes [..., D / 2] -> E2M1 codes [..., D]: element 2 i from the low
    nibble of byte i, element 2 i + 1 from its high nibble."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def decode_mxfp4(packed, scales, block: int = 32) -> np.ndarray:
    """MXFP4 values (fp64): packed [..., D / 2] bytes of E2M1 pairs, scales
    [..., D / block] (uint8 E8M0); element d takes the scale of block d // block."""
    codes = unpack_fp4(packed)
    scales = np.asarray(scales, dtype=np.uint8)
    assert codes.shape[-1] == scales.shape[-1] * block and codes.shape[:-1] == scales.shape[:-1]
    return decode_e2m1(codes) * np.repeat(decode_e8m0(scales), block, axis=-1)
