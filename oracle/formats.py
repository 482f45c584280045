"""Number formats the layer's inputs use, decoded from their published bit
layouts (oracle; test infrastructure only).

The pages name the expert format only as NVFP4, a 4-bit floating point
format the model was trained in natively (yodev.dev article, section on what
Edge0-145B is; Hugging Face card header). They do not define it. The
definitions below are the OCP ones:

* e2m1 (OCP Microscaling Formats v1.0, FP4 element type): 1 sign bit, 2
  exponent bits with bias 1, 1 mantissa bit, no infinities or NaN. Exponent
  field 0 is subnormal: magnitude = mantissa * 2^(1-1) * 0.5.
* E4M3 (OCP 8-bit Floating Point v1.0, "fn" variant): 1 sign, 4 exponent bits
  with bias 7, 3 mantissa bits, no infinities; S.1111.111 is NaN. Exponent
  field 0 is subnormal: magnitude = mantissa/8 * 2^-6.
* bf16: the upper 16 bits of an IEEE binary32.

The mixed 3/4-bit record: the card's Q3_K build is only partly 3-bit and
its experts are fixed-size records (Hugging Face card "Edge0-145B . Q3_K",
section "Architecture", the paragraph on the 1,630,720-byte expert record),
but no page defines a 3-bit element format or its layout. The format below is
this repository's own design:

* E1M1 (3 bits): 1 sign bit, 1 exponent bit with bias 1, 1 mantissa bit;
  exponent 0 is subnormal. Magnitudes 0, 0.5, 1, 1.5 (so each value is the
  e2m1 value of the same sign and the low two bits). Gate and up use it with
  the same E4M3 per-16 block scales and fp32 matrix scale; down stays e2m1.
* Storage: per matrix row, one 12-byte chunk per 32 consecutive elements,
  read as three little-endian 32-bit words w0, w1, w2. Elements 0..23 of
  the chunk are e2m1 codes of their value: element 8g + p (g < 3) is nibble
  p of w_g (bits 4p .. 4p+3: sign at bit 3, exponent at bit 1, mantissa at
  bit 0). The nibbles' bit 2, the e2m1 high exponent bit that E1M1 never
  sets, holds element 24 + p: its mantissa at bit 4p+2 of w0, its exponent
  there in w1, its sign there in w2. (A decoder turns any group of eight
  into e2m1 nibbles with a few shifts and masks.)
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code) -> np.ndarray:
    """Value of 4-bit e2m1 codes (low 4 bits of each entry), float64."""
    c = np.asarray(code).astype(np.int64) & 0xF
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    normal = np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int32))
    subnormal = m * 0.5
    return sign * np.where(e == 0, subnormal, normal)


def e4m3fn_value(byte) -> np.ndarray:
    """Value of E4M3fn bytes, float64 (NaN for S.1111.111)."""
    b = np.asarray(byte).astype(np.int64) & 0xFF
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 7
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))
    subnormal = np.ldexp(m / 8.0, -6)
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def bf16_value(bits) -> np.ndarray:
    """Value of bf16 bit patterns (uint16), float64."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """[..., n, k/2] packed bytes -> [..., n, k] 4-bit codes; element 2j is the
    low nibble of byte j, element 2j+1 the high nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


def e1m1_value(code) -> np.ndarray:
    """Value of 3-bit E1M1 codes (bit 2 sign, bit 1 exponent, bit 0 mantissa),
    float64: sign * (exponent ? 1 + mantissa/2 : mantissa/2)."""
    c = np.asarray(code).astype(np.int64) & 7
    sign = np.where((c >> 2) & 1, -1.0, 1.0)
    e = (c >> 1) & 1
    m = c & 1
    return sign * np.where(e == 0, m * 0.5, 1.0 + m * 0.5)


def unpack_e1m1(codes: np.ndarray) -> np.ndarray:
    """[..., n, 3k/8] chunked bytes -> [..., n, k] 3-bit codes (sign << 2 |
    exponent << 1 | mantissa), from the 12-byte chunks described above."""
    codes = np.asarray(codes, dtype=np.uint8)
    lead, nb = codes.shape[:-1], codes.shape[-1]
    w = codes.reshape(lead + (nb // 12, 3, 4)).astype(np.uint32)
    w = w[..., 0] | (w[..., 1] << 8) | (w[..., 2] << 16) | (w[..., 3] << 24)  # [..., c, 3]
    p = np.arange(8, dtype=np.uint32)

    def bit(word, b):  # bit b of nibble p of a word, for p = 0..7
        return (word[..., None] >> (np.uint32(4) * p + np.uint32(b))) & np.uint32(1)

    groups = []
    for g in range(3):                     # elements 8g + p: e2m1 nibbles
        wg = w[..., g]
        groups.append((bit(wg, 3) << 2) | (bit(wg, 1) << 1) | bit(wg, 0))
    groups.append((bit(w[..., 2], 2) << 2) | (bit(w[..., 1], 2) << 1) | bit(w[..., 0], 2))
    out = np.stack(groups, axis=-2)        # [..., c, 4, 8]
    return out.reshape(lead + (nb // 12 * 32,)).astype(np.uint8)


def dequant_e1m1(codes: np.ndarray, scales: np.ndarray, gscale) -> np.ndarray:
    """One E1M1 matrix [n][k] -> float64 weights:
    W[n, k] = e1m1(code[n, k]) * e4m3(scale[n, k // 16]) * gscale."""
    # the values of all 8 codes and 256 scale bytes, looked up per element
    q = e1m1_value(np.arange(8))[unpack_e1m1(codes)]
    s = np.repeat(e4m3fn_value(np.arange(256))[np.asarray(scales, dtype=np.uint8)], 16, axis=-1)
    return q * s * np.float64(np.float32(gscale))


def dequant_fp4(codes: np.ndarray, scales: np.ndarray, gscale) -> np.ndarray:
    """One quantised matrix [n][k] -> float64 weights.

    W[n, k] = e2m1(code[n, k]) * e4m3(scale[n, k // 16]) * gscale
    (two-level NVFP4-style scaling: a block scale per 16 consecutive k of one
    row, and one fp32 scale for the whole matrix).
    """
    # the values of all 16 codes and 256 scale bytes, looked up per element
    q = e2m1_value(np.arange(16))[unpack_codes(codes)]
    s = e4m3fn_value(np.arange(256))[np.asarray(scales, dtype=np.uint8)]
    s_full = np.repeat(s, 16, axis=-1)
    return q * s_full * np.float64(np.float32(gscale))
