"""Decoders for the storage formats the pages name (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* ``float8_e4m3fn`` is the dtype of the indexer key cache in the ``Indexer``
  code block of "详解DSA" (the ``k_cache`` buffer).  The format is the OCP
  8-bit e4m3 "fn" variant: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits, subnormals m * 2^-9, no infinities, and the two codes with all
  exponent and mantissa bits set (0x7F, 0xFF) are NaN.  Largest finite value
  1.75 * 2^8 = 448.
* bfloat16 is the upper half of an IEEE binary32.

Decoding is written from those field definitions; the oracle never encodes.
"""

import numpy as np

E4M3_NAN_CODES = (0x7F, 0xFF)


def _fields(codes):
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError("e4m3fn codes must be uint8")
    if np.any((c & 0x7F) == 0x7F):
        raise ValueError("e4m3fn NaN code (0x7F/0xFF) in input")
    sign = (c >> 7).astype(np.int64)
    exp = ((c >> 3) & 0xF).astype(np.int64)
    man = (c & 0x7).astype(np.int64)
    return sign, exp, man


def e4m3fn_times_512(codes):
    """Exact integer value * 2^9 of e4m3fn codes, as int64.

    A normal code (exponent field e >= 1) encodes (1 + m/8) * 2^(e-7)
    = (8 + m) * 2^(e-10), so times 2^9 it is the integer (8 + m) * 2^(e-1).
    A subnormal code encodes m * 2^-9, i.e. the integer m.  |result| <= 229376.
    """
    sign, exp, man = _fields(codes)
    mag = np.where(exp == 0, man, (8 + man) << np.maximum(exp - 1, 0))
    return np.where(sign == 1, -mag, mag).astype(np.int64)


def decode_e4m3fn(codes):
    """e4m3fn codes -> float64 values (exact; 0x80 is -0.0)."""
    sign = (np.asarray(codes) >> 7).astype(bool)
    mag = np.abs(e4m3fn_times_512(codes)).astype(np.float64) / 512.0
    return np.where(sign, -mag, mag)


def decode_bf16(bits):
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 bit patterns must be uint16")
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
