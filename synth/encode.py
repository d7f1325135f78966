"""Storage encoders used to build inputs (round to nearest even).

* e4m3fn (OCP fp8, the ``float8_e4m3fn`` dtype of the indexer key cache):
  1 sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals m * 2^-9,
  largest finite 448, codes 0x7F/0xFF are NaN.  Encoding saturates to +-448.
* bfloat16: the upper 16 bits of an IEEE binary32, round to nearest even.
* Per-token fp8 quantisation of a key: one fp32 scale per 128-element block
  (one block per key), ``scale = amax / 448`` with amax floored at 2^-126.
"""

import numpy as np

E4M3_MAX = 448.0


def encode_e4m3fn_rne(x):
    """float array -> uint8 e4m3fn codes (RNE, saturating at +-448)."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value cannot be encoded")
    sign = (x < 0) | ((x == 0) & np.signbit(x))
    a = np.minimum(np.abs(x), E4M3_MAX)
    code = np.zeros(a.shape, dtype=np.int64)
    # subnormal range: |x| < 2^-6, step 2^-9 (a result of 8 is the smallest
    # normal, whose code is also 8)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 512.0).astype(np.int64)
    nrm = ~sub
    frac, ex = np.frexp(a[nrm])             # a = frac * 2^ex, frac in [0.5, 1)
    e = ex.astype(np.int64) - 1             # a = (2*frac) * 2^e, 2*frac in [1, 2)
    m = np.rint((2.0 * frac - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = e + carry
    m = np.where(carry, 0, m)
    code[nrm] = ((e + 7) << 3) | m
    if np.any(code > 0x7E):
        raise AssertionError("encoder produced a NaN code")
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def encode_bf16_rne(x):
    """float32 array -> uint16 bfloat16 bit patterns (RNE)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value cannot be encoded")
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def quantize_per_token(x):
    """Keys [..., 128] float -> (e4m3fn codes [..., 128], fp32 scale [...])."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.maximum(np.abs(x).max(axis=-1), 2.0 ** -126)
    scale = (amax / E4M3_MAX).astype(np.float32)
    codes = encode_e4m3fn_rne(x / scale.astype(np.float64)[..., None])
    return codes, scale
