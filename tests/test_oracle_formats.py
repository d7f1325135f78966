"""Pins for the oracle's storage-format decoders and the input encoders.

The decoders are checked against torch's own float8_e4m3fn / bfloat16
conversions (independent library routines) and against values fixed by the
OCP e4m3fn definition; the synth encoders must round-trip every code.
"""

import numpy as np
import pytest
import torch

from oracle.formats import decode_bf16, decode_e4m3fn, e4m3fn_times_512
from synth.encode import encode_bf16_rne, encode_e4m3fn_rne, quantize_per_token

ALL_FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_e4m3fn_matches_torch_for_every_finite_code():
    ours = decode_e4m3fn(ALL_FINITE)
    ref = torch.from_numpy(ALL_FINITE.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))   # 0x80 is -0.0


def test_e4m3fn_landmarks_from_the_format_definition():
    d = lambda c: float(decode_e4m3fn(np.array([c], np.uint8))[0])
    assert d(0x7E) == 448.0            # largest finite
    assert d(0xFE) == -448.0
    assert d(0x01) == 2.0 ** -9        # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9    # largest subnormal
    assert d(0x08) == 2.0 ** -6        # smallest normal
    assert d(0x38) == 1.0              # bias 7 (FNUZ would read 0.5)
    assert d(0xB8) == -1.0
    pos = decode_e4m3fn(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)    # codes 0x00..0x7E strictly increasing


def test_e4m3fn_nan_codes_rejected():
    for c in (0x7F, 0xFF):
        with pytest.raises(ValueError):
            decode_e4m3fn(np.array([c], np.uint8))


def test_e4m3fn_integer_form_is_exact():
    vals = e4m3fn_times_512(ALL_FINITE)
    assert vals.dtype == np.int64
    assert np.array_equal(vals.astype(np.float64) / 512.0, decode_e4m3fn(ALL_FINITE))
    assert np.abs(vals).max() == 448 * 512


def test_bf16_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 16, 4096, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # drop inf/nan patterns
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(decode_bf16(bits), ref)


def test_encoders_round_trip_and_round_to_nearest_even():
    # every finite code survives decode -> encode
    assert np.array_equal(encode_e4m3fn_rne(decode_e4m3fn(ALL_FINITE)), ALL_FINITE)
    # torch's own e4m3fn cast (RNE, saturating here because inputs stay <= 448)
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * 40).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode_e4m3fn_rne(x), ref)
    # halfway cases: 1 + 1/16 lies between 1 and 1.125 -> even mantissa (1.0)
    assert decode_e4m3fn(encode_e4m3fn_rne(np.array([1.0625])))[0] == 1.0
    assert decode_e4m3fn(encode_e4m3fn_rne(np.array([1.1875])))[0] == 1.25
    assert decode_e4m3fn(encode_e4m3fn_rne(np.array([1e6])))[0] == 448.0
    # bf16 against torch's RNE conversion
    y = (rng.standard_normal(20000) * 3).astype(np.float32)
    refb = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(encode_bf16_rne(y), refb)


def test_per_token_quantisation_scale():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 128))
    codes, scale = quantize_per_token(x)
    assert scale.dtype == np.float32
    assert np.allclose(scale, np.abs(x).max(axis=1) / 448.0, rtol=1e-6)
    deq = decode_e4m3fn(codes) * scale.astype(np.float64)[:, None]
    # e4m3 has 3 mantissa bits: relative error <= 2^-4 for normals
    big = np.abs(x) > 0.05 * np.abs(x).max(axis=1, keepdims=True)
    assert np.all(np.abs(deq - x)[big] <= 2.0 ** -4 * np.abs(x)[big] + 1e-12)
    assert np.abs(decode_e4m3fn(codes)).max() <= 448.0
