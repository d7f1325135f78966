"""Pins for the oracle's per-block fp8 quantisation and key-cache append
(the ``act_quant`` / ``k_cache[:bsz, start_pos:end_pos] = k_fp8`` steps of the
``Indexer`` code block in "详解DSA").

The rounding is checked against torch's own float32 -> float8_e4m3fn cast (an
independent library routine), against values derived by hand from the e4m3fn
field definition, and against the rounding error bound of the format.
"""

import numpy as np
import torch

from oracle.formats import decode_e4m3fn
from oracle.quant import cache_append, e4m3fn_nearest, quantize_blocks

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def _torch_e4m3(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_nearest_is_exact_on_every_finite_value():
    assert np.array_equal(e4m3fn_nearest(decode_e4m3fn(FINITE)), FINITE)


def test_nearest_matches_torch_cast_including_every_midpoint():
    pos = decode_e4m3fn(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2.0                    # exact in fp32 (5 significant bits)
    rng = np.random.default_rng(7)
    rand = np.concatenate([rng.uniform(-448, 448, 20000),
                           rng.uniform(-1, 1, 20000) * 2.0 ** rng.integers(-12, 0, 20000)])
    v = np.concatenate([mids, -mids, rand]).astype(np.float32)
    assert np.array_equal(e4m3fn_nearest(v), _torch_e4m3(v))


def test_ties_go_to_the_even_code_by_hand():
    # 1.0 = 0x38, 1.125 = 0x39, 1.25 = 0x3A (mantissa step 1/8 at exponent 0):
    # 1.0625 sits between 0x38 and 0x39 -> even 0x38; 1.1875 between 0x39 and
    # 0x3A -> even 0x3A.  Subnormal step 2^-9: 1.5 * 2^-9 -> 2 * 2^-9 (0x02).
    got = e4m3fn_nearest(np.array([1.0625, 1.1875, 1.5 * 2.0 ** -9, -1.0625]))
    assert list(got) == [0x38, 0x3A, 0x02, 0xB8]


def test_block_scale_and_codes_by_hand():
    # amax 3 -> scale = fp32(3/448); 3/scale is 448 (code 0x7E, exponent field
    # 15, mantissa 6: 1.75 * 2^8); -1.5/scale = -224 = -1.75 * 2^7 -> 0xF6;
    # 0.75/scale = 112 = 1.75 * 2^6 -> 0x6E; zeros stay 0x00.
    x = np.zeros((1, 128), np.float32)
    x[0, :3] = [3.0, -1.5, 0.75]
    codes, scale = quantize_blocks(x)
    assert scale[0] == np.float32(3.0) / np.float32(448.0)
    assert list(codes[0, :4]) == [0x7E, 0xF6, 0x6E, 0x00]
    assert np.all(codes[0, 3:] == 0)


def test_zero_block_and_negative_underflow():
    x = np.zeros((2, 128), np.float32)
    x[1, 0] = 1.0
    x[1, 1] = -1e-30                                      # rounds to -0: code 0x80
    codes, scale = quantize_blocks(x)
    assert scale[0] == np.float32(2.0 ** -126) / np.float32(448.0)
    assert np.all(codes[0] == 0)
    assert codes[1, 0] == 0x7E and codes[1, 1] == 0x80


def test_quantisation_error_within_half_a_step():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((512, 128)) * 2.0 ** rng.integers(-20, 20, (512, 1))).astype(np.float32)
    codes, scale = quantize_blocks(x)
    q = x / scale[:, None].astype(np.float64)
    deq = decode_e4m3fn(codes)
    a = np.abs(q)
    # step of the format at |q|: 2^-9 below 2^-6, else 2^(floor(log2|q|) - 3)
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(np.abs(deq - q) <= step / 2 * (1 + 1e-6))
    # the block maximum lands on +-448 (the fp32 quotient is 448 up to one rounding)
    top = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(deq[np.arange(512), top]) == 448.0)


def test_cache_append_writes_only_the_new_positions():
    rng = np.random.default_rng(5)
    B, S_max, q_len = 3, 40, 4
    seq_lens = np.array([10, 40, 2])                      # the last one: only 2 positions exist
    cache = rng.integers(0, 0x7E, (B, S_max, 128)).astype(np.uint8)
    scales = rng.uniform(1, 2, (B, S_max)).astype(np.float32)
    k_new = rng.standard_normal((B, q_len, 128)).astype(np.float32)
    c2, s2 = cache_append(cache, scales, k_new, seq_lens, q_len)
    codes, sc = quantize_blocks(k_new)
    for b in range(B):
        for i in range(q_len):
            s = seq_lens[b] - q_len + i
            if s >= 0:
                assert np.array_equal(c2[b, s], codes[b, i]) and s2[b, s] == sc[b, i]
    written = np.zeros((B, S_max), bool)
    for b in range(B):
        lo = max(seq_lens[b] - q_len, 0)
        written[b, lo:seq_lens[b]] = True
    assert np.array_equal(c2[~written], cache[~written]) and np.array_equal(s2[~written], scales[~written])
