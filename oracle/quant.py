"""Per-block fp8 quantisation of the indexer's queries and keys (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The ``Indexer`` code block of "详解DSA" quantises q and k with
``act_quant(x, block_size, scale_fmt)`` and writes the key codes and their
scales into ``k_cache`` / ``k_scale_cache`` at the positions
``start_pos .. end_pos - 1``; its "DSA计算流" section adds that q and k are
quantised to FP8, that the key cache keeps the codes together with their
scale, and that the q-scale is later folded into the head weights.  The pages
do not print ``act_quant`` itself.  The reading used here, the plainest one
the fp8 cache format supports:

* one scale per block of 128 consecutive elements (``block_size`` equal to
  the 128-wide index head, so one scale per key and per (query, head));
* ``scale = amax / 448`` computed in fp32, where ``amax`` is the largest
  ``|x|`` of the block and 448 the largest finite e4m3fn value; an all-zero
  block takes ``amax = 2^-126`` so its scale stays positive;
* ``code = e4m3fn(x / scale)``: the fp32 quotient rounded to the nearest
  e4m3fn value, ties to the even code, with a quotient beyond 448 (possible
  only through the fp32 rounding of the scale) taking 448; the sign of the
  quotient is kept, so a negative value that rounds to zero gives -0.

The rounding is a nearest-value search over the decoded table of every
finite code (the decoder in ``formats`` is the format definition), so it
shares no arithmetic with any encoder.
"""

import numpy as np

from .formats import decode_e4m3fn

BLOCK = 128
E4M3_MAX = 448.0
AMAX_FLOOR = 2.0 ** -126

# codes 0x00 .. 0x7E: every finite non-negative e4m3fn value, increasing
_POS_CODES = np.arange(0, 0x7F, dtype=np.uint8)
_POS_VALUES = decode_e4m3fn(_POS_CODES)


def e4m3fn_nearest(v):
    """float array -> uint8 e4m3fn codes of the nearest value, ties to even.

    For ``|v|`` between two consecutive finite values the nearer one wins; at
    the exact midpoint the code with a zero last mantissa bit (an even code)
    wins.  ``|v| >= 448`` gives 448.  The sign bit is the sign of ``v``.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite value")
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")      # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 7)


def quantize_blocks(x):
    """``act_quant`` of the ``Indexer`` code block on blocks of 128.

    ``x``: float32 array [..., 128] (bf16 inputs are widened exactly to fp32
    first).  Returns ``(codes uint8 [..., 128], scale float32 [...])`` with
    ``scale = fp32(max(amax, 2^-126) / 448)`` and
    ``codes = e4m3fn_nearest(fp32(x / scale))``; both divisions are IEEE fp32
    divisions (round to nearest even), the precision a GPU kernel uses.
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("quantize_blocks takes float32 (widen bf16 exactly first)")
    if x.shape[-1] != BLOCK:
        raise ValueError("last dimension must be 128")
    amax = np.maximum(np.abs(x).max(axis=-1), np.float32(AMAX_FLOOR)).astype(np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    quot = (x / scale[..., None]).astype(np.float32)
    return e4m3fn_nearest(quot), scale


def cache_append(k_cache, k_scale_cache, k_new, seq_lens, q_len):
    """The ``self.k_cache[:bsz, start_pos:end_pos] = k_fp8`` step.

    ``k_new`` [B, q_len, 128] float32 holds the new keys of every sequence;
    they are the last ``q_len`` tokens of sequence b, i.e. positions
    ``L_b - q_len + i`` with ``L_b = seq_lens[b]`` (``end_pos``, the same
    convention as ``query_positions``).  As everywhere in the C ABI,
    ``seq_lens[b]`` is clamped into ``[0, S_max]`` first and positions below
    zero are not written.  Returns updated copies of ``k_cache``
    [B, S_max, 128] uint8 and ``k_scale_cache`` [B, S_max] float32; every
    other entry is left as it was.
    """
    k_cache = np.array(k_cache, dtype=np.uint8, copy=True)
    k_scale_cache = np.array(k_scale_cache, dtype=np.float32, copy=True)
    B, S_max, d = k_cache.shape
    k_new = np.asarray(k_new)
    if k_new.shape != (B, q_len, d) or d != BLOCK:
        raise ValueError("shape mismatch")
    codes, scale = quantize_blocks(k_new)
    for b in range(B):
        for i in range(q_len):
            s = min(max(int(seq_lens[b]), 0), S_max) - q_len + i
            if s >= 0:
                k_cache[b, s] = codes[b, i]
                k_scale_cache[b, s] = scale[b, i]
    return k_cache, k_scale_cache
