"""CPU checks of the attention verdict's weight-rounding allowance
(tests/gpu_util.weight_rounding_bound): when the softmax weights are rounded
to bf16 before the value product and normalised by the sum of the rounded
weights (the "详解DSA" MLA forward casts its fp32 softmax to the value dtype),
the output moves by at most the bound, per value dim; and the bound is not
vacuous (the worst case over many draws uses a good part of it)."""

import numpy as np
import torch

from synth.encode import encode_bf16_rne
from tests.gpu_util import U_BF16, bf16_ulp, weight_rounding_bound


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _case(rng, m, scale, peaked):
    q = encode_bf16_rne((rng.standard_normal((1, 1, 576)) * scale).astype(np.float32))
    kv = encode_bf16_rne(rng.standard_normal((1, m, 576)).astype(np.float32))
    if peaked:  # a few rows aligned with q: weights spread over a handful of rows
        qf = (q[0, 0].astype(np.uint32) << 16).view(np.float32)
        for j in range(min(3, m)):
            kv[0, j] = encode_bf16_rne((1.5 * qf + 0.2 * rng.standard_normal(576)).astype(np.float32))
    return q, kv


def test_bf16_weights_stay_within_the_bound():
    rng = np.random.default_rng(0)
    sm = 1.0 / np.sqrt(192.0)
    used = 0.0
    for it in range(60):
        m = int(rng.integers(2, 300))
        q, kv = _case(rng, m, scale=float(rng.choice([0.3, 1.0, 3.0])), peaked=bool(it % 2))
        c = (kv[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        qf = (q[0, 0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        z = sm * (c @ qf)
        p = np.exp(z - z.max())
        exact = (p / p.sum()) @ c[:, :512]
        pt = _bf16(p)                                    # weights rounded to bf16 (RNE)
        rounded = (pt @ c[:, :512]) / pt.sum()
        bound = weight_rounding_bound(q, "bf16", kv, "bf16", 0, np.arange(m), 0, 0, sm)
        dev = np.abs(rounded - exact)
        assert np.all(dev <= bound), f"case {it}: deviation {dev.max():.3g} above the bound"
        used = max(used, float((dev / np.maximum(bound, 1e-30)).max()))
    assert used > 0.2, f"the bound is never approached (worst use {used:.2f})"


def test_bound_is_zero_for_a_single_row_and_tiny_against_half_ulp_for_flat_weights():
    rng = np.random.default_rng(1)
    q, kv = _case(rng, 1, 1.0, False)
    b = weight_rounding_bound(q, "bf16", kv, "bf16", 0, np.arange(1), 0, 0, 0.07)
    assert np.all(b <= 1e-6 * 8)                          # only the fp32 slack: one row is its own output
    q, kv = _case(rng, 2048, 0.0, False)                 # q = 0: uniform weights, all exactly representable
    b = weight_rounding_bound(q, "bf16", kv, "bf16", 0, np.arange(2048), 0, 0, 0.07)
    assert np.all(b <= 1.1 * U_BF16 * 4.0)
    assert np.all(bf16_ulp(np.array([1.0, 3.0, 5.0])) == np.array([2.0 ** -7, 2.0 ** -6, 2.0 ** -5]))
