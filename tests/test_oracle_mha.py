"""Pins of the MHA-mode prefill oracle (``oracle.mha``) against things other
than its own formula:

* weight absorption: MHA mode equals the (separately pinned) MQA-mode
  ``sparse_mla`` with every position selected, once the query's nope part is
  pushed through W_UK and the latent output through W_UV (the identity that
  makes the two modes of the luowle page's figure the same attention);
* torch's ``scaled_dot_product_attention`` (float64, causal) per head on a
  fresh prefill, with keys and values built from the decompression;
* closed forms: a query at position 0 returns its value row and lse = its one
  score; equal keys give equal weights;
* one element of the decompression summed by hand;
* the bf16 rounding of the decompressed rows against torch's float64 ->
  bfloat16 cast (round to nearest even), ties included.
"""

import numpy as np
import torch

from oracle import mha_prefill, mha_decompress, sparse_mla
from oracle.mha import D_LATENT, D_NOPE, D_ROPE, D_V, round_to_bf16


def _inputs(rng, B, q_len, S, H):
    q = rng.standard_normal((B * q_len, H, D_NOPE + D_ROPE)).astype(np.float32)
    kv = rng.standard_normal((B, S, D_LATENT + D_ROPE)).astype(np.float32)
    w = (rng.standard_normal((H, D_NOPE + D_V, D_LATENT)) / np.sqrt(D_LATENT)).astype(np.float32)
    return q, kv, w


def test_equals_absorbed_mqa_mode():
    rng = np.random.default_rng(1)
    B, q_len, S, H = 2, 3, 40, 4
    seq = np.array([40, 17])
    q, kv, w = _inputs(rng, B, q_len, S, H)
    sm = 1 / np.sqrt(192.0)
    out, lse = mha_prefill(q, "f32", kv, "f32", w, "f32", seq, q_len, sm)
    w_uk, w_uv = w[:, :D_NOPE].astype(np.float64), w[:, D_NOPE:].astype(np.float64)
    # q_latent[t, h] = W_UK[h]^T q_nope[t, h]; the rope part is unchanged
    q_lat = np.einsum("thd,hdc->thc", q[..., :D_NOPE].astype(np.float64), w_uk)
    q_mqa = np.concatenate([q_lat, q[..., D_NOPE:].astype(np.float64)], axis=-1).astype(np.float32)
    pos = np.repeat(seq, q_len) - q_len + np.tile(np.arange(q_len), B)
    idx = np.full((B * q_len, S), -1, np.int64)
    for t in range(B * q_len):
        idx[t, :pos[t] + 1] = np.arange(pos[t] + 1)
    o_lat, lse_mqa = sparse_mla(q_mqa, "f32", kv, "f32", idx, seq, q_len, sm)
    out_mqa = np.einsum("thc,hdc->thd", o_lat, w_uv)                 # v = W_UV c, so out = W_UV out_latent
    np.testing.assert_allclose(out, out_mqa, rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(lse, lse_mqa, rtol=1e-5, atol=1e-5)


def test_matches_torch_causal_sdpa_on_fresh_prefill():
    rng = np.random.default_rng(2)
    B, L, H = 1, 24, 3
    q, kv, w = _inputs(rng, B, L, L, H)
    sm = 0.07
    out, _ = mha_prefill(q, "f32", kv, "f32", w, "f32", np.array([L]), L, sm)
    k_nope, v = mha_decompress(kv, "f32", w, "f32")
    k = np.concatenate([k_nope[0], np.broadcast_to(kv[0, :, None, D_LATENT:].astype(np.float64),
                                                    (L, H, D_ROPE))], axis=-1)     # [L, H, 192]
    tq = torch.from_numpy(q.astype(np.float64)).transpose(0, 1)                     # [H, L, 192]
    tk = torch.from_numpy(np.ascontiguousarray(k)).transpose(0, 1)
    tv = torch.from_numpy(np.ascontiguousarray(v[0])).transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=sm)
    np.testing.assert_allclose(out, ref.transpose(0, 1).numpy(), rtol=1e-10, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(3)
    H = 2
    q, kv, w = _inputs(rng, 2, 1, 8, H)
    sm = 0.1
    # sequence 0 holds one token: its query (position 0) sees only key 0
    seq = np.array([1, 8])
    out, lse = mha_prefill(q, "f32", kv, "f32", w, "f32", seq, 1, sm)
    c0 = kv[0, 0, :D_LATENT].astype(np.float64)
    v0 = np.einsum("hdc,c->hd", w[:, D_NOPE:].astype(np.float64), c0)
    np.testing.assert_allclose(out[0], v0, rtol=1e-12, atol=1e-12)
    k0 = np.concatenate([np.einsum("hdc,c->hd", w[:, :D_NOPE].astype(np.float64), c0),
                         np.broadcast_to(kv[0, 0, D_LATENT:].astype(np.float64), (H, D_ROPE))], axis=1)
    np.testing.assert_allclose(lse[0], sm * np.sum(q[0].astype(np.float64) * k0, axis=1), rtol=1e-12)
    # identical key rows: uniform weights, so the output is the mean value row
    kv_same = np.broadcast_to(kv[1, :1], kv[1:].shape).copy()
    kv2 = np.concatenate([kv[:1], kv_same])
    out2, lse2 = mha_prefill(q, "f32", kv2, "f32", w, "f32", seq, 1, sm)
    v1 = np.einsum("hdc,c->hd", w[:, D_NOPE:].astype(np.float64), kv2[1, 0, :D_LATENT].astype(np.float64))
    np.testing.assert_allclose(out2[1], v1, rtol=1e-12, atol=1e-12)


def test_decompression_element_by_hand():
    rng = np.random.default_rng(4)
    q, kv, w = _inputs(rng, 2, 1, 5, 3)
    k_nope, v = mha_decompress(kv, "f32", w, "f32")
    b, s, h = 1, 3, 2
    for j in (0, 77, 127):
        want = sum(float(w[h, j, c]) * float(kv[b, s, c]) for c in range(D_LATENT))
        assert abs(k_nope[b, s, h, j] - want) < 1e-9
        want_v = sum(float(w[h, D_NOPE + j, c]) * float(kv[b, s, c]) for c in range(D_LATENT))
        assert abs(v[b, s, h, j] - want_v) < 1e-9


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(20000) * 2.0 ** rng.integers(-20, 20, 20000)
    # exact midpoints between neighbouring bf16 values (ties) in both directions
    base = rng.integers(0x3F00, 0x4100, 2000).astype(np.uint32) << 16
    mids = (base | 0x8000).view(np.float32).astype(np.float64)
    x = np.concatenate([x, mids, -mids, [0.0, -0.0, 1.0, 3.0e38]])
    want = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_to_bf16(x), want)
    q, kv, w = _inputs(rng, 1, 1, 6, 2)
    k_exact, v_exact = mha_decompress(kv, "f32", w, "f32")
    k_r, v_r = mha_decompress(kv, "f32", w, "f32", round_bf16=True)
    assert np.array_equal(k_r, round_to_bf16(k_exact)) and np.array_equal(v_r, round_to_bf16(v_exact))
