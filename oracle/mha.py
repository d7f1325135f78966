"""MHA-mode MLA prefill for sequences no longer than top-k (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources:

* "详解DSA", section "DSA计算流 & 性能分析": prefill inside top-k runs in MHA
  mode and beyond top-k in MQA mode; a sequence no longer than top-k keeps
  every position, so the indexer's work can be skipped.  The MLA forward
  code block on that page gives MHA mode (the branch taken when a mask is
  passed): ``wkv_b`` turns each cached latent row into per-head
  ``[k_nope | v]``, the key of head h is ``[k_nope_h, k_pe]`` (the rope part
  shared by every head), the scores are ``q . k * softmax_scale`` plus the
  index mask and the causal mask, softmax in fp32, output ``scores @ v``.
* charlestar page ("DeepSeek V3.2 稀疏注意力"), the short-prompt paragraph:
  when ``L <= k`` no position can be cut and short prefills emulate DSA with
  a masked MHA.
* luowle page ("NSA 与 DSA"), the MHA / MQA figure: MHA mode recovers each
  head's key and value from the latent.

With ``L <= k`` the index mask keeps every position, so the computation is
causal attention over the decompressed keys and values; that is what is
written out here.  Shapes follow the public configuration: 128-dim nope and
64-dim rope query parts, 128-dim values, a 512-wide latent.
"""

import numpy as np

from .dsa import _decode, query_positions
from .formats import decode_bf16

D_NOPE, D_ROPE, D_V, D_LATENT = 128, 64, 128, 512


def round_to_bf16(x):
    """float64 -> the nearest bfloat16 value (ties to even), as float64.

    Written from the format: keep the top 8 significand bits of the fp32
    value, rounding the dropped 16 bits to nearest, ties to even.  Values are
    first rounded to fp32 (inputs here are far from the fp32 / bf16 limits).
    """
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return decode_bf16(r)


def decompress(kv, kv_fmt, wkv_b, w_fmt, round_bf16=False):
    """``kv = wkv_b(kv)`` of the MLA forward code block, split per head.

    ``kv`` [B, S, 512 + 64] (latent after its norm, then k_pe), ``wkv_b``
    [H, 128 + 128, 512] (the Linear weight ``[H*256, 512]`` seen per head:
    rows 0..127 give k_nope, rows 128..255 give v).  Returns float64
    ``(k_nope [B, S, H, 128], v [B, S, H, 128])``; with ``round_bf16`` each
    is rounded to bf16, the dtype that Linear's output has in the code block
    (bf16 activations and weights).
    """
    c = _decode(kv, kv_fmt)[..., :D_LATENT]
    w = _decode(wkv_b, w_fmt)
    H = w.shape[0]
    kvb = c @ w.reshape(H * (D_NOPE + D_V), D_LATENT).T        # [B, S, H*256]
    kvb = kvb.reshape(c.shape[:-1] + (H, D_NOPE + D_V))
    if round_bf16:
        kvb = round_to_bf16(kvb)
    return kvb[..., :D_NOPE], kvb[..., D_NOPE:]


def mha_prefill(q, q_fmt, kv, kv_fmt, wkv_b, w_fmt, seq_lens, q_len, sm_scale, rows=None, heads=None,
                round_bf16=False):
    """MHA-mode attention of each query over every key up to its position.

    ``q`` [T, H, 192] = ``[q_nope (128) | q_pe (64)]``; ``kv`` [B, S_max, 576];
    ``wkv_b`` [H, 256, 512].  For row t (sequence b, position pos) and head h:
    ``k_s = [k_nope[b, s, h], kv[b, s, 512:576]]`` and
    ``z_s = sm_scale * q[t, h] . k_s`` for ``s = 0 .. pos``;
    ``out[t, h] = sum_s softmax(z)_s * v[b, s, h]``; ``lse = log sum_s exp z_s``
    (``-inf`` and a zero output when pos < 0).  This equals the page's MHA
    branch with the index mask of a top-k that keeps every position, i.e.
    whenever ``seq_lens[b] <= k``.  Heads are independent, so ``heads``
    (default: all) restricts the work to a subset.  ``round_bf16`` keeps the
    decompressed keys and values in bf16 as the code block's bf16 Linear
    does; everything after that is exact.  Returns float64
    ``(out [R, len(heads), 128], lse [R, len(heads)])``.
    """
    if heads is not None:
        heads = np.asarray(heads, dtype=np.int64)
        q, wkv_b = np.asarray(q)[:, heads], np.asarray(wkv_b)[heads]
    qd = _decode(q, q_fmt)
    T, H, _ = qd.shape
    batch, pos = query_positions(seq_lens, q_len)
    k_nope, v = decompress(kv, kv_fmt, wkv_b, w_fmt, round_bf16=round_bf16)
    k_pe = _decode(kv, kv_fmt)[..., D_LATENT:]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), H, D_V))
    lse = np.full((len(rows), H), -np.inf)
    for r, t in enumerate(rows):
        b, p = batch[t], pos[t]
        if p < 0:
            continue
        n = p + 1
        # scores of every head against keys 0..pos: nope part per head, rope part shared
        z = np.einsum("hd,shd->hs", qd[t, :, :D_NOPE], k_nope[b, :n]) + qd[t, :, D_NOPE:] @ k_pe[b, :n].T
        z *= sm_scale
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        l = e.sum(axis=1, keepdims=True)
        out[r] = np.einsum("hs,shd->hd", e, v[b, :n]) / l
        lse[r] = zmax[:, 0] + np.log(l[:, 0])
    return out, lse
