"""Plain float64 definitions of the three DSA forward stages (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Notation (shared with the C ABI): ``B`` sequences, ``q_len`` new queries per
sequence, ``T = B * q_len`` query rows, row ``t = b * q_len + i``.  The keys
visible to the last query of sequence ``b`` are ``0 .. seq_lens[b]-1`` (the
``end_pos`` of the ``Indexer`` code block in "详解DSA"), so query ``i`` of
sequence ``b`` sits at position ``pos = seq_lens[b] - q_len + i`` and sees the
keys ``s <= pos`` (causal, inclusive).

Formats: ``'e4m3fn'`` (uint8 codes), ``'bf16'`` (uint16 bit patterns),
``'f32'`` (float32 values).  Every input is widened exactly to float64 before
any arithmetic; fp8 dot products are formed exactly on integers.
"""

import numpy as np

from .formats import decode_bf16, decode_e4m3fn, e4m3fn_times_512


def _decode(a, fmt):
    if fmt == "e4m3fn":
        return decode_e4m3fn(a)
    if fmt == "bf16":
        return decode_bf16(a)
    if fmt == "f32":
        a = np.asarray(a)
        if a.dtype != np.float32:
            raise TypeError("f32 input must be float32")
        return a.astype(np.float64)
    raise ValueError(f"unknown format {fmt!r}")


def query_positions(seq_lens, q_len):
    """Position of every query row: ``pos[b*q_len+i] = seq_lens[b]-q_len+i``.

    Follows ``end_pos = start_pos + seqlen`` in the ``Indexer`` code block of
    "详解DSA": the new tokens are the last ``q_len`` positions of the cache.
    Returns ``(batch_of_row, pos_of_row)`` as int64 arrays of length T.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    if q_len < 1 or np.any(seq_lens < q_len):
        raise ValueError("need 1 <= q_len <= seq_lens[b]")
    b = np.repeat(np.arange(len(seq_lens), dtype=np.int64), q_len)
    i = np.tile(np.arange(q_len, dtype=np.int64), len(seq_lens))
    return b, seq_lens[b] - q_len + i


def _raw_dots(q_rows, q_fmt, keys, k_fmt):
    """D[r, j, s] = sum_d q[r, j, d] * k[s, d]   ("详解DSA" Eq.(1), inner dot).

    fp8 x fp8: the dot is formed on the exact integers value*2^9, so every
    partial sum is an integer below 2^43 and the float64 GEMM is exact; the
    result is then scaled by 2^-18 (exact).  f32: a float64 GEMM of the
    widened values.
    """
    nr, h, d = q_rows.shape
    if q_fmt == "e4m3fn" and k_fmt == "e4m3fn":
        qi = e4m3fn_times_512(q_rows).astype(np.float64).reshape(nr * h, d)
        ki = e4m3fn_times_512(keys).astype(np.float64)
        return (qi @ ki.T).reshape(nr, h, -1) * 2.0 ** -18
    qf = _decode(q_rows, q_fmt).reshape(nr * h, d)
    kf = _decode(keys, k_fmt)
    return (qf @ kf.T).reshape(nr, h, -1)


def indexer_scores(q, q_fmt, w, w_fmt, k, k_fmt, seq_lens, q_len,
                   k_scale=None, q_scale=None, rows=None, chunk=16):
    """Lightning Indexer scores, "详解DSA" Eq.(1) with the fp8 scale fold.

    ``I[t, s] = k_scale[b, s] * sum_j (w[t, j] * q_scale[t, j]) * ReLU(D[t, j, s])``
    for ``s <= pos(t)``, and ``-inf`` for ``s > pos(t)`` (the causal
    ``index_score += mask`` of the ``Indexer`` code block).

    Where the scales enter follows the "DSA计算流" section of the same page:
    the q-scale multiplies the per-head ReLU output (it is folded into the
    weights as in the ``weights = ... * q_scale`` line) and the k-scale
    multiplies the sum over heads.  Both scales are positive, so this equals
    Eq.(1) on the dequantised q and k.  ``w`` is used as given (any softmax /
    head-count factors are the caller's).

    Shapes: q [T, H_I, d], w [T, H_I], k [B, S_max, d], k_scale [B, S_max] or
    None, q_scale [T, H_I] or None.  Returns float64 [len(rows), S_max].
    """
    q = np.asarray(q)
    T, HI, d = q.shape
    B, S_max, dk = np.asarray(k).shape
    if dk != d or len(seq_lens) != B or T != B * q_len:
        raise ValueError("shape mismatch")
    batch, pos = query_positions(seq_lens, q_len)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    weff = _decode(w, w_fmt)
    if q_scale is not None:
        weff = weff * np.asarray(q_scale, dtype=np.float32).astype(np.float64)
    out = np.full((len(rows), S_max), -np.inf)
    for b in range(B):
        sel = np.nonzero(batch[rows] == b)[0]
        if len(sel) == 0:
            continue
        ks = None if k_scale is None else \
            np.asarray(k_scale, dtype=np.float32)[b].astype(np.float64)
        for c0 in range(0, len(sel), chunk):
            part = sel[c0:c0 + chunk]
            trows = rows[part]
            smax = int(pos[trows].max()) + 1
            D = _raw_dots(q[trows], q_fmt, np.asarray(k)[b, :smax], k_fmt)
            I = np.einsum("rj,rjs->rs", weff[trows], np.maximum(D, 0.0))
            if ks is not None:
                I = I * ks[None, :smax]
            s = np.arange(smax)[None, :]
            I = np.where(s <= pos[trows][:, None], I, -np.inf)
            out[part, :smax] = I
    return out


def topk_select(scores_row, pos, k):
    """Top-k of one query row ("详解DSA": ``topk(min(index_topk, end_pos))``).

    The valid set is ``V = {s <= pos}``.  If ``|V| <= k`` every valid position
    is kept ("详解DSA", DSA计算流: a sequence shorter than top-k keeps all of
    its tokens).  Otherwise V is ordered by score descending, equal scores by
    position ascending (ties go to the lower index), and the first k are
    taken.  Returns ``(idx, tau)``: the chosen positions in ascending order,
    padded with -1 to length k, and the k-th largest score (``-inf`` when no
    position was dropped).
    """
    scores_row = np.asarray(scores_row, dtype=np.float64)
    n = int(pos) + 1
    vals = scores_row[:n]
    out = np.full(k, -1, dtype=np.int64)
    if n <= k:
        out[:n] = np.arange(n)
        return out, -np.inf
    order = np.lexsort((np.arange(n), -vals))
    chosen = order[:k]
    out[:] = np.sort(chosen)
    return out, float(vals[order[k - 1]])


def sparse_mla(q, q_fmt, kv, kv_fmt, idx, seq_lens, q_len, sm_scale,
               dv=512, rows=None):
    """Sparse MQA-mode MLA over the selected latent rows.

    "详解DSA" Eq.(2): ``u_t = Attn(h_t, {c_s : s in S_t})``; MQA mode ("DSA 怎样
    嵌入 MLA" on the charlestar page, MQA mode in section 3.1 of the luowle
    page): every query head attends to the same selected latent entries
    ``c_s`` (576 wide: 512 latent + 64 rope), the key is the whole entry and
    the value its first ``dv`` = 512 dims.  The softmax runs over the selected
    set only, in fp32-or-better as in the ``scores.softmax(dim=-1,
    dtype=torch.float32)`` line of the page's MLA forward.

    For each row t and head h over ``S_t = {idx[t, m] >= 0}``:
    ``z_m = sm_scale * q[t, h, :] . kv[b, s_m, :]``,
    ``out[t, h] = sum_m softmax(z)_m * kv[b, s_m, :dv]``,
    ``lse[t, h] = log sum_m exp(z_m)``.
    An empty set gives ``out = 0`` and ``lse = -inf``.

    Shapes: q [T, H, Dqk], kv [B, S_max, Dqk], idx [T, k].  Returns float64
    ``(out [R, H, dv], lse [R, H])``.
    """
    q = np.asarray(q)
    kv = np.asarray(kv)
    idx = np.asarray(idx)
    T, H, dqk = q.shape
    batch, pos = query_positions(seq_lens, q_len)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), H, dv))
    lse = np.full((len(rows), H), -np.inf)
    for r, t in enumerate(rows):
        sel = idx[t][idx[t] >= 0].astype(np.int64)
        if len(sel) == 0:
            continue
        if len(np.unique(sel)) != len(sel) or sel.max() > pos[t]:
            raise ValueError(f"row {t}: indices must be unique and <= pos")
        c = _decode(kv[batch[t], sel], kv_fmt)          # [m, Dqk]
        z = sm_scale * (_decode(q[t], q_fmt) @ c.T)     # [H, m]
        zmax = z.max(axis=1, keepdims=True)
        p = np.exp(z - zmax)
        l = p.sum(axis=1, keepdims=True)
        out[r] = (p @ c[:, :dv]) / l
        lse[r] = zmax[:, 0] + np.log(l[:, 0])
    return out, lse


def dsa_forward(qi, qi_fmt, w, w_fmt, ki, ki_fmt, qm, qm_fmt, kv, kv_fmt,
                seq_lens, q_len, topk, sm_scale, k_scale=None, q_scale=None,
                dv=512, rows=None):
    """Indexer -> top-k -> sparse MLA for the given rows (the two-stage data
    flow of the charlestar page, "DSA 的两段式数据流").

    Returns ``(idx [R, topk], tau [R], out [R, H, dv], lse [R, H],
    scores [R, S_max])``.
    """
    T = np.asarray(qi).shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    _, pos = query_positions(seq_lens, q_len)
    scores = indexer_scores(qi, qi_fmt, w, w_fmt, ki, ki_fmt, seq_lens, q_len,
                            k_scale=k_scale, q_scale=q_scale, rows=rows)
    idx_rows = np.full((len(rows), topk), -1, dtype=np.int64)
    tau = np.empty(len(rows))
    for r, t in enumerate(rows):
        idx_rows[r], tau[r] = topk_select(scores[r], pos[t], topk)
    idx_full = np.full((T, topk), -1, dtype=np.int64)
    idx_full[rows] = idx_rows
    out, lse = sparse_mla(qm, qm_fmt, kv, kv_fmt, idx_full, seq_lens, q_len,
                          sm_scale, dv=dv, rows=rows)
    return idx_rows, tau, out, lse, scores
