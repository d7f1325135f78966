"""Indexer KL objective, forward only (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"详解DSA", the two-stage training passage, Eq.(3)-(6) (restated by the
charlestar page's "Dense warm-up" / "Sparse training" sections and the
luowle page's section 3.3):

* Eq.(3): the target of query t is the main attention's scores summed over
  all heads, L1-normalised over the positions: ``p = v / sum(v)`` with
  ``v_s = sum_h AttentionScore^(h)_{t,s}``;
* Eq.(4): the indexer's prediction ``p_hat = Softmax(I_{t,:})``;
* Eq.(5): dense warm-up, ``L = sum_t KL(p_t || p_hat_t)`` over every visible
  position (s <= pos);
* Eq.(6): sparse training, the same over the selected set S_t only.

Readings (the pages leave these open): AttentionScore^(h) is head h's
attention weight ``exp(z_h,s - lse_h)`` with ``z_h,s = sm_scale * q_h . c_s``
(MQA mode: the 576-wide latent entry is every head's key) and ``lse_h`` the
log-sum-exp the attention itself used, an input here as a training step has
it from the attention forward; on S_t both distributions are normalised over
S_t (the attention only saw S_t, and Softmax(I_{t,S_t}) is over S_t).
``KL(p || q) = sum_s p_s log(p_s / q_s)`` with ``0 log 0 = 0``.
"""

import numpy as np

from .dsa import _decode, query_positions


def indexer_kl(q, q_fmt, kv, kv_fmt, lse, scores, idx, seq_lens, q_len, sm_scale, rows=None):
    """Per-row KL of Eq.(5) (``idx`` None: every position s <= pos) or
    Eq.(6) (``idx`` [T, k]: the entries ``0 <= idx <= pos``; -1 skipped).

    ``q`` [T, H, 576], ``kv`` [B, S_max, 576] (MQA-mode attention inputs),
    ``lse`` [T, H] natural-log normalisers of the attention, ``scores``
    [T, >= S_max] indexer scores I.  Returns float64 ``(kl [R], sum)``; a row
    with an empty set has KL 0.
    """
    qd = _decode(q, q_fmt)
    kvd = _decode(kv, kv_fmt)
    lse = np.asarray(lse, dtype=np.float64)
    scores = np.asarray(scores, dtype=np.float64)
    T = qd.shape[0]
    batch, pos = query_positions(seq_lens, q_len)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    kl = np.zeros(len(rows))
    for r, t in enumerate(rows):
        if idx is None:
            sel = np.arange(pos[t] + 1)
        else:
            row = np.asarray(idx[t]).astype(np.int64)
            sel = row[(row >= 0) & (row <= pos[t])]
            if len(np.unique(sel)) != len(sel):
                raise ValueError(f"row {t}: duplicate positions")
        if len(sel) == 0:
            continue
        z = sm_scale * (qd[t] @ kvd[batch[t], sel].T)                 # [H, n]
        v = np.exp(z - lse[t][:, None]).sum(axis=0)                    # Eq.(3) before the normalisation
        p = v / v.sum()
        i_sel = scores[t, sel]
        log_phat = i_sel - (i_sel.max() + np.log(np.exp(i_sel - i_sel.max()).sum()))   # Eq.(4)
        nz = p > 0
        kl[r] = np.sum(p[nz] * (np.log(p[nz]) - log_phat[nz]))         # Eq.(5) / (6)
    return kl, float(kl.sum())


def attention_lse(q, q_fmt, kv, kv_fmt, idx, seq_lens, q_len, sm_scale):
    """Per-head natural-log normaliser of MQA-mode attention over the same
    set as ``indexer_kl`` (None: every s <= pos): ``log sum_s exp(z_h,s)``
    (-inf for an empty set).  Test input for ``indexer_kl``."""
    qd = _decode(q, q_fmt)
    kvd = _decode(kv, kv_fmt)
    T, H, _ = qd.shape
    batch, pos = query_positions(seq_lens, q_len)
    out = np.full((T, H), -np.inf)
    for t in range(T):
        if idx is None:
            sel = np.arange(pos[t] + 1)
        else:
            row = np.asarray(idx[t]).astype(np.int64)
            sel = row[(row >= 0) & (row <= pos[t])]
        if len(sel) == 0:
            continue
        z = sm_scale * (qd[t] @ kvd[batch[t], sel].T)
        m = z.max(axis=1)
        out[t] = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    return out
