"""Helpers shared by the GPU parity tests: upload seeded workloads, compare
against the oracle with the stated tolerances."""

import numpy as np
import torch

from oracle import decode_bf16, indexer_scores, query_positions, sparse_mla, topk_select

# Tolerances of the DSA forward path (float64 oracle vs the HIP path):
SCORE_RTOL = 2e-2      # indexer scores, relative (fp8 inputs, fp32 accumulate)
SCORE_FLOOR = 1e-2     # ... relative to 1e-2 * row max where scores cancel toward 0
BAND_RTOL = 1e-3       # top-k: positions within 1e-3 relative of the k-th score are exempt
ATTN_ATOL = 1e-2       # attention output, max abs (bf16)


def to_dev(a, dev="cuda"):
    """numpy -> torch device tensor, keeping bit patterns (uint16 -> bfloat16)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def from_dev(t):
    if t.dtype == torch.bfloat16:
        u = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.cpu().numpy()


class Uploaded:
    """A workload's inputs as host arrays (the oracle's copies) and device tensors."""

    def __init__(self, wl, dev="cuda", with_mla=True, qm_rows=None):
        self.wl = wl
        self.qi = wl.qi()
        self.w = wl.w()
        self.ki, self.ks = wl.ki_all()
        self.d_qi, self.d_w, self.d_ki, self.d_ks = to_dev(self.qi), to_dev(self.w), to_dev(self.ki), to_dev(self.ks)
        self.d_seq = torch.from_numpy(wl.seq_lens.astype(np.int32)).to(dev)
        if with_mla:
            if qm_rows is None:
                self.qm = wl.qm()
            else:  # only the sampled rows carry the recipe's values, the rest are zero
                self.qm = np.zeros((wl.T, wl.H, 576), dtype=np.uint16 if wl.fp8 else np.float32)
                self.qm[qm_rows] = wl.qm(qm_rows)
            self.kv = wl.kv_all()
            self.d_qm, self.d_kv = to_dev(self.qm), to_dev(self.kv)

    def geom(self, lcl):
        return lcl.make_geom(self.wl.B, self.wl.q_len, self.wl.S_max, self.d_seq)

    def oracle_scores(self, rows=None):
        wl = self.wl
        return indexer_scores(self.qi, wl.qi_fmt, self.w, wl.w_fmt, self.ki, wl.ki_fmt, wl.seq_lens, wl.q_len,
                              k_scale=self.ks, rows=rows)


def check_scores(got, ref, pos):
    """Indexer verdict: within SCORE_RTOL relative (with a row-max floor) on
    valid entries, exactly -inf beyond pos."""
    worst = 0.0
    for r in range(ref.shape[0]):
        p = pos[r]
        if p >= 0:
            o, g = ref[r, :p + 1], got[r, :p + 1].astype(np.float64)
            floor = SCORE_FLOOR * np.abs(o).max()
            err = np.abs(g - o) / np.maximum(np.abs(o), max(floor, 1e-30))
            worst = max(worst, float(err.max()))
            assert np.all(np.isfinite(g)), f"row {r}: non-finite score in the valid range"
        assert np.all(np.isneginf(got[r, p + 1:ref.shape[1]])), f"row {r}: masked entries must be -inf"
    assert worst <= SCORE_RTOL, f"score error {worst:.3g} > {SCORE_RTOL}"
    return worst


def check_topk(idx_gpu, ref_scores, pos, k):
    """Top-k verdict against oracle scores: identical outside the 1e-3 band,
    same size, valid, unique, ascending."""
    n_band = 0
    for r in range(ref_scores.shape[0]):
        got = idx_gpu[r]
        sel = got[got >= 0]
        n = pos[r] + 1
        want, tau = topk_select(ref_scores[r], pos[r], k)
        want = want[want >= 0]
        assert len(sel) == len(want) == min(n, k), f"row {r}: {len(sel)} selected, expected {min(n, k)}"
        assert np.all(got[len(sel):] == -1), f"row {r}: padding must be -1"
        assert np.all(np.diff(sel) > 0), f"row {r}: indices must be ascending and unique"
        assert sel.min() >= 0 and sel.max() <= pos[r], f"row {r}: index out of range"
        if n <= k:
            assert np.array_equal(sel, np.arange(n)), f"row {r}: short row must keep every position"
            continue
        row = ref_scores[r, :n]
        scale = max(abs(tau), 1e-6 * np.abs(row).max())
        band = np.abs(row - tau) <= BAND_RTOL * scale
        gs = np.zeros(n, bool)
        gs[sel] = True
        os_ = np.zeros(n, bool)
        os_[want] = True
        diff = (gs != os_) & ~band
        assert not diff.any(), f"row {r}: {int(diff.sum())} selection differences outside the band"
        n_band += int(((gs != os_) & band).sum())
    return n_band


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def attention_tolerance(ref, bf16_output):
    """1e-2 absolute.  For a bf16 output the bound is raised to half a bf16
    ulp of the exact value where that is larger (|x| >= 4): the nearest bf16
    number to x is within half an ulp, and no closer one need exist."""
    if not bf16_output:
        return ATTN_ATOL
    return np.maximum(ATTN_ATOL, 0.5 * bf16_ulp(ref))


U_BF16 = 2.0 ** -9   # unit roundoff of bfloat16 (round to nearest, ties to even)


def weight_rounding_bound(qm, qm_fmt, kv, kv_fmt, b, sel, t, h, sm_scale):
    """Per value dim: the most the bf16 rounding of the attention weights can
    move an exact output, u/(1-u) * sum_m p_m |v_m - o|.  The pages' MLA
    forward casts the fp32 softmax to the value dtype before the value
    product ("详解DSA", MLA code block: scores.type_as(x)); with the weights
    p_m (1 + d_m), |d_m| <= u, and the normaliser summing the same rounded
    weights, the output moves by sum_m p_m d_m (v_m - o) / sum_m p_m (1 + d_m).
    A 10% margin covers the fp32 score and accumulation error."""
    c = decode_bf16(kv[b, sel]) if kv_fmt == "bf16" else np.asarray(kv[b, sel], np.float64)
    q = decode_bf16(qm[t, h]) if qm_fmt == "bf16" else np.asarray(qm[t, h], np.float64)
    z = sm_scale * (c @ q)
    p = np.exp(z - z.max())
    p /= p.sum()
    v = c[:, :512]
    o = p @ v
    return 1.1 * U_BF16 / (1 - U_BF16) * (p @ np.abs(v - o)) + 1e-6 * np.abs(v).max()


def check_attention(out_gpu, lse_gpu, up, idx, rows):
    """Attention verdict on the GPU's own index sets: |out - oracle| within
    attention_tolerance elementwise; a bf16 element beyond it may exceed half
    an ulp only by the weight-rounding bound of its (row, head), the case of
    an exact value within that bound of a bf16 rounding midpoint.  lse within
    1e-2."""
    wl = up.wl
    idx_full = np.full((wl.T, idx.shape[1]), -1, dtype=np.int64)
    idx_full[rows] = idx
    ref, ref_lse = sparse_mla(up.qm, wl.qm_fmt, up.kv, wl.kv_fmt, idx_full, wl.seq_lens, wl.q_len, wl.sm_scale,
                              rows=rows)
    err = np.abs(out_gpu - ref)
    bf16 = wl.qm_fmt == "bf16"
    tol = attention_tolerance(ref, bf16)
    bad = err > tol
    n_allow = 0
    if bf16 and bad.any():
        batch, _ = query_positions(wl.seq_lens, wl.q_len)
        for r, h in sorted(set(zip(*np.nonzero(bad.any(axis=2))))):
            t = int(np.asarray(rows)[r])
            sel = idx_full[t][idx_full[t] >= 0]
            eps = weight_rounding_bound(up.qm, wl.qm_fmt, up.kv, wl.kv_fmt, int(batch[t]), sel, t, h, wl.sm_scale)
            allow = 0.5 * bf16_ulp(ref[r, h]) + eps
            n_allow += int((bad[r, h] & (err[r, h] <= allow)).sum())
            bad[r, h] &= err[r, h] > allow
    assert not bad.any(), (f"attention error {err[bad].max():.3g} above tolerance at {int(bad.sum())} elements "
                           f"(max abs error {err.max():.3g})")
    err_max = float(err.max())
    small = np.abs(ref) < 2.0
    err_small = float(err[small].max()) if small.any() else 0.0
    print(f"  attention: max |out - oracle| = {err_max:.3g} (max |ref| = {np.abs(ref).max():.3g}; "
          f"{err_small:.3g} where |ref| < 2; {n_allow} elements within the weight-rounding allowance)", flush=True)
    if lse_gpu is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(lse_gpu), fin)
        lerr = np.abs(lse_gpu[fin] - ref_lse[fin]).max() if fin.any() else 0.0
        assert lerr <= 1e-2, f"lse error {lerr:.3g}"
    return err_max
