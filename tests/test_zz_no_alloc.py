"""GPU check of dsa_forward_noalloc (through the C ABI): on the same inputs
it gives exactly what dsa_forward gives with a workspace of its own (same
kernels, same plan, the scratch in the library's static array instead),
on consecutive calls of decreasing size (the second call runs on what the
first left in the array), and a streamed prefill shape; the first case is
also checked against the oracle.  A call that needs more than the array
holds returns DSA_ERR_WORKSPACE."""

import numpy as np
import pytest
import torch

from synth import make_workload
from tests.gpu_util import Uploaded, check_attention, check_topk, from_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


CASES = [
    # name, B, q_len, seq_lens, S_max, topk, H, ki_mode
    ("decode_big", 4, 2, [20000, 17001, 20000, 9000], 20000, 2048, 128, "pool"),
    ("decode_small", 2, 1, [5000, 3000], 5000, 512, 64, "normal"),
    ("prefill_streamed", 1, 700, [700], 700, 128, 16, "normal"),
]


def _run_both(lcl, wl, up, idx_out=True):
    g = up.geom(lcl)
    T, H, k = wl.T, wl.H, wl.topk
    outs = []
    for fn in (lcl.forward, lcl.forward_noalloc):
        idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda") if idx_out else False
        out = torch.full((T, H, 512), 3.0, dtype=torch.bfloat16, device="cuda")
        lse = torch.full((T, H), 5.0, dtype=torch.float32, device="cuda")
        res = fn(g, k, wl.sm_scale, up.d_qi, up.d_w, up.d_ki, up.d_qm, up.d_kv, index_k_scale=up.d_ks, idx=idx,
                 out=out, lse=lse)
        torch.cuda.synchronize()
        outs.append(res)
    return outs


def test_forward_noalloc_equals_forward(dsa_gpu):
    lcl = dsa_gpu
    for n, (name, B, q_len, seq, S, k, H, mode) in enumerate(CASES):
        _say(f"[noalloc] {name}")
        wl = make_workload(name, B, q_len, seq, S, k, H, seed=61 + n, ki_mode=mode)
        up = Uploaded(wl)
        need = lcl.forward_workspace_size(B, q_len, S, H, k, lcl.FP8_E4M3FN, lcl.BF16)
        assert need <= lcl.NOALLOC_SCRATCH_BYTES
        (i0, o0, l0), (i1, o1, l1) = _run_both(lcl, wl, up)
        assert torch.equal(i0, i1), "selection differs from dsa_forward"
        assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)), "output differs from dsa_forward"
        assert torch.equal(l0, l1), "lse differs from dsa_forward"
        if n == 0:
            gi = i1.cpu().numpy()
            check_topk(gi, up.oracle_scores(), wl.positions(), k)
            check_attention(from_dev(o1), l1.cpu().numpy(), up, gi.astype(np.int64), np.arange(wl.T))
        if n == 1:  # idx_out = NULL: the selection lives in the scratch array too
            (_, o2, l2), (_, o3, l3) = _run_both(lcl, wl, up, idx_out=False)
            assert torch.equal(o2.view(torch.int16), o3.view(torch.int16)) and torch.equal(l2, l3)
            assert torch.equal(o0.view(torch.int16), o3.view(torch.int16))


def test_forward_noalloc_rejects_what_does_not_fit(dsa_gpu):
    lcl = dsa_gpu
    _say("[noalloc] too large: an 8192-token prefill")
    B, L, H, k = 1, 8192, 128, 2048
    assert lcl.forward_workspace_size(B, L, L, H, k, lcl.FP8_E4M3FN, lcl.BF16) > lcl.NOALLOC_SCRATCH_BYTES
    seq = torch.full((B,), L, dtype=torch.int32, device="cuda")
    g = lcl.make_geom(B, L, L, seq)
    qi = torch.zeros((L, 64, 128), dtype=torch.uint8, device="cuda")
    w = torch.zeros((L, 64), dtype=torch.bfloat16, device="cuda")
    ki = torch.zeros((B, L, 128), dtype=torch.uint8, device="cuda")
    qm = torch.zeros((L, H, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, L, 576), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lcl.DsaError) as e:
        lcl.forward_noalloc(g, k, 0.07, qi, w, ki, qm, kv)
    assert e.value.status == 3
