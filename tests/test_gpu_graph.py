"""dsa_forward under HIP graph capture (torch.cuda.CUDAGraph on ROCm) on the
128K decode workload: every buffer is allocated before capture, the path
makes no allocation, host synchronisation or memset, and each replay of the
captured step (with eager work and synchronisations between replays)
reproduces the eager call bit for bit.  The same for dsa_forward_noalloc,
whose scratch is the library's static array."""

import pytest
import torch

from synth import standard_workload
from tests.gpu_util import Uploaded

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("entry", ["forward", "forward_noalloc"])
def test_graph_capture_replays_the_decode_step(dsa_gpu, entry):
    lcl = dsa_gpu
    _say(f"[graph] decode128k, {entry}")
    wl = standard_workload("decode128k")
    up = Uploaded(wl)
    g = up.geom(lcl)
    T, H, k = wl.T, wl.H, wl.topk
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    kw = dict(index_k_scale=up.d_ks, idx=idx, out=out, lse=lse)
    if entry == "forward":
        kw["ws"] = torch.empty(lcl.forward_workspace_size(wl.B, wl.q_len, wl.S_max, H, k, lcl.FP8_E4M3FN, lcl.BF16),
                               dtype=torch.uint8, device="cuda")
    fn = getattr(lcl, entry)

    def step():
        fn(g, k, wl.sm_scale, up.d_qi, up.d_w, up.d_ki, up.d_qm, up.d_kv, **kw)

    step()  # eager reference (also the first call that looks up the static scratch)
    torch.cuda.synchronize()
    ref = (idx.clone(), out.clone(), lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        idx.fill_(-5)
        out.fill_(7.0)
        lse.fill_(1.0)
        step() if rep == 1 else None      # an eager step between replays
        torch.cuda.synchronize()
        idx.fill_(-5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]), f"replay {rep}: selection differs from the eager call"
        assert torch.equal(out.view(torch.int16), ref[1].view(torch.int16)), f"replay {rep}: output differs"
        assert torch.equal(lse, ref[2]), f"replay {rep}: lse differs"
    _say("  3 replays identical to the eager call")
