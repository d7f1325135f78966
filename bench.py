#!/usr/bin/env python3
"""Benchmark of the DSA forward path (indexer -> top-k -> sparse MQA-MLA) on
one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-prefill] [--no-cpu-baseline]

One step = one dsa_forward over one batch of the 128K-context decode workload
(16 sequences x 2 new queries, context 131072, indexer 64x128 fp8 with
per-token scales, top-k 2048, 128-head sparse MLA over the bf16 576-wide
latent cache).  Inputs are seeded synthetic data resident in HBM before the
timed region.  Before every step a 512 MiB buffer is read (not written, so no
dirty lines are left to write back) so the 256 MiB last-level cache does not
hold the previous step's caches; each step is timed with HIP events on the
launch stream and ms_per_step is their mean.

Prints ONE JSON line with the headline decode throughput, per-stage timings
and roofline fractions, the 64K-token prefill throughput, and the float64
CPU oracle timed on a bounded sample of the decode workload.
"""

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-scrub", action="store_true", help="do not evict the last-level cache between steps")
    ap.add_argument("--prefill-steps", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="run the CPU oracle on whole decode sequences until this much time has passed")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 256 MiB device copy (a known-size kernel for HBM counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the work; --gpus {args.gpus} is not supported "
              f"(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import long_context_lightning_amd as lcl
    from synth import standard_workload

    lcl.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.copy_probe:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)  # 256 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: 268435456 bytes read, 268435456 bytes written")
        del src, dst

    # ------------------------------------------------------------ decode 128K
    wl = standard_workload("decode128k")
    log(f"generating {wl.name}: B={wl.B} q_len={wl.q_len} S={wl.S_max} k={wl.topk} H={wl.H}")
    t0 = time.time()
    qi, w = wl.qi(), wl.w()
    ki, ks = wl.ki_all()
    qm = wl.qm()
    kv = wl.kv_all()
    log(f"generated in {time.time() - t0:.1f}s; uploading")

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    d = dict(qi=up(qi), w=up(w), ki=up(ki), ks=up(ks), qm=up(qm), kv=up(kv),
             seq=torch.from_numpy(wl.seq_lens.astype(np.int32)).to(dev))
    del kv
    geom = lcl.make_geom(wl.B, wl.q_len, wl.S_max, d["seq"])
    T, k, H = wl.T, wl.topk, wl.H
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.empty(lcl.forward_workspace_size(wl.B, wl.q_len, wl.S_max, H, k, lcl.FP8_E4M3FN, lcl.BF16),
                     dtype=torch.uint8, device=dev)
    scrub = torch.ones(128 << 20, dtype=torch.float32, device=dev)  # 512 MiB
    scrub_out = torch.empty(1, dtype=torch.float32, device=dev)

    def forward():
        lcl.forward(geom, k, wl.sm_scale, d["qi"], d["w"], d["ki"], d["qm"], d["kv"], index_k_scale=d["ks"],
                    idx=idx, out=out, lse=lse, ws=ws)

    def evict():
        if not args.no_scrub:
            torch.sum(scrub, dim=0, out=scrub_out[0])

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        evict()
        forward()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        evict()
        ev[i][0].record(stream)
        forward()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [a.elapsed_time(b) for a, b in ev]
    ms = sum(step_ms) / len(step_ms)
    value = T / (ms / 1e3)
    log(f"decode forward: {ms * 1e3:.1f} us/step -> {value:,.0f} queries/s (wall {wall:.3f}s incl. scrubs)")

    # Per-stage timing: the same kernels through the three stage calls.
    scores = ws[: T * wl.S_max * 4].view(torch.float32).view(T, wl.S_max)
    tk_ws = torch.empty(max(lcl.topk_workspace_size(T, wl.S_max, k), 256), dtype=torch.uint8, device=dev)
    mla_ws = torch.empty(max(lcl.sparse_mla_workspace_size(wl.B, wl.q_len, H, k, lcl.BF16), 256),
                         dtype=torch.uint8, device=dev)
    st = {n: [] for n in ("indexer", "topk", "sparse_mla")}
    for i in range(args.warmup + args.steps):
        evict()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        lcl.indexer_scores(geom, d["qi"], d["w"], d["ki"], k_scale=d["ks"], scores=scores)
        e[1].record(stream)
        lcl.topk(geom, scores, k, idx=idx, ws=tk_ws)
        e[2].record(stream)
        lcl.sparse_mla(geom, d["qm"], d["kv"], idx, wl.sm_scale, out=out, lse=lse, ws=mla_ws)
        e[3].record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            st["indexer"].append(e[0].elapsed_time(e[1]))
            st["topk"].append(e[1].elapsed_time(e[2]))
            st["sparse_mla"].append(e[2].elapsed_time(e[3]))
    st_ms = {n: sum(v) / len(v) for n, v in st.items()}
    # algorithmic bytes per launch (decode is HBM-bound)
    idx_bytes = wl.B * wl.S_max * (128 + 4)
    topk_bytes = T * wl.S_max * 4
    mla_bytes = T * k * 1152 + T * H * 576 * 2 + T * H * 512 * 2 + T * k * 4
    stage_bytes = {"indexer": idx_bytes, "topk": topk_bytes, "sparse_mla": mla_bytes}
    stages = {}
    for n in st_ms:
        gbs = stage_bytes[n] / (st_ms[n] * 1e-3) / 1e9
        stages[n] = {"us": round(st_ms[n] * 1e3, 2), "bytes": stage_bytes[n], "GB_s": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        log(f"  {n:10s} {st_ms[n] * 1e3:8.1f} us  {gbs:8.1f} GB/s  ({gbs / HBM_PEAK_GBS:.1%} of HBM peak)")
    # The longest kernel of a decode step is the indexer's, k_indexer_fp8.
    # In the timed step it runs right after the last-level cache scrub, so its
    # launch duration is taken in that same condition: the event pair around
    # the single dsa_indexer_scores launch of each stage step above (the
    # step's own launch also clears the top-k counters, a few KB).  The rate
    # of 10 back-to-back launches (no scrub between them) is reported beside
    # it for context.  Its measured HBM traffic per launch comes from the
    # committed counter summary, valid only for the sources it was taken on.
    reps = 10
    evict()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record(stream)
    for _ in range(reps):
        lcl.indexer_scores(geom, d["qi"], d["w"], d["ki"], k_scale=d["ks"], scores=scores)
    e[1].record(stream)
    torch.cuda.synchronize()
    b2b_us = e[0].elapsed_time(e[1]) * 1e3 / reps
    dom_us = st_ms["indexer"] * 1e3
    dom_gbs = stage_bytes["indexer"] / (dom_us * 1e-6) / 1e9
    log(f"  k_indexer_fp8 in the step (after the scrub): {dom_us:.1f} us/launch = {dom_gbs:.1f} GB/s; "
        f"back-to-back {b2b_us:.1f} us/launch = {stage_bytes['indexer'] / (b2b_us * 1e-6) / 1e9:.1f} GB/s")
    roofline = {"kernel": "k_indexer_fp8 (decode128k, 32 rows x 131072 keys, after the LLC scrub as in the step)",
                "bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "us_per_launch": round(dom_us, 2),
                "back_to_back_us_per_launch": round(b2b_us, 2),
                "traffic": measured_traffic("indexer_fp8_decode128k")}
    del scores

    # ------------------------------------------- paged caches, same decode
    paged = bench_paged(args, lcl, torch, np, dev, stream, evict, wl, d, geom, idx, out, lse, ms)

    # ------------------------------------------- fp8 quantisation / append
    quant = bench_quant(lcl, torch, dev, stream, evict, wl)

    # ------------------------------------ short prefill: MHA mode vs MQA mode
    mha = bench_mha(lcl, torch, dev, stream, evict)

    # ------------------------------------------------ indexer KL objective
    kl = bench_kl(lcl, torch, dev, stream, evict)

    # ---------------------------- the other decode and prefill configurations
    del d, idx, out, lse, ws, tk_ws, mla_ws
    torch.cuda.empty_cache()
    other = {
        "decode32k": bench_forward_config(lcl, torch, dev, stream, evict, "decode32k: 64 seqs x 1 query, ctx 32768",
                                          B=64, q_len=1, S=32768, k=2048, H=128, steps=args.steps, unit="queries/s"),
        "prefill8k": bench_forward_config(lcl, torch, dev, stream, evict, "prefill8k: 1 x 8192 causal",
                                          B=1, q_len=8192, S=8192, k=2048, H=128, steps=max(3, args.steps // 4),
                                          unit="tokens/s"),
    }

    # --------------------------------------------------------- prefill 64K
    prefill = None
    if not args.no_prefill:
        prefill = bench_prefill(args, lcl, torch, np, dev, stream, evict)

    # ------------------------------------------------------ CPU baseline
    cpu = cpu_other = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, qi, w, ki, ks, qm, np, args.cpu_seconds)
        cpu_other = cpu_baseline_configs(np, args.cpu_seconds)

    line = {
        "metric": "DSA decode queries/s @128K ctx (dsa_forward: indexer + top-k + sparse MLA)",
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 indexer / fp32 accumulate / bf16 attention",
        "data": "synthetic (seeded; shapes and distributions of the 128K decode workload)",
        "config": {"workload": "decode128k: 16 seqs x 2 queries, ctx 131072, indexer 64x128 fp8, top-k 2048, "
                               "128-head MQA-MLA bf16 576/512",
                   "batch_queries": T, "context": wl.S_max, "topk": k, "heads": H,
                   "llc_scrub_between_steps": not args.no_scrub},
        "roofline": roofline,
        "stages": stages,
        "quantize": quant,
        "paged": paged,
        "mha_prefill": mha,
        "indexer_kl": kl,
        "other_configs": other,
        "prefill": prefill,
        "cpu_baseline": cpu,
        "cpu_baseline_configs": cpu_other,
        "workspace_bytes": lcl.forward_workspace_size(wl.B, wl.q_len, wl.S_max, H, k, lcl.FP8_E4M3FN, lcl.BF16),
        "system": system_info(torch, lcl),
    }
    print(json.dumps(line), flush=True)


def bench_paged(args, lcl, torch, np, dev, stream, evict, wl, d, geom, idx, out, lse, contiguous_ms):
    """The same 128K decode step on paged caches (dsa_forward_paged): the
    three caches copied into pools of 64-token pages in the scattered order of
    a seeded block table, timed like the contiguous step (LLC eviction before
    each step, event pair around it), plus its two paged stages alone."""
    from synth import make_block_table
    P = 64
    _, clean, num_pages = make_block_table(10, wl.B, wl.seq_lens, wl.S_max, P)
    table = torch.from_numpy(clean).to(dev)
    dst = torch.from_numpy(clean.reshape(-1).astype(np.int64)).to(dev)

    def pool(c, tail):
        p = torch.zeros((num_pages, P) + tail, dtype=c.dtype, device=dev)
        return p.index_copy_(0, dst, c.reshape((-1, P) + tail))

    ki_pool, ks_pool, kv_pool = pool(d["ki"], (128,)), pool(d["ks"], ()), pool(d["kv"], (576,))
    pages = lcl.make_pages(table, P, num_pages)
    T, k, H = wl.T, wl.topk, wl.H
    ws = torch.empty(lcl.forward_paged_workspace_size(wl.B, wl.q_len, wl.S_max, H, k, lcl.FP8_E4M3FN, lcl.BF16),
                     dtype=torch.uint8, device=dev)

    def forward():
        lcl.forward(geom, k, wl.sm_scale, d["qi"], d["w"], ki_pool, d["qm"], kv_pool, index_k_scale=ks_pool,
                    idx=idx, out=out, lse=lse, ws=ws, pages=pages)

    for _ in range(args.warmup):
        evict()
        forward()
    torch.cuda.synchronize()
    scores = torch.empty((T, wl.S_max), dtype=torch.float32, device=dev)
    mla_ws = torch.empty(max(lcl.sparse_mla_paged_workspace_size(wl.B, wl.q_len, H, k, lcl.BF16), 256),
                         dtype=torch.uint8, device=dev)
    st = {n: [] for n in ("forward", "indexer", "sparse_mla")}
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        evict()
        e[0].record(stream)
        forward()
        e[1].record(stream)
        evict()
        e[2].record(stream)
        lcl.indexer_scores(geom, d["qi"], d["w"], ki_pool, k_scale=ks_pool, scores=scores, pages=pages)
        e[3].record(stream)
        evict()
        e[4].record(stream)
        lcl.sparse_mla(geom, d["qm"], kv_pool, idx, wl.sm_scale, out=out, lse=lse, ws=mla_ws, pages=pages)
        e[5].record(stream)
        torch.cuda.synchronize()
        st["forward"].append(e[0].elapsed_time(e[1]))
        st["indexer"].append(e[2].elapsed_time(e[3]))
        st["sparse_mla"].append(e[4].elapsed_time(e[5]))
    us = {n: sum(v) / len(v) * 1e3 for n, v in st.items()}
    qps = T / (us["forward"] * 1e-6)
    log(f"paged decode (64-token pages): {us['forward']:.1f} us/step -> {qps:,.0f} queries/s "
        f"({us['forward'] / (contiguous_ms * 1e3):.3f}x the contiguous step); indexer {us['indexer']:.1f} us, "
        f"sparse MLA incl. page-row translation {us['sparse_mla']:.1f} us")
    del ki_pool, ks_pool, kv_pool, ws, scores, mla_ws
    torch.cuda.empty_cache()
    return {"page_size": P, "num_pages": int(num_pages), "us_per_step": round(us["forward"], 2),
            "queries_per_s": round(qps, 1), "vs_contiguous_step": round(us["forward"] / (contiguous_ms * 1e3), 4),
            "indexer_us": round(us["indexer"], 2), "sparse_mla_us": round(us["sparse_mla"], 2)}


def bench_mha(lcl, torch, dev, stream, evict, steps=5):
    """Prefill of 4 prompts of 2048 tokens (= top-k, so every position is
    kept) with 128 heads, both ways: dsa_mha_prefill (MHA mode: wkv_b
    decompression + causal attention over 192/128-dim heads) and dsa_forward
    in MQA mode on the absorbed shapes (the indexer is bypassed there, since
    S_max <= top-k; the attention covers every position with 576/512-dim
    entries).  Inputs drawn on the GPU with torch's seeded generator: q, the
    latent cache and the MQA queries ~ N(0,1) bf16, wkv_b ~ N(0, 1/512) bf16.
    Each call is timed after a last-level cache eviction (mean of `steps`)."""
    B, L, H, k = 4, 2048, 128, 2048
    T = B * L
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    q = torch.randn((T, H, 192), generator=g, device=dev).to(torch.bfloat16)
    kv = torch.randn((B, L, 576), generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn((H, 256, 512), generator=g, device=dev) / math.sqrt(512.0)).to(torch.bfloat16)
    seq = torch.full((B,), L, dtype=torch.int32, device=dev)
    geom = lcl.make_geom(B, L, L, seq)
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(lcl.mha_prefill_workspace_size(B, L, H), dtype=torch.uint8, device=dev)
    sm = 1.0 / math.sqrt(192.0)

    def timed(fn):
        fn()
        ts = []
        for _ in range(steps):
            evict()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            fn()
            e[1].record(stream)
            torch.cuda.synchronize()
            ts.append(e[0].elapsed_time(e[1]) * 1e3)
        return sum(ts) / len(ts)

    mha_us = timed(lambda: lcl.mha_prefill(geom, q, kv, w, sm, out=out, ws=ws, want_lse=False))
    del q, out, ws
    qm = torch.randn((T, H, 576), generator=g, device=dev).to(torch.bfloat16)
    qi = torch.zeros((T, 64, 128), dtype=torch.uint8, device=dev)     # unused: the indexer is bypassed
    wi = torch.zeros((T, 64), dtype=torch.bfloat16, device=dev)
    ki = torch.zeros((B, L, 128), dtype=torch.uint8, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    outm = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    fws = torch.empty(lcl.forward_workspace_size(B, L, L, H, k, lcl.FP8_E4M3FN, lcl.BF16), dtype=torch.uint8,
                      device=dev)
    mqa_us = timed(lambda: lcl.forward(geom, k, sm, qi, wi, ki, qm, kv, idx=idx, out=outm, ws=fws, want_lse=False))
    del qm, qi, wi, ki, idx, outm, fws
    torch.cuda.empty_cache()
    pairs = B * L * (L + 1) // 2
    mha_flop = B * L * H * 256 * 512 * 2 + pairs * H * (192 + 128) * 2
    mqa_flop = pairs * H * (576 + 512) * 2
    log(f"short prefill 4 x 2048 (<= top-k): MHA mode {mha_us:.1f} us ({mha_flop / 1e12:.3f} TFLOP, "
        f"{mha_flop / (mha_us * 1e-6) / 1e12:.1f} TFLOP/s); MQA-mode forward {mqa_us:.1f} us "
        f"({mqa_flop / 1e12:.3f} TFLOP); MHA mode {mqa_us / mha_us:.2f}x faster")
    return {"workload": "4 prompts x 2048 tokens (= top-k), 128 heads", "mha_us": round(mha_us, 1),
            "mha_tokens_per_s": round(T / (mha_us * 1e-6), 1), "mha_tflop": round(mha_flop / 1e12, 4),
            "mha_tflops": round(mha_flop / (mha_us * 1e-6) / 1e12, 1), "mqa_forward_us": round(mqa_us, 1),
            "mqa_tflop": round(mqa_flop / 1e12, 4), "mha_speedup": round(mqa_us / mha_us, 3)}


def system_info(torch, lcl):
    """Versions and target of the run: HIP runtime, torch, device and gfx
    architecture, library version."""
    props = torch.cuda.get_device_properties(0)
    return {"device": props.name, "gfx": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count,
            "hip": torch.version.hip, "torch": torch.__version__, "libdsa": lcl.load().dsa_version().decode()}


def bench_forward_config(lcl, torch, dev, stream, evict, label, B, q_len, S, k, H, steps, unit):
    """dsa_forward on another of the five configurations, inputs drawn on the
    GPU with torch's seeded generator following the decode recipe (indexer q
    and k ~ N(0,1) -> e4m3, k with per-token amax/448 scales, w ~ N(0,1)/8
    bf16, MLA q and latent cache ~ N(0,1) bf16; full cache lengths).  Two
    warm-up steps, then the mean of `steps`, each after the cache scrub.
    Returns the rate in queries/s (decode) or tokens/s (prefill)."""
    T = B * q_len
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    qi = torch.randn((T, 64, 128), generator=g, device=dev).to(torch.float8_e4m3fn)
    ki = torch.empty((B, S, 128), dtype=torch.float8_e4m3fn, device=dev)
    ks = torch.empty((B, S), dtype=torch.float32, device=dev)
    for b in range(B):
        kf = torch.randn((S, 128), generator=g, device=dev)
        ks[b] = (kf.abs().amax(dim=-1).clamp_min(2.0 ** -126) / 448.0).float()
        ki[b] = (kf / ks[b][:, None]).to(torch.float8_e4m3fn)
    w = (torch.randn((T, 64), generator=g, device=dev) / 8).to(torch.bfloat16)
    qm = torch.empty((T, H, 576), dtype=torch.bfloat16, device=dev)
    for r0 in range(0, T, 4096):
        qm[r0:r0 + 4096] = torch.randn((min(4096, T - r0), H, 576), generator=g, device=dev).to(torch.bfloat16)
    kv = torch.empty((B, S, 576), dtype=torch.bfloat16, device=dev)
    for b in range(B):
        kv[b] = torch.randn((S, 576), generator=g, device=dev).to(torch.bfloat16)
    seq = torch.full((B,), S, dtype=torch.int32, device=dev)
    geom = lcl.make_geom(B, q_len, S, seq)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(lcl.forward_workspace_size(B, q_len, S, H, k, lcl.FP8_E4M3FN, lcl.BF16), dtype=torch.uint8,
                     device=dev)
    sm = 1.0 / math.sqrt(192.0)

    def fwd():
        lcl.forward(geom, k, sm, qi, w, ki, qm, kv, index_k_scale=ks, idx=idx, out=out, ws=ws, want_lse=False)

    mla_ws = torch.empty(max(lcl.sparse_mla_workspace_size(B, q_len, H, k, lcl.BF16), 256), dtype=torch.uint8,
                         device=dev)
    sel = torch.empty_like(idx)
    sel_ws = torch.empty(max(lcl.indexer_topk_workspace_size(B, q_len, S, k, lcl.FP8_E4M3FN), 256),
                         dtype=torch.uint8, device=dev)

    def mla():
        lcl.sparse_mla(geom, qm, kv, idx, sm, out=out, ws=mla_ws, want_lse=False)

    def select():
        lcl.indexer_topk(geom, k, qi, w, ki, index_k_scale=ks, idx=sel, ws=sel_ws)

    for _ in range(2):
        evict()
        fwd()
    ts, tm, tsel = [], [], []
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        evict()
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        evict()
        e[2].record(stream)
        mla()
        e[3].record(stream)
        evict()
        e[4].record(stream)
        select()
        e[5].record(stream)
        torch.cuda.synchronize()
        ts.append(e[0].elapsed_time(e[1]))
        tm.append(e[2].elapsed_time(e[3]))
        tsel.append(e[4].elapsed_time(e[5]))
    ms = sum(ts) / len(ts)
    mla_ms = sum(tm) / len(tm)
    sel_ms = sum(tsel) / len(tsel)
    rate = T / (ms * 1e-3)
    # roofline of the whole step: decode shapes against the HBM floor of the
    # algorithmic bytes, prefill shapes against the MFMA floor of the
    # algorithmic flops (indexer fp8, attention bf16)
    sel = sum(min(t + 1, k) for t in range(S - q_len, S)) * B
    if q_len == 1:
        idx_bytes = B * S * (128 + 4)
        mla_bytes = sel * 1152 + T * H * 576 * 2 + T * H * 512 * 2 + T * k * 4
        floor_us = (idx_bytes + T * S * 4 + mla_bytes) / (HBM_PEAK_GBS * 1e3)
        roof = {"bound": "hbm", "algorithmic_bytes": idx_bytes + T * S * 4 + mla_bytes,
                "floor_us": round(floor_us, 2), "frac": round(floor_us / (ms * 1e3), 4),
                "sparse_mla_us": round(mla_ms * 1e3, 2),
                "sparse_mla_hbm_frac": round(mla_bytes / (mla_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    else:
        pairs = B * q_len * (q_len + 1) // 2
        idx_flop, mla_flop = pairs * 64 * 128 * 2, sel * H * (576 + 512) * 2
        floor_ms = idx_flop / (FP8_PEAK_TFLOPS * 1e9) + mla_flop / (BF16_PEAK_TFLOPS * 1e9)
        # indexer + top-k timed as its own call (dsa_indexer_topk, the same
        # launches as inside the forward); the forward's attention is the rest
        i_ms = sel_ms
        a_ms = max(ms - i_ms, 1e-6)
        roof = {"bound": "mfma", "indexer_tflop": round(idx_flop / 1e12, 4), "sparse_mla_tflop": round(mla_flop / 1e12, 4),
                "floor_ms": round(floor_ms, 4), "frac": round(floor_ms / ms, 4),
                "indexer_topk_ms": round(i_ms, 3),
                "indexer_fp8_mfma_frac": round(idx_flop / (i_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                "sparse_mla_ms": round(a_ms, 3),
                "sparse_mla_bf16_mfma_frac": round(mla_flop / (a_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "sparse_mla_standalone_ms": round(mla_ms, 3)}
    log(f"{label}: {ms * 1e3:.1f} us/step -> {rate:,.0f} {unit}; roofline frac {roof['frac']:.3f} ({roof['bound']})")
    del qi, ki, ks, w, qm, kv, idx, out, ws, mla_ws
    torch.cuda.empty_cache()
    return {"workload": label, "us_per_step": round(ms * 1e3, 2), "value": round(rate, 1), "unit": unit,
            "steps": steps, "roofline": roof,
            "workspace_bytes": lcl.forward_workspace_size(B, q_len, S, H, k, lcl.FP8_E4M3FN, lcl.BF16)}


def bench_kl(lcl, torch, dev, stream, evict, steps=5):
    """The indexer's KL objective over the selected sets (Eq.(6)) for an
    8192-token prefill: 8192 query rows x top-2048 sets (selected by dsa_topk
    from the scores), 128 heads.  Inputs drawn on the GPU with torch's seeded
    generator: MLA queries and latent cache ~ N(0,1) bf16, indexer scores
    ~ N(0,4) fp32 (causally masked), per-head lse ~ 5 + N(0,1).  Timed per
    call after a last-level cache eviction (mean of `steps`)."""
    L, k, H = 8192, 2048, 128
    g = torch.Generator(device=dev)
    g.manual_seed(9)
    qm = torch.randn((L, H, 576), generator=g, device=dev).to(torch.bfloat16)
    kv = torch.randn((1, L, 576), generator=g, device=dev).to(torch.bfloat16)
    sc = torch.randn((L, L), generator=g, device=dev) * 2.0
    sc = torch.where(torch.arange(L, device=dev)[None, :] <= torch.arange(L, device=dev)[:, None], sc,
                     torch.tensor(float("-inf"), device=dev)).contiguous()
    lse = 5.0 + torch.randn((L, H), generator=g, device=dev)
    seq = torch.tensor([L], dtype=torch.int32, device=dev)
    geom = lcl.make_geom(1, L, L, seq)
    idx = lcl.topk(geom, sc, k)
    kl = torch.empty((L,), dtype=torch.float32, device=dev)
    loss = torch.empty((1,), dtype=torch.float32, device=dev)
    ws = torch.empty(max(lcl.indexer_kl_workspace_size(1, L, L, k), 256), dtype=torch.uint8, device=dev)
    sm = 1.0 / math.sqrt(192.0)

    def call():
        lcl.indexer_kl(geom, qm, kv, lse, sc, sm, idx=idx, kl=kl, loss=loss, ws=ws)

    call()
    ts = []
    for _ in range(steps):
        evict()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        call()
        e[1].record(stream)
        torch.cuda.synchronize()
        ts.append(e[0].elapsed_time(e[1]) * 1e3)
    us = sum(ts) / len(ts)
    entries = float((idx >= 0).sum().item())
    flop = entries * H * 576 * 2
    log(f"indexer KL (Eq.6) 8192 rows x top-{k}, {H} heads: {us:.1f} us, {flop / 1e12:.3f} TFLOP -> "
        f"{flop / (us * 1e-6) / 1e12:.1f} TFLOP/s ({flop / (us * 1e-6) / 2.5e15:.1%} of bf16 peak)")
    del qm, kv, sc, lse, idx, kl, loss, ws
    torch.cuda.empty_cache()
    return {"workload": "8192-token prefill, top-2048 sets, 128 heads", "us": round(us, 1),
            "tflop": round(flop / 1e12, 4), "tflops": round(flop / (us * 1e-6) / 1e12, 1),
            "mfma_frac": round(flop / (us * 1e-6) / 2.5e15, 4)}


def bench_quant(lcl, torch, dev, stream, evict, wl):
    """The indexer's fp8 quantisation kernels: the per-step key-cache append
    and query quantisation of the 128K decode step, and the query
    quantisation of a 64K-token prefill ([65536*64, 128] bf16 in, codes and
    scales out); each is timed as single launches, each after a last-level
    cache eviction (median of 20, or 10 for the prefill shape)."""
    T = wl.T
    g = torch.Generator(device=dev)
    g.manual_seed(5)

    def timed(fn, reps=20):
        ts = []
        for _ in range(reps + 3):
            evict()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            fn()
            e[1].record(stream)
            torch.cuda.synchronize()
            ts.append(e[0].elapsed_time(e[1]) * 1e3)
        ts = sorted(ts[3:])
        return ts[len(ts) // 2]

    seq = torch.full((wl.B,), wl.S_max, dtype=torch.int32, device=dev)
    geom = lcl.make_geom(wl.B, wl.q_len, wl.S_max, seq)
    k_new = torch.randn((wl.B, wl.q_len, 128), generator=g, device=dev).to(torch.bfloat16)
    kc = torch.zeros((wl.B, wl.S_max, 128), dtype=torch.uint8, device=dev)
    kcs = torch.zeros((wl.B, wl.S_max), dtype=torch.float32, device=dev)
    app_us = timed(lambda: lcl.indexer_cache_append(geom, k_new, kc, kcs))
    q_dec = torch.randn((T * 64, 128), generator=g, device=dev).to(torch.bfloat16)
    qd_us = timed(lambda: lcl.indexer_quantize(q_dec))
    del kc, kcs
    rows = 65536 * 64
    q_pf = torch.randn((rows, 128), generator=g, device=dev).to(torch.bfloat16)
    codes = torch.empty((rows, 128), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows,), dtype=torch.float32, device=dev)
    qp_us = timed(lambda: lcl.indexer_quantize(q_pf, codes=codes, scales=scales), reps=10)
    qp_bytes = rows * (128 * 2 + 128 + 4)
    qp_gbs = qp_bytes / (qp_us * 1e-6) / 1e9
    log(f"quantize: decode128k key append {app_us:.1f} us, decode128k q ({T * 64} rows) {qd_us:.1f} us; "
        f"prefill64k q ({rows} rows bf16) {qp_us:.1f} us = {qp_gbs:.1f} GB/s ({qp_gbs / HBM_PEAK_GBS:.1%} of HBM peak)")
    del q_pf, codes, scales
    return {"decode128k_key_append_us": round(app_us, 2), "decode128k_q_quantize_us": round(qd_us, 2),
            "prefill64k_q_quantize": {"us": round(qp_us, 2), "bytes": qp_bytes, "GB_s": round(qp_gbs, 1),
                                      "hbm_frac": round(qp_gbs / HBM_PEAK_GBS, 4)}}


def measured_traffic(name):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated against a
    plain copy) from profiles/<name>_traffic.txt, or None when that file is
    missing or was taken on different kernel sources."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"{name}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "|")):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    h = hashlib.sha256()
    for src in fields.get("sources", "").split():
        with open(os.path.join(here, src), "rb") as f:
            h.update(f.read())
    if not fields.get("sources") or h.hexdigest() != fields.get("sources_sha256"):
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def bench_prefill(args, lcl, torch, np, dev, stream, evict):
    """64K-token causal prefill; inputs drawn on the GPU with torch's seeded
    generator following the same recipe (q, k ~ N(0,1) -> e4m3 with per-token
    k scales, w ~ N(0,1)/8 bf16, MLA q and cache ~ N(0,1) bf16)."""
    L, k, H = 65536, 2048, 128
    log(f"prefill: L={L} k={k} H={H}; drawing inputs on the GPU")
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    qi = torch.randn((L, 64, 128), generator=gen, device=dev).to(torch.float8_e4m3fn)
    kf = torch.randn((1, L, 128), generator=gen, device=dev)
    ks = (kf.abs().amax(dim=-1).clamp_min(2.0 ** -126) / 448.0).float()
    ki = (kf / ks[..., None]).to(torch.float8_e4m3fn)
    del kf
    w = (torch.randn((L, 64), generator=gen, device=dev) / 8).to(torch.bfloat16)
    qm = torch.empty((L, H, 576), dtype=torch.bfloat16, device=dev)
    for r0 in range(0, L, 4096):
        qm[r0:r0 + 4096] = torch.randn((4096, H, 576), generator=gen, device=dev).to(torch.bfloat16)
    kv = torch.randn((1, L, 576), generator=gen, device=dev).to(torch.bfloat16)
    seq = torch.tensor([L], dtype=torch.int32, device=dev)
    geom = lcl.make_geom(1, L, L, seq)
    idx = torch.empty((L, k), dtype=torch.int32, device=dev)
    out = torch.empty((L, H, 512), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(lcl.forward_workspace_size(1, L, L, H, k, lcl.FP8_E4M3FN, lcl.BF16), dtype=torch.uint8,
                     device=dev)
    mla_ws = torch.empty(256, dtype=torch.uint8, device=dev)
    sel = torch.empty_like(idx)
    sel_ws = torch.empty(max(lcl.indexer_topk_workspace_size(1, L, L, k, lcl.FP8_E4M3FN), 256), dtype=torch.uint8,
                         device=dev)
    sm = 1.0 / math.sqrt(192.0)
    fwd_ms, mla_ms, sel_ms = [], [], []
    n = args.prefill_steps
    for i in range(1 + n):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        evict()
        e[0].record(stream)
        lcl.forward(geom, k, sm, qi, w, ki, qm, kv, index_k_scale=ks, idx=idx, out=out, ws=ws, want_lse=False)
        e[1].record(stream)
        lcl.sparse_mla(geom, qm, kv, idx, sm, out=out, ws=mla_ws, want_lse=False)
        e[2].record(stream)
        evict()
        e[3].record(stream)
        lcl.indexer_topk(geom, k, qi, w, ki, index_k_scale=ks, idx=sel, ws=sel_ws)
        e[4].record(stream)
        torch.cuda.synchronize()
        if i >= 1:
            fwd_ms.append(e[0].elapsed_time(e[1]))
            mla_ms.append(e[1].elapsed_time(e[2]))
            sel_ms.append(e[3].elapsed_time(e[4]))
        log(f"prefill step {i}: forward {e[0].elapsed_time(e[1]):.2f} ms, indexer + top-k alone "
            f"{e[3].elapsed_time(e[4]):.2f} ms, sparse MLA alone {e[1].elapsed_time(e[2]):.2f} ms")
    del sel, sel_ws
    f_ms = sum(fwd_ms) / len(fwd_ms)
    s_ms = sum(mla_ms) / len(mla_ms)   # the standalone attention call (reads every idx entry)
    # indexer + top-k timed as its own call (dsa_indexer_topk, the same launches
    # as inside the forward); the forward's attention is the rest
    i_ms = sum(sel_ms) / len(sel_ms)
    m_ms = max(f_ms - i_ms, 1e-6)
    # the same prefill on 64-token pages (scattered seeded table): it streams too
    from synth import make_block_table
    P = 64
    table, clean, num_pages = make_block_table(10, 1, np.array([L]), L, P)
    dst = torch.from_numpy(clean.reshape(-1).astype(np.int64)).to(dev)

    def pool(c, tail):
        return torch.zeros((num_pages, P) + tail, dtype=c.dtype, device=dev).index_copy_(0, dst, c.reshape((-1, P) + tail))

    ki_p, ks_p, kv_p = pool(ki.view(torch.uint8), (128,)), pool(ks, ()), pool(kv, (576,))
    pages = lcl.make_pages(torch.from_numpy(table).to(dev), P, num_pages)
    pws = torch.empty(lcl.forward_paged_workspace_size(1, L, L, H, k, lcl.FP8_E4M3FN, lcl.BF16), dtype=torch.uint8,
                      device=dev)
    paged_ms = []
    for i in range(2):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        evict()
        e[0].record(stream)
        lcl.forward(geom, k, sm, qi, w, ki_p, qm, kv_p, index_k_scale=ks_p, idx=idx, out=out, ws=pws, want_lse=False,
                    pages=pages)
        e[1].record(stream)
        torch.cuda.synchronize()
        if i >= 1:
            paged_ms.append(e[0].elapsed_time(e[1]))
    p_ms = sum(paged_ms) / len(paged_ms)
    log(f"prefill on 64-token pages: {p_ms:.2f} ms ({p_ms / f_ms:.3f}x the contiguous forward)")
    del ki_p, ks_p, kv_p, pws
    pairs = L * (L + 1) // 2
    idx_tflops = pairs * 64 * 128 * 2 / (i_ms * 1e-3) / 1e12
    sel_rows = sum(min(t + 1, k) for t in range(L))
    mla_tflops = sel_rows * H * (576 + 512) * 2 / (m_ms * 1e-3) / 1e12
    log(f"prefill: {L / (f_ms * 1e-3):,.0f} tokens/s; indexer+top-k {i_ms:.2f} ms = {idx_tflops:.0f} TFLOP/s "
        f"({idx_tflops / FP8_PEAK_TFLOPS:.1%} fp8 peak); sparse MLA {m_ms:.2f} ms = {mla_tflops:.0f} TFLOP/s "
        f"({mla_tflops / BF16_PEAK_TFLOPS:.1%} bf16 peak; the standalone call, which reads every idx entry, "
        f"{s_ms:.2f} ms)")
    res = {"workload": "prefill64k: 1 x 65536 causal, indexer fp8 64x128, top-k 2048, 128-head MQA-MLA bf16",
           "tokens_per_s": round(L / (f_ms * 1e-3), 1), "ms_per_step": round(f_ms, 3), "steps": n,
           "indexer_topk_ms": round(i_ms, 3), "indexer_tflops": round(idx_tflops, 1),
           "indexer_fp8_mfma_frac": round(idx_tflops / FP8_PEAK_TFLOPS, 4),
           "sparse_mla_ms": round(m_ms, 3), "sparse_mla_tflops": round(mla_tflops, 1),
           "sparse_mla_bf16_mfma_frac": round(mla_tflops / BF16_PEAK_TFLOPS, 4),
           "sparse_mla_standalone_ms": round(s_ms, 3),
           "paged_64_token_pages": {"ms_per_step": round(p_ms, 3), "tokens_per_s": round(L / (p_ms * 1e-3), 1),
                                    "vs_contiguous": round(p_ms / f_ms, 4)},
           "workspace_bytes": lcl.forward_workspace_size(1, L, L, H, k, lcl.FP8_E4M3FN, lcl.BF16),
           "data": "synthetic, drawn on the GPU with torch's seeded generator (same recipe)"}
    del qi, ki, ks, w, qm, kv, idx, out, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(wl, qi, w, ki, ks, qm, np, budget_s):
    """The float64 oracle on a bounded sample of the decode workload: whole
    sequences (both queries, all three stages), one after another, until
    budget_s seconds of oracle time have passed (at least one sequence)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    log(f"cpu baseline: oracle on whole decode sequences for ~{budget_s:.0f}s, {cores} cores")
    spent, nseq = 0.0, 0
    while nseq < wl.B and (nseq == 0 or spent < budget_s):
        b = nseq
        rows = np.arange(b * wl.q_len, (b + 1) * wl.q_len)
        kv = wl.kv(b)[None]
        t0 = time.perf_counter()
        oracle.dsa_forward(qi[rows], "e4m3fn", w[rows], "bf16", ki[b:b + 1], "e4m3fn", qm[rows], "bf16", kv,
                           "bf16", wl.seq_lens[b:b + 1], wl.q_len, wl.topk, wl.sm_scale, k_scale=ks[b:b + 1])
        spent += time.perf_counter() - t0
        nseq += 1
    nq = nseq * wl.q_len
    log(f"cpu baseline: {spent:.1f}s for {nq} queries")
    return {"value": round(nq / spent, 4), "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": f"{nq} queries ({nseq} of the {wl.B} sequences x {wl.q_len}) of the 128K decode workload, "
                      f"all three stages in float64 NumPy, {spent:.1f}s"}


def _oracle_rows(oracle, np, wl, rows, qi, w, ki, ks, qm, kv):
    """The oracle's three stages for the given query rows (time in seconds)."""
    t0 = time.perf_counter()
    oracle.dsa_forward(qi, "e4m3fn", w, "bf16", ki, "e4m3fn", qm, "bf16", kv, "bf16", wl.seq_lens, wl.q_len, wl.topk,
                       wl.sm_scale, k_scale=ks, rows=rows)
    return time.perf_counter() - t0


def cpu_baseline_configs(np, budget_s):
    """The float64 oracle on the other fp8 configurations, each on a bounded
    sample, on the host cores:
      decode32k   whole sequences (one query each) until about budget_s / 3
                  seconds have passed, queries/s;
      prefill8k   the 32 planted rows plus 32 seeded uniformly random rows
                  (a fixed sample of about a second): rows/s on the sample,
                  and the full 8192-row run extrapolated from the random rows
                  (mean time per row x L);
      prefill64k  12 seeded uniformly random rows, same report.
    Inputs follow the same recipe (synth); only the sampled rows' queries
    are drawn."""
    import oracle
    from synth import standard_workload
    cores = len(os.sched_getaffinity(0))
    res = {}
    wl = standard_workload("decode32k")
    log(f"cpu baseline (configs): {wl.name}")
    spent, n = 0.0, 0
    while n < wl.B and (n == 0 or spent < budget_s / 3):
        rows = np.array([n])
        ki, ks = wl.ki(n)
        # sequence n as a B = 1 geometry of the same recipe
        sub = type(wl)(name=wl.name, B=1, q_len=1, S_max=wl.S_max, seq_lens=wl.seq_lens[n:n + 1], topk=wl.topk,
                       H=wl.H, seed=wl.seed)
        spent += _oracle_rows(oracle, np, sub, np.array([0]), wl.qi(rows), wl.w(rows), ki[None], ks[None], wl.qm(rows),
                              wl.kv(n)[None])
        n += 1
    res["decode32k"] = {"value": round(n / spent, 4), "unit": "queries/s", "cores": cores, "kind": "oracle",
                        "sample": f"{n} of the 64 sequences (1 query each), all three stages, {spent:.1f}s"}
    for name, n_rand in (("prefill8k", 32), ("prefill64k", 12)):
        wl = standard_workload(name)
        log(f"cpu baseline (configs): {wl.name}")
        L = wl.T
        rng = np.random.default_rng(17)
        rand = np.sort(rng.choice(L, n_rand, replace=False))
        planted = wl.planted_rows if wl.planted_rows is not None else np.array([], np.int64)
        sample = np.unique(np.concatenate([planted, rand]))
        qi = np.zeros((L, 64, 128), np.uint8)
        qi[sample] = wl.qi(sample)
        w = wl.w()
        qm = np.zeros((L, wl.H, 576), np.uint16)
        qm[sample] = wl.qm(sample)
        ki, ks = wl.ki_all()
        kv = wl.kv_all()
        t_rand = 0.0
        for t in rand:
            t_rand += _oracle_rows(oracle, np, wl, np.array([t]), qi, w, ki, ks, qm, kv)
        t_all = t_rand
        others = np.setdiff1d(sample, rand)
        if len(others):
            t_all += _oracle_rows(oracle, np, wl, others, qi, w, ki, ks, qm, kv)
        extrap = t_rand / len(rand) * L
        res[name] = {"value": round(len(sample) / t_all, 4), "unit": "tokens/s (sampled rows)", "cores": cores,
                     "kind": "oracle",
                     "sample": f"{len(sample)} query rows ({len(planted)} planted, {len(rand)} seeded uniform random) "
                               f"of the {L}-token prefill, all three stages, {t_all:.1f}s",
                     "extrapolated_full_run_s": round(extrap, 1),
                     "extrapolated_note": "mean oracle time of the uniform random rows x L (an estimate, not a run)"}
        del qi, qm, kv
    return res


if __name__ == "__main__":
    main()
