"""GPU parity of the per-block fp8 quantisation and the indexer key-cache
append (dsa_indexer_quantize / dsa_indexer_cache_append, through the C ABI)
against the oracle's ``quantize_blocks`` / ``cache_append``: codes and scales
must be bit-exact (both sides divide in fp32 and round the quotient to the
nearest e4m3fn value)."""

import numpy as np
import pytest
import torch

from oracle import cache_append, quantize_blocks
from oracle.formats import decode_e4m3fn
from synth.encode import encode_bf16_rne

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _rows(rng, n, bf16):
    """Rows of 128 with magnitudes from 2^-30 to 2^30, zero rows, and rows whose
    quotients land exactly on e4m3fn midpoints (scale a power of two)."""
    x = rng.standard_normal((n, 128)) * 2.0 ** rng.integers(-30, 30, (n, 1))
    x[::97] = 0.0
    pos = decode_e4m3fn(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2.0
    for r in range(5, n, 61):
        s = 2.0 ** int(rng.integers(-8, 8))
        row = rng.choice(mids, 128) * rng.choice([-1.0, 1.0], 128)
        row[int(rng.integers(0, 128))] = 448.0           # amax: scale = s exactly
        x[r] = row * s
    x = x.astype(np.float32)
    if bf16:
        bits = encode_bf16_rne(x)
        return bits, (bits.astype(np.uint32) << 16).view(np.float32)
    return x, x


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
def test_quantize_bit_exact(dsa_gpu, bf16):
    lcl = dsa_gpu
    rng = np.random.default_rng(11 if bf16 else 12)
    for n in (1, 7, 1000, 20001):                           # ragged against 8 blocks per workgroup
        _say(f"[quant] dsa_indexer_quantize bf16={bf16} rows={n}")
        host, x32 = _rows(rng, n, bf16)
        codes, scales = lcl.indexer_quantize(_dev(host))
        torch.cuda.synchronize()
        want_c, want_s = quantize_blocks(x32)
        assert np.array_equal(codes.cpu().numpy(), want_c), f"codes differ (rows={n})"
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), want_s.view(np.uint32)), f"scales (rows={n})"


def test_quantize_full_prefill_q_sampled(dsa_gpu):
    """The 64K prefill's indexer queries, [65536 * 64, 128] bf16 (the shape the
    bench times), checked on sampled rows."""
    lcl = dsa_gpu
    _say("[quant] dsa_indexer_quantize on [65536*64, 128] bf16, sampled rows")
    g = torch.Generator(device="cuda")
    g.manual_seed(21)
    x = torch.randn((65536 * 64, 128), generator=g, device="cuda").to(torch.bfloat16)
    codes, scales = lcl.indexer_quantize(x)
    torch.cuda.synchronize()
    rows = np.concatenate([[0, 1, 63, 64, 65536 * 64 - 1],
                           np.random.default_rng(3).integers(0, 65536 * 64, 2048)])
    rt = torch.from_numpy(rows).cuda()
    xs = x[rt].view(torch.int16).cpu().numpy().view(np.uint16)
    want_c, want_s = quantize_blocks((xs.astype(np.uint32) << 16).view(np.float32))
    assert np.array_equal(codes[rt].cpu().numpy(), want_c)
    assert np.array_equal(scales[rt].cpu().numpy().view(np.uint32), want_s.view(np.uint32))


@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
def test_cache_append_bit_exact_and_in_place(dsa_gpu, bf16):
    lcl = dsa_gpu
    rng = np.random.default_rng(31)
    B, q_len, S_max = 5, 3, 300
    seq_lens = np.array([300, 10, 2, 150, 3], dtype=np.int32)   # full, short, shorter than q_len, ...
    _say(f"[quant] dsa_indexer_cache_append bf16={bf16} B={B} q_len={q_len} S_max={S_max}")
    host, x32 = _rows(rng, B * q_len, bf16)
    cache0 = np.full((B, S_max, 128), 0x55, np.uint8)
    scale0 = np.full((B, S_max), -7.0, np.float32)
    d_cache, d_scale = _dev(cache0), _dev(scale0)
    d_seq = torch.from_numpy(seq_lens).cuda()
    geom = lcl.make_geom(B, q_len, S_max, d_seq)
    lcl.indexer_cache_append(geom, _dev(host).view(B, q_len, 128), d_cache, d_scale)
    torch.cuda.synchronize()
    want_c, want_s = cache_append(cache0, scale0, x32.reshape(B, q_len, 128), seq_lens, q_len)
    assert np.array_equal(d_cache.cpu().numpy(), want_c)
    assert np.array_equal(d_scale.cpu().numpy().view(np.uint32), want_s.view(np.uint32))


def test_quantized_inputs_drive_the_indexer(dsa_gpu):
    """q quantised by dsa_indexer_quantize and k appended by
    dsa_indexer_cache_append give the same scores as the oracle's indexer on
    the oracle's own quantisation (identical fp8 inputs)."""
    from oracle import indexer_scores
    from tests.gpu_util import check_scores
    lcl = dsa_gpu
    rng = np.random.default_rng(41)
    B, q_len, S_max = 2, 2, 1024
    seq_lens = np.array([1024, 777], dtype=np.int32)
    _say("[quant] quantise q, append k step by step, then dsa_indexer_scores")
    q = rng.standard_normal((B * q_len, 64, 128)).astype(np.float32)
    keys = rng.standard_normal((B, S_max, 128)).astype(np.float32)
    w = encode_bf16_rne((rng.standard_normal((B * q_len, 64)) / 8).astype(np.float32))
    d_seq = torch.from_numpy(seq_lens).cuda()
    cache = torch.zeros((B, S_max, 128), dtype=torch.uint8, device="cuda")
    kscale = torch.zeros((B, S_max), dtype=torch.float32, device="cuda")
    # fill the cache q_len keys at a time, as decode steps would
    for L in range(q_len, S_max + 1, q_len):
        lens = np.minimum(seq_lens, L).astype(np.int32)
        lens = np.maximum(lens, q_len)
        d_lens = torch.from_numpy(lens).cuda()            # kept alive until the append is enqueued
        geom = lcl.make_geom(B, q_len, S_max, d_lens)
        new = np.stack([keys[b, lens[b] - q_len:lens[b]] for b in range(B)])
        lcl.indexer_cache_append(geom, _dev(new), cache, kscale)
    qc, qs = lcl.indexer_quantize(_dev(q))
    geom = lcl.make_geom(B, q_len, S_max, d_seq)
    scores = lcl.indexer_scores(geom, qc, _dev(w), cache, k_scale=kscale, q_scale=qs)
    torch.cuda.synchronize()
    oqc, oqs = quantize_blocks(q)
    okc, oks = quantize_blocks(keys)
    for b in range(B):                                      # positions past seq_lens were never written
        okc[b, seq_lens[b]:] = 0
        oks[b, seq_lens[b]:] = 0
    assert np.array_equal(cache.cpu().numpy(), okc)
    want = indexer_scores(oqc, "e4m3fn", w, "bf16", okc, "e4m3fn", seq_lens, q_len, k_scale=oks, q_scale=oqs)
    from oracle import query_positions
    _, pos = query_positions(seq_lens, q_len)
    check_scores(scores.cpu().numpy().astype(np.float64), want, pos)
