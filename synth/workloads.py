"""Seeded synthetic workloads with the shapes and structure of the five DSA
forward configurations (tiny prefill, 32K decode, 8K planted prefill, 64K
prefill, 128K tied decode), plus smaller variants of the same recipe.

Every tensor is drawn lazily and reproducibly: a tensor is split into blocks
(rows of queries, or 4096-position chunks of one sequence's cache) and each
block has its own PCG64 stream keyed by ``(seed, tensor, block...)``.  Any
subset of rows can therefore be regenerated bit-exactly without drawing the
rest, which lets a test or a CPU baseline look at a few rows of a 64K-token
prefill without materialising all of it.

Recipe (values are generated in float32 / float64 on the host, then encoded):

* fp8 configs: indexer q = e4m3fn(N(0,1)) with no scale; indexer k =
  per-token quantised N(0,1) (e4m3fn codes + fp32 scale amax/448); head
  weights w = bf16(N(0,1)/8); MLA q and latent cache = bf16(N(0,1)); for
  MHA mode, q = bf16(N(0,1)) [T, H, 192] and wkv_b = bf16(N(0,1)/sqrt(512));
  for the KL objective, indexer scores I ~ N(0, 4) float32 [T, S_max].
* fp32 config ("tiny"): indexer q, k ~ N(0,1)/sqrt(128), w ~ N(0,1), MLA q
  and latent cache ~ N(0,1), all float32, no scales.
* ``plant``: one template (q*, w*) is drawn; the planted query rows get
  ``q* + 0.1 N(0,1)`` and ``w*``; one set P of positions gets keys
  ``u * sqrt(128)/|u| + 0.1 N(0,1)`` with ``u = sum_j w*_j q*_j`` (the
  w-weighted mean of the template's head queries), so P is the top-k set of
  every planted row.
* ``pool``: keys are drawn from a pool of 256 quantised rows, each position
  taking a uniformly random pool row, so equal scores occur exactly.
"""

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .encode import encode_bf16_rne, encode_e4m3fn_rne, quantize_per_token

HI, DI, DQK, DV = 64, 128, 576, 512
ROW_BLOCK = 64
POS_BLOCK = 4096

_STREAM = {"qi": 1, "w": 2, "ki": 3, "qm": 4, "kv": 5, "plant": 6, "pool": 7, "qh": 8, "wkvb": 9, "kls": 10}
D_QH, D_NOPE_V = 192, 256   # MHA mode: q = [nope 128 | rope 64]; wkv_b rows per head = [k_nope 128 | v 128]


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _normal32(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _pmap(fn, items, threads=8):
    items = list(items)
    if len(items) <= 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(max_workers=min(threads, len(items))) as ex:
        return list(ex.map(fn, items))


@dataclass
class Workload:
    name: str
    B: int
    q_len: int
    S_max: int
    seq_lens: np.ndarray
    topk: int
    H: int
    fp8: bool = True
    seed: int = 0
    sm_scale: float = 1.0 / math.sqrt(192.0)
    ki_mode: str = "normal"          # "normal" | "pool"
    plant: dict = field(default=None)  # {"n_rows", "row_lo", "row_hi", "set_size", "set_hi"}

    def __post_init__(self):
        self.seq_lens = np.asarray(self.seq_lens, dtype=np.int32)
        if self.seq_lens.shape != (self.B,):
            raise ValueError("seq_lens must have B entries")
        if np.any(self.seq_lens < self.q_len) or np.any(self.seq_lens > self.S_max):
            raise ValueError("need q_len <= seq_lens[b] <= S_max")
        self._plant_cache = None
        self._pool_cache = None

    # ---- geometry -----------------------------------------------------
    @property
    def T(self):
        return self.B * self.q_len

    @property
    def qi_fmt(self):
        return "e4m3fn" if self.fp8 else "f32"

    ki_fmt = qi_fmt

    @property
    def w_fmt(self):
        return "bf16" if self.fp8 else "f32"

    qm_fmt = w_fmt
    kv_fmt = w_fmt

    def positions(self):
        """Position of each query row (last q_len positions of its sequence)."""
        b = np.repeat(np.arange(self.B), self.q_len)
        i = np.tile(np.arange(self.q_len), self.B)
        return self.seq_lens[b].astype(np.int64) - self.q_len + i

    # ---- planted structure ---------------------------------------------
    def _planted(self):
        if self.plant is None:
            return None
        if self._plant_cache is None:
            p = self.plant
            g = _rng(self.seed, _STREAM["plant"])
            qstar = g.standard_normal((HI, DI))
            wstar = encode_bf16_rne((g.standard_normal(HI) / 8.0).astype(np.float32))
            rows = np.sort(g.choice(np.arange(p["row_lo"], p["row_hi"]), p["n_rows"], replace=False))
            pset = np.sort(g.choice(p["set_hi"], p["set_size"], replace=False))
            qnoise = g.standard_normal((p["n_rows"], HI, DI)) * 0.1
            knoise = g.standard_normal((p["set_size"], DI)) * 0.1
            wdec = (wstar.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            u = (wdec[:, None] * qstar).sum(axis=0)
            u = u * (math.sqrt(DI) / np.linalg.norm(u))
            kcodes, kscale = quantize_per_token(u[None, :] + knoise)
            qcodes = encode_e4m3fn_rne(qstar[None] + qnoise)
            self._plant_cache = dict(rows=rows, set=pset, w=wstar, q=qcodes,
                                     k=kcodes, k_scale=kscale)
        return self._plant_cache

    @property
    def planted_rows(self):
        p = self._planted()
        return None if p is None else p["rows"]

    @property
    def planted_set(self):
        p = self._planted()
        return None if p is None else p["set"]

    def _pool(self):
        if self._pool_cache is None:
            g = _rng(self.seed, _STREAM["pool"])
            codes, scale = quantize_per_token(g.standard_normal((256, DI)))
            self._pool_cache = (codes, scale)
        return self._pool_cache

    # ---- row-blocked query-side tensors -------------------------------
    def _rows(self, rows):
        return np.arange(self.T) if rows is None else np.asarray(rows, dtype=np.int64)

    def _by_blocks(self, rows, stream, make_block, shape_tail, dtype):
        rows = self._rows(rows)
        out = np.empty((len(rows),) + shape_tail, dtype=dtype)
        blocks = np.unique(rows // ROW_BLOCK)

        def one(blk):
            n = min(ROW_BLOCK, self.T - blk * ROW_BLOCK)
            data = make_block(_rng(self.seed, _STREAM[stream], int(blk)), n)
            sel = np.nonzero(rows // ROW_BLOCK == blk)[0]
            out[sel] = data[rows[sel] - blk * ROW_BLOCK]

        _pmap(one, blocks)
        return out

    def qi(self, rows=None):
        """Indexer queries [R, 64, 128]: e4m3fn codes (fp8) or float32."""
        if self.fp8:
            mk = lambda g, n: encode_e4m3fn_rne(_normal32(g, (n, HI, DI)))
            out = self._by_blocks(rows, "qi", mk, (HI, DI), np.uint8)
        else:
            mk = lambda g, n: _normal32(g, (n, HI, DI)) / np.float32(math.sqrt(DI))
            out = self._by_blocks(rows, "qi", mk, (HI, DI), np.float32)
        return self._apply_plant(rows, out, "q")

    def w(self, rows=None):
        """Per-query head weights [R, 64]: bf16 bits (fp8 configs) or float32."""
        if self.fp8:
            mk = lambda g, n: encode_bf16_rne(_normal32(g, (n, HI)) / np.float32(8.0))
            out = self._by_blocks(rows, "w", mk, (HI,), np.uint16)
        else:
            mk = lambda g, n: _normal32(g, (n, HI))
            out = self._by_blocks(rows, "w", mk, (HI,), np.float32)
        return self._apply_plant(rows, out, "w")

    def qm(self, rows=None):
        """MLA queries [R, H, 576]: bf16 bits or float32."""
        if self.fp8:
            mk = lambda g, n: encode_bf16_rne(_normal32(g, (n, self.H, DQK)))
            return self._by_blocks(rows, "qm", mk, (self.H, DQK), np.uint16)
        mk = lambda g, n: _normal32(g, (n, self.H, DQK))
        return self._by_blocks(rows, "qm", mk, (self.H, DQK), np.float32)

    def qh(self, rows=None):
        """MHA-mode queries [R, H, 192] (nope | rope): bf16 bits or float32."""
        if self.fp8:
            mk = lambda g, n: encode_bf16_rne(_normal32(g, (n, self.H, D_QH)))
            return self._by_blocks(rows, "qh", mk, (self.H, D_QH), np.uint16)
        mk = lambda g, n: _normal32(g, (n, self.H, D_QH))
        return self._by_blocks(rows, "qh", mk, (self.H, D_QH), np.float32)

    def wkv_b(self):
        """Latent up-projection [H, 256, 512] (per head: k_nope rows, then v
        rows), N(0, 1/512) so decompressed keys and values are ~N(0, 1):
        bf16 bits or float32."""
        g = _rng(self.seed, _STREAM["wkvb"])
        w = _normal32(g, (self.H, D_NOPE_V, DQK - 64)) / np.float32(math.sqrt(DQK - 64))
        return encode_bf16_rne(w) if self.fp8 else w

    def kl_scores(self, rows=None):
        """Indexer scores standing in for I in the KL objective: [R, S_max]
        float32 ~ N(0, 4) (the objective reads only visible positions)."""
        mk = lambda g, n: _normal32(g, (n, self.S_max)) * np.float32(2.0)
        return self._by_blocks(rows, "kls", mk, (self.S_max,), np.float32)

    def _apply_plant(self, rows, out, what):
        p = self._planted()
        if p is None:
            return out
        rows = self._rows(rows)
        for r, t in enumerate(rows):
            hit = np.nonzero(p["rows"] == t)[0]
            if len(hit):
                out[r] = p["q"][hit[0]] if what == "q" else p["w"]
        return out

    # ---- per-sequence cache tensors -------------------------------------
    def _cache(self, b, stream, make_chunk, width, dtype):
        out = np.empty((self.S_max, width), dtype=dtype)

        def one(c):
            lo = c * POS_BLOCK
            n = min(POS_BLOCK, self.S_max - lo)
            out[lo:lo + n] = make_chunk(_rng(self.seed, _STREAM[stream], int(b), int(c)), n)

        _pmap(one, range((self.S_max + POS_BLOCK - 1) // POS_BLOCK))
        return out

    def ki(self, b):
        """Indexer key cache of sequence b: ([S_max, 128] codes or float32,
        [S_max] fp32 scale or None)."""
        if not self.fp8:
            mk = lambda g, n: _normal32(g, (n, DI)) / np.float32(math.sqrt(DI))
            return self._cache(b, "ki", mk, DI, np.float32), None
        if self.ki_mode == "pool":
            codes, scale = self._pool()
            assign = _rng(self.seed, _STREAM["ki"], int(b)).integers(0, 256, self.S_max)
            return codes[assign], scale[assign]
        scales = np.empty(self.S_max, dtype=np.float32)

        def mk(g, n):
            c, s = quantize_per_token(_normal32(g, (n, DI)))
            return np.concatenate([c, s.view(np.uint8).reshape(n, 4)], axis=1)

        packed = self._cache(b, "ki", mk, DI + 4, np.uint8)
        codes = np.ascontiguousarray(packed[:, :DI])
        scales[:] = np.ascontiguousarray(packed[:, DI:]).view(np.float32)[:, 0]
        p = self._planted()
        if p is not None and b == 0:
            codes[p["set"]] = p["k"]
            scales[p["set"]] = p["k_scale"]
        return codes, scales

    def kv(self, b):
        """Latent cache of sequence b [S_max, 576]: bf16 bits or float32."""
        if self.fp8:
            mk = lambda g, n: encode_bf16_rne(_normal32(g, (n, DQK)))
            return self._cache(b, "kv", mk, DQK, np.uint16)
        mk = lambda g, n: _normal32(g, (n, DQK))
        return self._cache(b, "kv", mk, DQK, np.float32)

    def ki_all(self):
        parts = [self.ki(b) for b in range(self.B)]
        codes = np.stack([p[0] for p in parts])
        scales = None if parts[0][1] is None else np.stack([p[1] for p in parts])
        return codes, scales

    def kv_all(self):
        return np.stack([self.kv(b) for b in range(self.B)])


def make_workload(name, B, q_len, seq_lens, S_max, topk, H, fp8=True, seed=0,
                  ki_mode="normal", plant=None):
    return Workload(name=name, B=B, q_len=q_len, S_max=S_max,
                    seq_lens=np.broadcast_to(np.asarray(seq_lens), (B,)).copy(),
                    topk=topk, H=H, fp8=fp8, seed=seed, ki_mode=ki_mode,
                    plant=plant)


WORKLOAD_NAMES = ("tiny512", "decode32k", "prefill8k", "prefill64k", "decode128k")


def standard_workload(name):
    """The five configurations at their full sizes."""
    if name == "tiny512":
        return make_workload(name, 1, 512, 512, 512, 64, 16, fp8=False, seed=0)
    if name == "decode32k":
        return make_workload(name, 64, 1, 32768, 32768, 2048, 128, seed=1)
    if name == "prefill8k":
        return make_workload(name, 1, 8192, 8192, 8192, 2048, 128, seed=2,
                             plant=dict(n_rows=32, row_lo=4096, row_hi=8192,
                                        set_size=2048, set_hi=4096))
    if name == "prefill64k":
        return make_workload(name, 1, 65536, 65536, 65536, 2048, 128, seed=3)
    if name == "decode128k":
        return make_workload(name, 16, 2, 131072, 131072, 2048, 128, seed=4,
                             ki_mode="pool")
    raise KeyError(name)
