"""Python binding of libdsa, the MI355X (gfx950) DSA forward path.

Argument marshalling only: every stage runs in the HIP kernels of libdsa.so
(built in-tree by ``long_context_lightning_amd.build``).  torch tensors supply
device memory and the current stream.  Functions mirror the C ABI in
include/dsa.h and raise ``DsaError`` on any non-OK status.  There is no
fallback: if the library is missing or fails to load, ``load()`` raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

F32, BF16, FP8_E4M3FN = 0, 1, 2
_STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE",
           4: "DSA_ERR_HIP"}

_lib = None


class DsaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)}")


class Geom(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("q_len", ctypes.c_int32), ("S_max", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p)]


class Pages(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int64)]


def load(path=None):
    """Load libdsa.so (once).  Raises if it is missing or incomplete."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m long_context_lightning_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    gp = ctypes.POINTER(Geom)
    pp = ctypes.POINTER(Pages)
    sig = {
        "dsa_indexer_scores": (i32, [gp, vp, i32, vp, vp, i32, vp, i32, vp, i32, i32, vp, i64, vp]),
        "dsa_topk": (i32, [gp, vp, i64, i32, i32, i32, vp, vp, sz, vp]),
        "dsa_topk_workspace_size": (sz, [i32, i32, i32]),
        "dsa_sparse_mla": (i32, [gp, i32, i32, f32, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
        "dsa_sparse_mla_workspace_size": (sz, [i32, i32, i32, i32, i32]),
        "dsa_forward": (i32, [gp, i32, i32, f32, vp, i32, vp, vp, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz,
                              vp]),
        "dsa_forward_workspace_size": (sz, [i32, i32, i32, i32, i32, i32, i32]),
        "dsa_indexer_topk": (i32, [gp, i32, vp, i32, vp, vp, i32, vp, vp, vp, vp, sz, vp]),
        "dsa_indexer_topk_workspace_size": (sz, [i32, i32, i32, i32, i32]),
        "dsa_indexer_quantize": (i32, [vp, i32, i64, vp, vp, vp]),
        "dsa_indexer_cache_append": (i32, [gp, vp, i32, vp, vp, vp]),
        "dsa_indexer_scores_paged": (i32, [gp, pp, vp, i32, vp, vp, i32, vp, i32, vp, i32, i32, vp, i64, vp]),
        "dsa_sparse_mla_paged": (i32, [gp, pp, i32, i32, f32, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
        "dsa_sparse_mla_paged_workspace_size": (sz, [i32, i32, i32, i32, i32]),
        "dsa_forward_paged": (i32, [gp, pp, i32, i32, f32, vp, i32, vp, vp, i32, vp, vp, vp, vp, i32, vp, vp, vp,
                                    vp, sz, vp]),
        "dsa_forward_paged_workspace_size": (sz, [i32, i32, i32, i32, i32, i32, i32]),
        "dsa_indexer_cache_append_paged": (i32, [gp, pp, vp, i32, vp, vp, vp]),
        "dsa_mha_prefill": (i32, [gp, i32, f32, vp, vp, vp, i32, vp, vp, vp, sz, vp]),
        "dsa_mha_prefill_workspace_size": (sz, [i32, i32, i32]),
        "dsa_indexer_kl": (i32, [gp, i32, f32, vp, vp, i32, vp, vp, i64, vp, i32, vp, vp, vp, sz, vp]),
        "dsa_indexer_kl_workspace_size": (sz, [i32, i32, i32, i32]),
        "dsa_workspace_size": (sz, [i32, i32, i32, i32, i32, ctypes.c_int]),
        "dsa_forward_noalloc": (i32, [gp, i32, i32, f32, vp, i32, vp, vp, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp]),
        "dsa_status_string": (ctypes.c_char_p, [i32]),
        "dsa_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)  # AttributeError if the symbol is not exported
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


ABI_FUNCTIONS = ("dsa_indexer_scores", "dsa_topk", "dsa_topk_workspace_size", "dsa_sparse_mla",
                 "dsa_sparse_mla_workspace_size", "dsa_forward", "dsa_forward_workspace_size",
                 "dsa_indexer_topk", "dsa_indexer_topk_workspace_size",
                 "dsa_indexer_quantize", "dsa_indexer_cache_append", "dsa_indexer_scores_paged",
                 "dsa_sparse_mla_paged", "dsa_sparse_mla_paged_workspace_size", "dsa_forward_paged",
                 "dsa_forward_paged_workspace_size", "dsa_indexer_cache_append_paged", "dsa_mha_prefill",
                 "dsa_mha_prefill_workspace_size", "dsa_indexer_kl", "dsa_indexer_kl_workspace_size",
                 "dsa_workspace_size", "dsa_forward_noalloc", "dsa_status_string", "dsa_version")

NOALLOC_SCRATCH_BYTES = 96 << 20   # DSA_NOALLOC_SCRATCH_BYTES

# which_call values of dsa_workspace_size
CALL_TOPK, CALL_SPARSE_MLA, CALL_FORWARD, CALL_SPARSE_MLA_PAGED, CALL_FORWARD_PAGED, CALL_MHA_PREFILL, \
    CALL_INDEXER_KL, CALL_INDEXER_TOPK = range(8)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, where):
    if status != 0:
        raise DsaError(status, where)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dev(t, name, dtypes):
    _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous device tensor")
    _need(t.dtype in dtypes, f"{name} has dtype {t.dtype}, expected one of {dtypes}")


_FP8 = torch.float8_e4m3fn


def _index_dtype(t):
    # fp8 tensors may come as float8_e4m3fn or as their uint8 codes
    if t.dtype in (_FP8, torch.uint8):
        return FP8_E4M3FN
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"indexer tensor dtype {t.dtype} unsupported")


def _w_dtype(t):
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"weight dtype {t.dtype} unsupported")


def _mla_dtype(t):
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"MLA tensor dtype {t.dtype} unsupported")


def make_geom(B, q_len, S_max, seq_lens):
    """Geometry struct; ``seq_lens`` is an int32 device tensor of length B (kept alive by the caller)."""
    _dev(seq_lens, "seq_lens", (torch.int32,))
    _need(seq_lens.numel() == B, "seq_lens must have B entries")
    return Geom(B, q_len, S_max, seq_lens.data_ptr())


def make_pages(block_table, page_size, num_pages):
    """Page-table struct; ``block_table`` is an int32 device tensor [B, max_pages] (kept alive by the caller)."""
    _dev(block_table, "block_table", (torch.int32,))
    _need(block_table.dim() == 2, "block_table must be [B, max_pages]")
    return Pages(block_table.data_ptr(), block_table.shape[1], page_size, num_pages)


def _cache_shape(geom, pages, tail):
    """Expected shape of a cache: [B, S_max, *tail], or the pool [num_pages, page_size, *tail]."""
    if pages is None:
        return (geom.B, geom.S_max) + tail
    return (pages.num_pages, pages.page_size) + tail


def indexer_scores(geom, q, w, k, k_scale=None, q_scale=None, row_begin=0, row_count=None, scores=None,
                   stream=None, pages=None):
    """dsa_indexer_scores (dsa_indexer_scores_paged when ``pages`` is given,
    with ``k`` / ``k_scale`` the page pools): returns fp32 scores [row_count, S_max]."""
    lib = load()
    T = geom.B * geom.q_len
    row_count = T - row_begin if row_count is None else row_count
    _dev(q, "q", (_FP8, torch.uint8, torch.float32))
    _dev(k, "k", (_FP8, torch.uint8, torch.float32))
    _dev(w, "w", (torch.bfloat16, torch.int16, torch.uint16, torch.float32))
    _need(tuple(q.shape) == (T, 64, 128), f"q shape {tuple(q.shape)} != {(T, 64, 128)}")
    _need(tuple(k.shape) == _cache_shape(geom, pages, (128,)), "k shape mismatch")
    _need(tuple(w.shape) == (T, 64), "w shape mismatch")
    for name, s, shape in (("k_scale", k_scale, _cache_shape(geom, pages, ())), ("q_scale", q_scale, (T, 64))):
        if s is not None:
            _dev(s, name, (torch.float32,))
            _need(tuple(s.shape) == shape, f"{name} shape mismatch")
    if scores is None:
        scores = torch.empty((row_count, geom.S_max), dtype=torch.float32, device=q.device)
    _dev(scores, "scores", (torch.float32,))
    _need(scores.dim() == 2 and scores.shape[0] >= row_count, "scores too small")
    args = (_ptr(q), _index_dtype(q), _ptr(q_scale), _ptr(w), _w_dtype(w), _ptr(k), _index_dtype(k), _ptr(k_scale),
            row_begin, row_count, _ptr(scores), scores.stride(0), _stream(stream))
    if pages is None:
        _check(lib.dsa_indexer_scores(ctypes.byref(geom), *args), "dsa_indexer_scores")
    else:
        _check(lib.dsa_indexer_scores_paged(ctypes.byref(geom), ctypes.byref(pages), *args),
               "dsa_indexer_scores_paged")
    return scores


def workspace_size(B, q_len, S_max, H, k, which_call):
    """dsa_workspace_size: bytes enough for ``which_call`` (a CALL_* value) at
    this geometry with any supported dtype combination."""
    return int(load().dsa_workspace_size(B, q_len, S_max, H, k, which_call))


def topk_workspace_size(row_count, S_max, k):
    return int(load().dsa_topk_workspace_size(row_count, S_max, k))


def topk(geom, scores, k, row_begin=0, row_count=None, idx=None, ws=None, stream=None):
    """dsa_topk: returns int32 indices [row_count, k] (ascending, -1 padded)."""
    lib = load()
    T = geom.B * geom.q_len
    row_count = T - row_begin if row_count is None else row_count
    _dev(scores, "scores", (torch.float32,))
    if idx is None:
        idx = torch.empty((row_count, k), dtype=torch.int32, device=scores.device)
    _dev(idx, "idx", (torch.int32,))
    need = topk_workspace_size(row_count, geom.S_max, k)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=scores.device)
    st = lib.dsa_topk(ctypes.byref(geom), _ptr(scores), scores.stride(0), row_begin, row_count, k, _ptr(idx),
                      _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "dsa_topk")
    return idx


def sparse_mla_workspace_size(B, q_len, H, k, dtype):
    return int(load().dsa_sparse_mla_workspace_size(B, q_len, H, k, dtype))


def sparse_mla_paged_workspace_size(B, q_len, H, k, dtype):
    return int(load().dsa_sparse_mla_paged_workspace_size(B, q_len, H, k, dtype))


def sparse_mla(geom, q, kv, idx, sm_scale, out=None, lse=None, ws=None, want_lse=True, stream=None, pages=None):
    """dsa_sparse_mla (dsa_sparse_mla_paged when ``pages`` is given, with
    ``kv`` the page pool): returns (out [T, H, 512], lse [T, H] or None)."""
    lib = load()
    T = geom.B * geom.q_len
    _dev(q, "q", (torch.bfloat16, torch.float32, torch.int16, torch.uint16))
    _dev(kv, "kv", (q.dtype,))
    _dev(idx, "idx", (torch.int32,))
    _need(q.dim() == 3 and q.shape[0] == T and q.shape[2] == 576, "q must be [T, H, 576]")
    _need(tuple(kv.shape) == _cache_shape(geom, pages, (576,)), "kv shape mismatch")
    _need(idx.dim() == 2 and idx.shape[0] == T, "idx must be [T, k]")
    H, k = q.shape[1], idx.shape[1]
    if out is None:
        out = torch.empty((T, H, 512), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    dt = _mla_dtype(q)
    if pages is None:
        need = sparse_mla_workspace_size(geom.B, geom.q_len, H, k, dt)
    else:
        need = sparse_mla_paged_workspace_size(geom.B, geom.q_len, H, k, dt)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    args = (H, k, float(sm_scale), _ptr(q), dt, _ptr(kv), _ptr(idx), _ptr(out), _ptr(lse), _ptr(ws),
            ws.numel() * ws.element_size(), _stream(stream))
    if pages is None:
        _check(lib.dsa_sparse_mla(ctypes.byref(geom), *args), "dsa_sparse_mla")
    else:
        _check(lib.dsa_sparse_mla_paged(ctypes.byref(geom), ctypes.byref(pages), *args), "dsa_sparse_mla_paged")
    return out, lse


def forward_workspace_size(B, q_len, S_max, H, topk_k, index_dtype, mla_dtype):
    return int(load().dsa_forward_workspace_size(B, q_len, S_max, H, topk_k, index_dtype, mla_dtype))


def indexer_topk_workspace_size(B, q_len, S_max, topk_k, index_dtype):
    return int(load().dsa_indexer_topk_workspace_size(B, q_len, S_max, topk_k, index_dtype))


def indexer_topk(geom, topk_k, index_q, index_w, index_k, index_k_scale=None, index_q_scale=None, idx=None, ws=None,
                 stream=None):
    """dsa_indexer_topk: the indexer and the top-k of dsa_forward, without the
    attention.  Returns idx [T, topk_k] int32 (ascending, -1 padded)."""
    lib = load()
    T = geom.B * geom.q_len
    dev = index_q.device
    if idx is None:
        idx = torch.empty((T, topk_k), dtype=torch.int32, device=dev)
    idt = _index_dtype(index_q)
    need = indexer_topk_workspace_size(geom.B, geom.q_len, geom.S_max, topk_k, idt)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    for name, t in (("index_q", index_q), ("index_w", index_w), ("index_k", index_k), ("idx", idx)):
        _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous device tensor")
    _need(tuple(index_q.shape) == (T, 64, 128) and tuple(index_k.shape) == _cache_shape(geom, None, (128,)),
          "indexer shapes mismatch")
    _need(tuple(idx.shape) == (T, topk_k) and idx.dtype == torch.int32, "idx must be [T, topk] int32")
    _check(lib.dsa_indexer_topk(ctypes.byref(geom), topk_k, _ptr(index_q), idt, _ptr(index_q_scale), _ptr(index_w),
                                _w_dtype(index_w), _ptr(index_k), _ptr(index_k_scale), _ptr(idx), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)), "dsa_indexer_topk")
    return idx


def forward_paged_workspace_size(B, q_len, S_max, H, topk_k, index_dtype, mla_dtype):
    return int(load().dsa_forward_paged_workspace_size(B, q_len, S_max, H, topk_k, index_dtype, mla_dtype))


def forward(geom, topk_k, sm_scale, index_q, index_w, index_k, mla_q, mla_kv, index_k_scale=None,
            index_q_scale=None, idx=None, out=None, lse=None, ws=None, want_lse=True, stream=None, pages=None):
    """dsa_forward: indexer -> top-k -> sparse MLA (dsa_forward_paged when
    ``pages`` is given, with ``index_k``, ``index_k_scale`` and ``mla_kv`` the
    page pools).  ``idx=False`` passes idx_out = NULL (the selection stays in
    the workspace and None is returned for it).  Returns (idx, out, lse)."""
    lib = load()
    T = geom.B * geom.q_len
    H = mla_q.shape[1]
    dev = mla_q.device
    no_idx = idx is False
    if idx is None:
        idx = torch.empty((T, topk_k), dtype=torch.int32, device=dev)
    elif no_idx:
        idx = None
    if out is None:
        out = torch.empty((T, H, 512), dtype=mla_q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    idt, mdt = _index_dtype(index_q), _mla_dtype(mla_q)
    size_fn = forward_workspace_size if pages is None else forward_paged_workspace_size
    need = size_fn(geom.B, geom.q_len, geom.S_max, H, topk_k, idt, mdt)
    if no_idx:
        need += (T * topk_k * 4 + 255) // 256 * 256
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    for name, t in (("index_q", index_q), ("index_w", index_w), ("index_k", index_k), ("mla_q", mla_q),
                    ("mla_kv", mla_kv), ("idx", idx), ("out", out)):
        if t is not None:
            _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous device tensor")
    _need(tuple(index_q.shape) == (T, 64, 128) and tuple(index_k.shape) == _cache_shape(geom, pages, (128,)),
          "indexer shapes mismatch")
    _need(tuple(mla_kv.shape) == _cache_shape(geom, pages, (576,)) and mla_q.shape[0] == T, "MLA shapes mismatch")
    args = (H, topk_k, float(sm_scale), _ptr(index_q), idt, _ptr(index_q_scale), _ptr(index_w), _w_dtype(index_w),
            _ptr(index_k), _ptr(index_k_scale), _ptr(mla_q), _ptr(mla_kv), mdt, _ptr(idx), _ptr(out), _ptr(lse),
            _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if pages is None:
        _check(lib.dsa_forward(ctypes.byref(geom), *args), "dsa_forward")
    else:
        _check(lib.dsa_forward_paged(ctypes.byref(geom), ctypes.byref(pages), *args), "dsa_forward_paged")
    return idx, out, lse


def forward_noalloc(geom, topk_k, sm_scale, index_q, index_w, index_k, mla_q, mla_kv, index_k_scale=None,
                    index_q_scale=None, idx=None, out=None, lse=None, want_lse=True, stream=None):
    """dsa_forward_noalloc: dsa_forward with the library's static scratch
    instead of a workspace (pass preallocated idx / out / lse to allocate
    nothing at all).  ``idx=False`` passes idx_out = NULL.  Returns (idx, out, lse)."""
    lib = load()
    T = geom.B * geom.q_len
    H = mla_q.shape[1]
    dev = mla_q.device
    no_idx = idx is False
    if idx is None:
        idx = torch.empty((T, topk_k), dtype=torch.int32, device=dev)
    elif no_idx:
        idx = None
    if out is None:
        out = torch.empty((T, H, 512), dtype=mla_q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    for name, t in (("index_q", index_q), ("index_w", index_w), ("index_k", index_k), ("mla_q", mla_q),
                    ("mla_kv", mla_kv), ("idx", idx), ("out", out)):
        if t is not None:
            _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous device tensor")
    _need(tuple(index_q.shape) == (T, 64, 128) and tuple(index_k.shape) == (geom.B, geom.S_max, 128),
          "indexer shapes mismatch")
    _need(tuple(mla_kv.shape) == (geom.B, geom.S_max, 576) and mla_q.shape[0] == T, "MLA shapes mismatch")
    st = lib.dsa_forward_noalloc(ctypes.byref(geom), H, topk_k, float(sm_scale), _ptr(index_q), _index_dtype(index_q),
                                 _ptr(index_q_scale), _ptr(index_w), _w_dtype(index_w), _ptr(index_k),
                                 _ptr(index_k_scale), _ptr(mla_q), _ptr(mla_kv), _mla_dtype(mla_q), _ptr(idx),
                                 _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "dsa_forward_noalloc")
    return idx, out, lse


def _quant_dtype(t):
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"quantisation input dtype {t.dtype} unsupported")


def indexer_quantize(x, codes=None, scales=None, stream=None):
    """dsa_indexer_quantize: x [..., 128] bf16/fp32 -> (uint8 codes [..., 128], fp32 scales [...])."""
    lib = load()
    _dev(x, "x", (torch.bfloat16, torch.int16, torch.uint16, torch.float32))
    _need(x.dim() >= 1 and x.shape[-1] == 128, "x must be [..., 128]")
    rows = x.numel() // 128
    if codes is None:
        codes = torch.empty(tuple(x.shape), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(tuple(x.shape[:-1]), dtype=torch.float32, device=x.device)
    _dev(codes, "codes", (torch.uint8, _FP8))
    _dev(scales, "scales", (torch.float32,))
    _need(codes.numel() == x.numel() and scales.numel() == rows, "codes / scales size mismatch")
    st = lib.dsa_indexer_quantize(_ptr(x), _quant_dtype(x), rows, _ptr(codes), _ptr(scales), _stream(stream))
    _check(st, "dsa_indexer_quantize")
    return codes, scales


def indexer_cache_append(geom, k_new, k_cache, k_scale_cache, stream=None, pages=None):
    """dsa_indexer_cache_append (dsa_indexer_cache_append_paged when ``pages``
    is given, with the caches the page pools): quantise k_new [B, q_len, 128]
    into the caches in place."""
    lib = load()
    _dev(k_new, "k_new", (torch.bfloat16, torch.int16, torch.uint16, torch.float32))
    _dev(k_cache, "k_cache", (torch.uint8, _FP8))
    _dev(k_scale_cache, "k_scale_cache", (torch.float32,))
    _need(tuple(k_new.shape) == (geom.B, geom.q_len, 128), "k_new must be [B, q_len, 128]")
    _need(tuple(k_cache.shape) == _cache_shape(geom, pages, (128,)), "k_cache shape mismatch")
    _need(tuple(k_scale_cache.shape) == _cache_shape(geom, pages, ()), "k_scale_cache shape mismatch")
    args = (_ptr(k_new), _quant_dtype(k_new), _ptr(k_cache), _ptr(k_scale_cache), _stream(stream))
    if pages is None:
        _check(lib.dsa_indexer_cache_append(ctypes.byref(geom), *args), "dsa_indexer_cache_append")
    else:
        _check(lib.dsa_indexer_cache_append_paged(ctypes.byref(geom), ctypes.byref(pages), *args),
               "dsa_indexer_cache_append_paged")
    return k_cache, k_scale_cache


def mha_prefill_workspace_size(B, S_max, H):
    return int(load().dsa_mha_prefill_workspace_size(B, S_max, H))


def mha_prefill(geom, q, kv, wkv_b, sm_scale, out=None, lse=None, ws=None, want_lse=True, stream=None):
    """dsa_mha_prefill: MHA-mode prefill for sequences within top-k.
    q [T, H, 192], kv [B, S_max, 576], wkv_b [H, 256, 512] (bf16).
    Returns (out [T, H, 128], lse [T, H] or None)."""
    lib = load()
    T = geom.B * geom.q_len
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    _dev(q, "q", bf)
    _dev(kv, "kv", bf)
    _dev(wkv_b, "wkv_b", bf)
    _need(q.dim() == 3 and q.shape[0] == T and q.shape[2] == 192, "q must be [T, H, 192]")
    H = q.shape[1]
    _need(tuple(kv.shape) == (geom.B, geom.S_max, 576), "kv must be [B, S_max, 576]")
    _need(tuple(wkv_b.shape) == (H, 256, 512), "wkv_b must be [H, 256, 512]")
    if out is None:
        out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    need = mha_prefill_workspace_size(geom.B, geom.S_max, H)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib.dsa_mha_prefill(ctypes.byref(geom), H, float(sm_scale), _ptr(q), _ptr(kv), _ptr(wkv_b), BF16, _ptr(out),
                             _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "dsa_mha_prefill")
    return out, lse


def indexer_kl_workspace_size(B, q_len, S_max, k):
    return int(load().dsa_indexer_kl_workspace_size(B, q_len, S_max, k))


def indexer_kl(geom, q, kv, lse, scores, sm_scale, idx=None, kl=None, loss=None, ws=None, stream=None):
    """dsa_indexer_kl: the indexer's KL objective (forward).  q [T, H, 576] and
    kv [B, S_max, 576] bf16, lse [T, H] fp32, scores [T, >= S_max] fp32, idx
    [T, k] int32 or None (every visible position).  Returns (kl [T], loss [1])."""
    lib = load()
    T = geom.B * geom.q_len
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    _dev(q, "q", bf)
    _dev(kv, "kv", bf)
    _dev(lse, "lse", (torch.float32,))
    _need(q.dim() == 3 and q.shape[0] == T and q.shape[2] == 576, "q must be [T, H, 576]")
    H = q.shape[1]
    _need(tuple(kv.shape) == (geom.B, geom.S_max, 576), "kv must be [B, S_max, 576]")
    _need(tuple(lse.shape) == (T, H), "lse must be [T, H]")
    _need(scores.is_cuda and scores.dtype == torch.float32 and scores.dim() == 2 and scores.shape[0] == T
          and scores.stride(1) == 1, "scores must be a row-major fp32 device tensor [T, ld]")
    k = 0
    if idx is not None:
        _dev(idx, "idx", (torch.int32,))
        _need(idx.dim() == 2 and idx.shape[0] == T, "idx must be [T, k]")
        k = idx.shape[1]
    if kl is None:
        kl = torch.empty((T,), dtype=torch.float32, device=q.device)
    if loss is None:
        loss = torch.empty((1,), dtype=torch.float32, device=q.device)
    need = indexer_kl_workspace_size(geom.B, geom.q_len, geom.S_max, k)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.dsa_indexer_kl(ctypes.byref(geom), H, float(sm_scale), _ptr(q), _ptr(kv), BF16, _ptr(lse), _ptr(scores),
                            scores.stride(0), _ptr(idx), k, _ptr(kl), _ptr(loss), _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "dsa_indexer_kl")
    return kl, loss
