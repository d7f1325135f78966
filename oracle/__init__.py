"""CPU oracle for the DeepSeek Sparse Attention (DSA) forward path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``long_context_lightning_amd``) and never reads anything the GPU
computed except the values a test hands it to check.

Plain NumPy in float64 (int-exact for fp8 dot products).  Each function cites
the passage of the pages it follows:

* "详解DSA" (obnotes page): Eq.(1) Lightning Indexer score, Eq.(2) attention
  over the top-k entries, the ``Indexer`` code block (fp8 cache, the
  ``weights`` fold, ``+= mask`` and ``topk(min(index_topk, end_pos))``), and
  the "DSA计算流" section (q-scale multiplies the ReLU output per head, k-scale
  multiplies the head sum; short sequences keep every position).
* "DeepSeek V3.2 稀疏注意力" (charlestar page): the two-stage data flow, the
  MQA-mode sharing of one selected set by all heads, and the "Top-k 是算法与
  kernel 的交界面" list of what an implementation must define.
* "NSA 与 DSA" (luowle page) section 3.2: public config 64 heads x 128 dims,
  top-k 2048, one shared indexer key per token.
* ``quant``: the ``act_quant`` step of the ``Indexer`` code block (per-128
  block e4m3fn codes with an ``amax / 448`` scale) and the key-cache append
  ``k_cache[:bsz, start_pos:end_pos] = k_fp8``.
* ``mha``: MHA-mode prefill for sequences no longer than top-k ("详解DSA",
  "DSA计算流" and its MLA forward code block; the charlestar page's
  short-prompt paragraph): ``wkv_b`` decompression, causal attention over the
  per-head keys and values.
* ``kl``: the indexer's KL objective, forward only ("详解DSA" Eq.(3)-(6)):
  head-summed, L1-normalised attention weights against Softmax(I), on every
  visible position or on the selected set.
* ``paged``: paged caches (charlestar page, "Prefill 与 decode 中发生了什么"
  and "Top-k 是算法与 kernel 的交界面"): a block table maps a logical
  position to a page and an offset.

"""

from .formats import decode_bf16, decode_e4m3fn, e4m3fn_times_512
from .quant import cache_append, e4m3fn_nearest, quantize_blocks
from .paged import gather_pages, scatter_pages
from .mha import decompress as mha_decompress, mha_prefill
from .kl import attention_lse, indexer_kl
from .dsa import (
    query_positions,
    indexer_scores,
    topk_select,
    sparse_mla,
    dsa_forward,
)

__all__ = [
    "decode_bf16",
    "decode_e4m3fn",
    "e4m3fn_times_512",
    "query_positions",
    "indexer_scores",
    "topk_select",
    "sparse_mla",
    "dsa_forward",
    "e4m3fn_nearest",
    "quantize_blocks",
    "cache_append",
    "gather_pages",
    "scatter_pages",
    "mha_decompress",
    "mha_prefill",
    "attention_lse",
    "indexer_kl",
]
