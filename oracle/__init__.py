"""Plain fp64 CPU oracle for the hybrid compressed-attention path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
The HIP library never calls into this package and this package never calls
into the HIP library; the two share no code.  Everything here is NumPy in
float64, written for a reader to check against the pages by eye: no blocking,
fusion or reordering beyond what each definition states (chunking over
independent queries or entries, where present, only bounds host memory).

Sources (cited by page title and section):
  [HYB]  process-cxr.github.io, "Hybrid Attention" (ai-library/architecture/attention)
  [HCA]  daiw.net, "前代 · HCA：128 倍压缩后再做稠密注意力" (deepseek-v4-flash/hca)
  [HISA] my.qihongyi.cn/?p=787, "DeepSeek速度狂飙4倍还不丢精度"
  [CARD] models.inteligile.com, "Compressed Sparse Attention" technique card
  [TRDM] trdm.cn/news/749237, section 2.1 (CSA/HCA cost summary)

Every function is pinned by ``tests/test_oracle_*.py`` to something other
than itself (closed forms, library routines, brute force on tiny inputs,
invariants).  One property has no pin: agreement with any trained DeepSeek
model's own numerics ("parity unpinned": no weights or printed values exist).
"""

from .hattn_ref import (  # noqa: F401
    n_entries,
    entry_span,
    n_visible,
    compress,
    compress_channel_logits,
    compress_with_index,
    index_scores,
    topk_select,
    flat_topk,
    hisa_pool,
    hisa_topk,
    block_sparse_topk,
    window_rows,
    attend,
    sparse_attention,
    dense_compressed_attention,
    csa2_layer_group,
    lse_merge,
)
