"""Hybrid compressed attention (CSA + HCA + HISA) for MI355X (gfx950).

The compute path is libhattn.so: hand-written HIP kernels behind a C ABI
(include/hattn.h).  This package is its thin binding (``ops``) plus the
seeded synthetic-input recipes (``synth``).  The library is loaded on first
use; without it every op raises (there is no CPU fallback).
"""
from .ops import (  # noqa: F401
    compress,
    compress_channel_logits,
    compress_with_index,
    dense_compressed_attn,
    hisa_pool,
    block_sparse_topk,
    hisa_topk,
    index_topk,
    sparse_attn,
    timer_collect,
    timer_enable,
    visible_count,
)

__all__ = [
    "compress",
    "compress_with_index",
    "compress_channel_logits",
    "visible_count",
    "index_topk",
    "hisa_pool",
    "hisa_topk",
    "block_sparse_topk",
    "sparse_attn",
    "dense_compressed_attn",
    "timer_enable",
    "timer_collect",
]
