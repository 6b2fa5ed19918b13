"""GPU parity: sparse (CSA) and dense (HCA) MQA attention vs the oracle.

Index lists and compressed caches are drawn directly by the input generator,
so attention error is measured on its own.  Bar: max-abs <= 1e-2 (bf16 in,
fp32 accumulate and output)."""
import math

import numpy as np
import pytest
import torch

import oracle
from compressed_attention_amd import ops, synth
from helpers import f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-2


def _check(out, lse, ref_o, ref_l, tol=TOL):
    err = np.abs(f64(out) - ref_o).max()
    assert err <= tol, err
    if lse is not None:
        lerr = np.abs(f64(lse) - ref_l).max()
        assert lerr <= tol, lerr
    return err


def test_tiny_layer_fp32_sparse_and_dense():
    t = synth.tiny_hybrid_layer(0).tensors
    raw = t["raw_kv"].to(DEV)
    q = t["q"].to(DEV)
    pos = t["q_pos"].to(DEV)
    ckv = synth.normal((1, 1023, 128), 71).to(DEV)
    nv = ops.visible_count(pos, 8, 4, 1023)
    idx = synth.random_index_lists(nv.cpu()[0], 64, seed=72, n_pad_holes=3).reshape(1, 64, 64)
    out, lse = ops.sparse_attn(q, ckv, idx.to(DEV), raw, pos, 128, return_lse=True)
    ro, rl = oracle.sparse_attention(f64(t["q"][0]), f64(ckv[0]), idx[0].numpy(), f64(t["raw_kv"][0]),
                                     t["q_pos"][0].numpy(), 128, 1 / math.sqrt(64))
    assert _check(out[0], lse[0], ro, rl) < 1e-4
    hca = synth.normal((1, 32, 128), 73).to(DEV)
    nvh = ops.visible_count(pos, 128, 128, 32)
    out, lse = ops.dense_compressed_attn(q, hca, nvh, raw, pos, 128, return_lse=True)
    ro, rl = oracle.dense_compressed_attention(f64(t["q"][0]), f64(hca[0]), nvh.cpu().numpy()[0], f64(t["raw_kv"][0]),
                                               t["q_pos"][0].numpy(), 128, 1 / math.sqrt(64))
    assert _check(out[0], lse[0], ro, rl) < 1e-4


def test_prefill_chunk_sparse_bf16():
    t = synth.csa_prefill_chunk(0).tensors
    N, nq, k = 8191, 1024, 512
    pos = t["q_pos"].to(DEV)
    ckv = synth.normal((1, N, 256), 74, dtype=torch.bfloat16).to(DEV)
    nv = ops.visible_count(pos, 8, 4, N)
    idx = synth.random_index_lists(nv.cpu()[0], k, seed=75).reshape(1, nq, k)
    out, lse = ops.sparse_attn(t["q"].to(DEV), ckv, idx.to(DEV), t["raw_kv"].to(DEV), pos, 128, return_lse=True)
    torch.cuda.synchronize()
    rows = sorted(set(np.random.default_rng(1).choice(nq, 48, replace=False).tolist()) | {0, nq - 1})
    ro, rl = oracle.sparse_attention(f64(t["q"][0, rows]), f64(ckv[0]), idx[0, rows].numpy(), f64(t["raw_kv"][0]),
                                     t["q_pos"][0, rows].numpy(), 128, 1 / math.sqrt(128))
    _check(out[0, rows], lse[0, rows], ro, rl)


def test_hca_decode_full_size_sampled():
    # 32 sequences of 2^20 raw tokens (device-generated), 8192 entries each,
    # one query per sequence at L-1: the split-key path with 64-bit offsets.
    bt, L, N = 32, 1 << 20, 8192
    raw = synth.normal((bt, L, 256), 76, dtype=torch.bfloat16, device=DEV)
    ckv = synth.normal((bt, N, 256), 77, dtype=torch.bfloat16, device=DEV)
    q = synth.normal((bt, 1, 64, 128), 78, dtype=torch.bfloat16, device=DEV)
    pos = torch.full((bt, 1), L - 1, dtype=torch.int32, device=DEV)
    nv = ops.visible_count(pos, 128, 128, N)
    out, lse = ops.dense_compressed_attn(q, ckv, nv, raw, pos, 128, return_lse=True)
    torch.cuda.synchronize()
    assert int(nv[0, 0]) == N
    for b in (0, 13, 31):
        ro, rl = oracle.dense_compressed_attention(f64(q[b]), f64(ckv[b]), [N], f64(raw[b, L - 128:]),
                                                   np.array([127]), 128, 1 / math.sqrt(128))
        _check(out[b], lse[b], ro, rl)


@pytest.mark.parametrize("h,d", [(64, 128), (32, 128), (16, 128), (16, 64), (32, 64), (64, 64), (8, 128), (24, 64)])
def test_shapes_and_edges_dense(h, d):
    bt, nq, L, N = 2, 9, 900, 200
    dt = torch.bfloat16
    raw = synth.normal((bt, L, 2 * d), 80, dtype=dt).to(DEV)
    ckv = synth.normal((bt, N, 2 * d), 81, dtype=dt).to(DEV)
    q = synth.normal((bt, nq, h, d), 82, dtype=dt).to(DEV)
    pos = torch.tensor([[0, 1, 5, 126, 127, 128, 500, 898, 899]] * bt, dtype=torch.int32)
    nv = torch.tensor([[0, 0, 3, 64, 65, 1, 199, 200, 200], [0, 63, 17, 0, 128, 129, 2, 150, 200]], dtype=torch.int32)
    out, lse = ops.dense_compressed_attn(q, ckv, nv.to(DEV), raw, pos.to(DEV), 128, return_lse=True)
    torch.cuda.synchronize()
    for b in range(bt):
        ro, rl = oracle.dense_compressed_attention(f64(q[b]), f64(ckv[b]), nv[b].numpy(), f64(raw[b]),
                                                   pos[b].numpy(), 128, 1 / math.sqrt(d))
        _check(out[b], lse[b], ro, rl)


@pytest.mark.parametrize("d", [128, 64])
def test_dense_decode_ragged_visible_counts(d):
    """One query per sequence (the decode launch: streamed K|V, chunks of
    128 keys over 3,000 entries) with visible counts from 0 to all entries:
    a chunk's first tile is loaded before its query's visible count is
    known, and must be dropped and fetched again wherever the tile is not
    a full run of visible entries (chunks past the count, the window's
    chunk, empty chunks)."""
    bt, L, N, h = 8, 4000, 3000, 64
    dt = torch.bfloat16
    raw = synth.normal((bt, L, 2 * d), 110 + d, dtype=dt).to(DEV)
    ckv = synth.normal((bt, N, 2 * d), 111 + d, dtype=dt).to(DEV)
    q = synth.normal((bt, 1, h, d), 112 + d, dtype=dt).to(DEV)
    pos = torch.tensor([[0], [5], [300], [1000], [1999], [2500], [3998], [3999]], dtype=torch.int32)
    nv = torch.tensor([[0], [1], [63], [64], [65], [1500], [2999], [3000]], dtype=torch.int32)
    out, lse = ops.dense_compressed_attn(q, ckv, nv.to(DEV), raw, pos.to(DEV), 128, return_lse=True)
    torch.cuda.synchronize()
    for b in range(bt):
        ro, rl = oracle.dense_compressed_attention(f64(q[b]), f64(ckv[b]), nv[b].numpy(), f64(raw[b]),
                                                   pos[b].numpy(), 128, 1 / math.sqrt(d))
        _check(out[b], lse[b], ro, rl)


@pytest.mark.parametrize("h", [64, 16])
def test_sparse_edges_and_all_entries_equal_dense(h):
    bt, nq, L, N, d = 2, 6, 700, 300, 128
    dt = torch.bfloat16
    raw = synth.normal((bt, L, 2 * d), 90, dtype=dt).to(DEV)
    ckv = synth.normal((bt, N, 2 * d), 91, dtype=dt).to(DEV)
    q = synth.normal((bt, nq, h, d), 92, dtype=dt).to(DEV)
    pos = torch.tensor([[3, 64, 200, 450, 600, 699]] * bt, dtype=torch.int32).to(DEV)
    nv = ops.visible_count(pos, 8, 4, N)
    k = 320
    # every visible entry listed (padded with -1): must equal the dense path
    idx = torch.full((bt, nq, k), -1, dtype=torch.int32)
    for b in range(bt):
        for i in range(nq):
            n_ = int(nv[b, i])
            idx[b, i, :n_] = torch.arange(n_, dtype=torch.int32)
    o_s = ops.sparse_attn(q, ckv, idx.to(DEV), raw, pos, 128)
    o_d = ops.dense_compressed_attn(q, ckv, nv, raw, pos, 128)
    torch.cuda.synchronize()
    # The two calls may split the key list differently, which changes where
    # P is rounded to bf16; they agree to the attention tolerance, and each
    # matches the oracle.
    assert (o_s - o_d).abs().max().item() < TOL
    for b in range(bt):
        ro, _ = oracle.dense_compressed_attention(f64(q[b]), f64(ckv[b]), nv[b].cpu().numpy(), f64(raw[b]),
                                                  pos[b].cpu().numpy(), 128, 1 / math.sqrt(d))
        _check(o_s[b], None, ro, None)
    # holes, out-of-range entries and an all -1 row are skipped
    idx2 = synth.random_index_lists(nv.cpu().reshape(-1), 40, seed=93, n_pad_holes=5).reshape(bt, nq, 40)
    idx2[0, 0, :] = -1
    idx2[1, 2, 0] = N + 5
    out = ops.sparse_attn(q, ckv, idx2.to(DEV), raw, pos, 16)
    torch.cuda.synchronize()
    for b in range(bt):
        ii = idx2[b].numpy().copy()
        ii[ii >= N] = -1
        ro, _ = oracle.sparse_attention(f64(q[b]), f64(ckv[b]), ii, f64(raw[b]), pos[b].cpu().numpy(), 16,
                                        1 / math.sqrt(d))
        _check(out[b], None, ro, None)


def test_deterministic():
    bt, N, L = 4, 8192, 4096
    raw = synth.normal((bt, L, 256), 95, dtype=torch.bfloat16).to(DEV)
    ckv = synth.normal((bt, N, 256), 96, dtype=torch.bfloat16).to(DEV)
    q = synth.normal((bt, 1, 64, 128), 97, dtype=torch.bfloat16).to(DEV)
    pos = torch.full((bt, 1), L - 1, dtype=torch.int32, device=DEV)
    nv = torch.full((bt, 1), N, dtype=torch.int32, device=DEV)
    a = ops.dense_compressed_attn(q, ckv, nv, raw, pos, 128)
    b = ops.dense_compressed_attn(q, ckv, nv, raw, pos, 128)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("d", [128, 64])
def test_long_chunks_ragged(d):
    # 18 queries x ~6K keys, 64 heads: chunks of 320 keys (5 tiles, an odd
    # count) over ragged visible counts, partial windows and sparse holes.
    bt, nq, L, N, h = 2, 9, 6500, 6000, 64
    dt = torch.bfloat16
    raw = synth.normal((bt, L, 2 * d), 100 + d, dtype=dt).to(DEV)
    ckv = synth.normal((bt, N, 2 * d), 101 + d, dtype=dt).to(DEV)
    q = synth.normal((bt, nq, h, d), 102 + d, dtype=dt).to(DEV)
    pos = torch.tensor([[0, 1, 63, 127, 128, 3000, 6497, 6498, 6499]] * bt, dtype=torch.int32)
    nv = torch.tensor([[0, 1, 63, 64, 65, 4097, 5999, 6000, 6000], [6000, 0, 5937, 17, 6000, 4000, 2, 128, 5001]],
                      dtype=torch.int32)
    out, lse = ops.dense_compressed_attn(q, ckv, nv.to(DEV), raw, pos.to(DEV), 128, return_lse=True)
    k = 5000
    idx = synth.random_index_lists(nv.reshape(-1), k, seed=103 + d, n_pad_holes=7).reshape(bt, nq, k)
    idx[1, 4, 100] = N + 9  # out of range: skipped
    out_s, lse_s = ops.sparse_attn(q, ckv, idx.to(DEV), raw, pos.to(DEV), 128, return_lse=True)
    torch.cuda.synchronize()
    for b in range(bt):
        ro, rl = oracle.dense_compressed_attention(f64(q[b]), f64(ckv[b]), nv[b].numpy(), f64(raw[b]),
                                                   pos[b].numpy(), 128, 1 / math.sqrt(d))
        _check(out[b], lse[b], ro, rl)
        ii = idx[b].numpy().copy()
        ii[ii >= N] = -1
        ro, rl = oracle.sparse_attention(f64(q[b]), f64(ckv[b]), ii, f64(raw[b]), pos[b].numpy(), 128,
                                         1 / math.sqrt(d))
        _check(out_s[b], lse_s[b], ro, rl)


def _ring_of(raw, R, last):
    """Rows last-R+1 .. last of raw [bt][L][C] at slots r % R (rows < 0
    left as NaN: nothing may read them)."""
    out = torch.full((raw.shape[0], R, raw.shape[2]), float("nan"), dtype=raw.dtype, device=raw.device)
    rows = torch.arange(max(0, last - R + 1), last + 1, device=raw.device)
    out[:, rows % R] = raw[:, rows]
    return out


@pytest.mark.parametrize("h,d,dt", [(64, 128, torch.bfloat16), (128, 64, torch.bfloat16), (24, 64, torch.bfloat16),
                                    (16, 64, torch.float32)])
def test_ring_window_reads_match_full(h, d, dt):
    """Both attention calls reading the window from a ring of the newest
    R raw rows give bit-for-bit what they give from all L rows: a chunk of
    queries whose windows straddle the ring's wrap, and one sequence still
    inside its first window."""
    bt, L, N, k, R = 2, 5000, 1249, 64, 256
    raw = synth.normal((bt, L, 2 * d), 90, dtype=dt).to(DEV)
    ckv = synth.normal((bt, N, 2 * d), 91, dtype=dt).to(DEV)
    q = synth.normal((bt, 13, h, d), 92, dtype=dt).to(DEV)
    # sequence 0: positions 3000 .. 3120 (their windows reach back to 2873;
    # slot 0 holds row 3072); sequence 1: positions 0 .. 120
    p0 = [3000, 3001, 3010, 3071, 3072, 3073, 3090, 3100, 3110, 3117, 3118, 3119, 3120]
    p1 = [0, 1, 2, 5, 63, 64, 100, 111, 112, 113, 118, 119, 120]
    pos = torch.tensor([p0, p1], dtype=torch.int32, device=DEV)
    ring = torch.stack([_ring_of(raw[b:b + 1], R, max(pp))[0] for b, pp in enumerate((p0, p1))])
    nv = ops.visible_count(pos, 8, 4, N)
    idx = torch.stack([synth.random_index_lists(nv.cpu()[b], k, seed=93 + b, n_pad_holes=2) for b in range(bt)])
    idx = idx.reshape(bt, 13, k).to(DEV)
    o_full, l_full = ops.sparse_attn(q, ckv, idx, raw, pos, 128, return_lse=True)
    o_ring, l_ring = ops.sparse_attn(q, ckv, idx, ring, pos, 128, return_lse=True, L=L)
    n_full = ops.sparse_attn_noalloc(q, ckv, idx, raw, pos, 128)
    n_ring = ops.sparse_attn_noalloc(q, ckv, idx, ring, pos, 128, L=L)
    d_full, dl_full = ops.dense_compressed_attn(q, ckv, nv, raw, pos, 128, return_lse=True)
    d_ring, dl_ring = ops.dense_compressed_attn(q, ckv, nv, ring, pos, 128, return_lse=True, L=L)
    torch.cuda.synchronize()
    for a, b in ((o_full, o_ring), (l_full, l_ring), (n_full, n_ring), (d_full, d_ring), (dl_full, dl_ring)):
        assert torch.isfinite(b).all()
        assert torch.equal(a, b)
    # and the full-array results are the oracle's
    for b, pp in enumerate((p0, p1)):
        ro, rl = oracle.sparse_attention(f64(q[b]), f64(ckv[b]), idx[b].cpu().numpy(), f64(raw[b]), np.array(pp),
                                         128, 1 / math.sqrt(d))
        _check(o_ring[b], l_ring[b], ro, rl)


@pytest.mark.parametrize("vscale,qscale", [(1000.0, 1.0), (1.0, 6.0), (1e6, 1.0), (1e30, 6.0)])
def test_split_partials_large_values(vscale, qscale):
    # Long key lists split over several workgroups, whose partial outputs are
    # kept as fp16 O/l: V rows of magnitude ~1,000 (O/l is a convex
    # combination of them, below fp16's 65,504), of magnitude ~1e6 and ~1e30
    # (beyond fp16's range: each split's O/l is scaled by a power of two
    # before it is stored), and sharp logits (q x 6, the lazy rescale moving
    # often).  The error must stay within the bound of the arithmetic:
    # |err| <= (2^-9 for the bf16 weights + 2^-11 for the fp16 partial) *
    # max |V|, with a factor 4 for accumulation.
    bt, nq, N, L, h, d = 2, 3, 8000, 9000, 64, 128
    dt = torch.bfloat16
    raw = synth.normal((bt, L, 2 * d), 120, dtype=dt)
    ckv = synth.normal((bt, N, 2 * d), 121, dtype=dt)
    raw[..., d:] = (raw[..., d:].float() * vscale).to(dt)
    ckv[..., d:] = (ckv[..., d:].float() * vscale).to(dt)
    q = (synth.normal((bt, nq, h, d), 122) * qscale).to(dt)
    pos = torch.tensor([[8999, 5000, 300]] * bt, dtype=torch.int32)
    nv = torch.tensor([[N, 1200, 9], [N - 1, 4000, 50]], dtype=torch.int32)
    out, lse = ops.dense_compressed_attn(q.to(DEV), ckv.to(DEV), nv.to(DEV), raw.to(DEV), pos.to(DEV), 128,
                                         return_lse=True)
    torch.cuda.synchronize()
    vmax = float(max(raw[..., d:].float().abs().max(), ckv[..., d:].float().abs().max()))
    bound = 4 * (2.0**-9 + 2.0**-11) * vmax
    for b in range(bt):
        ro, rl = oracle.dense_compressed_attention(f64(q[b]), f64(ckv[b]), nv[b].numpy(), f64(raw[b]),
                                                   pos[b].numpy(), 128, 1 / math.sqrt(d))
        got = f64(out[b])
        assert np.isfinite(got).all(), (vscale, qscale, b)
        err = float(np.abs(got - ro).max())
        assert err <= bound, (vscale, qscale, b, err, bound)
        assert float(np.abs(f64(lse[b]) - rl).max()) <= 1e-2
