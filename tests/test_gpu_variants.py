"""GPU parity for kernel variants the workload tests do not reach: HISA's
stage 1 and stage 2 for few queries and fp32 inputs, the flat indexer's
vector kernel in bf16 and its fused path at d_i = 32, the streamed (one
query per sequence) and sparse attention kernels at every MFMA head shape,
and the general split-K merge (more than 64 splits per query, or head sizes
off the fast merge's grid).  Each case is checked against the oracle:
selections bit-exact on integer grids, attention within 1e-2 (1e-4 fp32)."""
import math

import numpy as np
import pytest
import torch

import oracle
from compressed_attention_amd import ops, synth
from helpers import f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _stage1_exact(q, k_i, B, weight_bits):
    # block sums S_b are integers and representatives S_b / B; with head
    # weights v / 2^bits every stage-1 partial sum is exact in fp32 when
    # max_v * sum_h sum_c |q_hc S_bc| < 2^24
    nb = -(-k_i.shape[0] // B)
    S = np.stack([k_i[j * B:(j + 1) * B].sum(0) for j in range(nb)])
    worst = (np.abs(q).reshape(-1, q.shape[-1]) @ np.abs(S).T).reshape(q.shape[0], q.shape[1], nb).sum(1).max()
    assert worst * ((1 << weight_bits) - 1) < 2**24, worst


@pytest.mark.parametrize("dtype,d_i,nq", [(torch.float32, 32, 1), (torch.float32, 32, 5), (torch.float32, 128, 5),
                                          (torch.bfloat16, 32, 1), (torch.bfloat16, 32, 5), (torch.bfloat16, 64, 1),
                                          (torch.bfloat16, 64, 5), (torch.bfloat16, 128, 5)])
def test_hisa_few_queries_exact(dtype, d_i, nq):
    # Fewer queries than the multi-query kernels take (stage 1 with one or
    # four queries per workgroup, stage 2 per chosen block), fp32 and bf16,
    # ragged visibility and a ragged last block; integer grid, 4-bit weights.
    bt, N, B, m, k = 2, 3001, 64, 6, 100
    q_i = synth.int_grid((bt, nq, 16, d_i), 501 + d_i + nq, -4, 4, dtype=dtype)
    k_i = synth.int_grid((bt, N, d_i), 502 + d_i, -4, 4, dtype=dtype)
    w_i = synth.dyadic_uniform((bt, nq, 16), 503 + nq, bits=4)
    nv = torch.tensor([[N - 3 * j for j in range(nq)], [B * 5 + 7 + 100 * j for j in range(nq)]], dtype=torch.int32)
    kd = k_i.to(DEV)
    reps = ops.hisa_pool(kd, B)
    idx, blk = ops.hisa_topk(q_i.to(DEV), kd, w_i.to(DEV), nv.to(DEV), reps, B, m, k, return_blocks=True)
    torch.cuda.synchronize()
    for b in range(bt):
        q, kk, ww = f64(q_i[b]), f64(k_i[b]), f64(w_i[b])
        _stage1_exact(q, kk, B, 4)
        ref, ref_blk = oracle.hisa_topk(q, kk, ww, nv[b].numpy(), B, m, k)
        assert np.array_equal(blk.cpu().numpy()[b], ref_blk), b
        assert np.array_equal(idx.cpu().numpy()[b], ref), b


def test_flat_bf16_vector_kernel_exact():
    # 4 indexer heads (the MFMA kernels take 16): the vector kernel in bf16.
    bt, nq, N, k = 2, 8, 700, 64
    q_i = synth.int_grid((bt, nq, 4, 32), 511, -8, 8, dtype=torch.bfloat16)
    k_i = synth.int_grid((bt, N, 32), 512, -8, 8, dtype=torch.bfloat16)
    w_i = synth.dyadic_uniform((bt, nq, 4), 513)
    nv = torch.tensor([[N - 11 * j for j in range(nq)], [5 + 80 * j for j in range(nq)]], dtype=torch.int32)
    idx = ops.index_topk(q_i.to(DEV), k_i.to(DEV), w_i.to(DEV), nv.to(DEV), k)
    torch.cuda.synchronize()
    for b in range(bt):
        ref = oracle.flat_topk(f64(q_i[b]), f64(k_i[b]), f64(w_i[b]), nv[b].numpy(), k)
        assert np.array_equal(idx.cpu().numpy()[b], ref), b


def test_flat_fused_long_rows_d32_exact():
    # Rows past 16,384 keys with 16 queries per workgroup at d_i = 32: the
    # sampled threshold and the collecting score pass of that width.
    bt, nq, N, k = 1, 32, 20000, 256
    q_i = synth.int_grid((bt, nq, 16, 32), 521, -8, 8, dtype=torch.bfloat16)
    k_i = synth.int_grid((bt, N, 32), 522, -8, 8, dtype=torch.bfloat16)
    w_i = synth.dyadic_uniform((bt, nq, 16), 523)
    pos = torch.arange(N - nq, N, dtype=torch.int32).reshape(1, nq)
    nv = ops.visible_count(pos.to(DEV), 1, 1, N)
    idx = ops.index_topk(q_i.to(DEV), k_i.to(DEV), w_i.to(DEV), nv, k)
    torch.cuda.synchronize()
    rows = [0, 7, 16, 31]
    ref = oracle.flat_topk(f64(q_i[0, rows]), f64(k_i[0]), f64(w_i[0, rows]), nv.cpu().numpy()[0][rows], k)
    assert np.array_equal(idx.cpu().numpy()[0, rows], ref)


@pytest.mark.parametrize("h,d", [(16, 64), (16, 128), (32, 64), (32, 128), (64, 64), (64, 128)])
def test_decode_shape_attention_every_mfma_shape(h, d):
    # One query per sequence (K|V streamed) for sparse and dense attention at
    # every MFMA head shape; ragged visible counts, holes in the index lists.
    bt, L, N, k = 3, 3000, 2000, 256
    dt = torch.bfloat16
    raw = synth.normal((bt, L, 2 * d), 531 + d, dtype=dt).to(DEV)
    ckv = synth.normal((bt, N, 2 * d), 532 + d, dtype=dt).to(DEV)
    q = synth.normal((bt, 1, h, d), 533 + h, dtype=dt).to(DEV)
    pos = torch.tensor([[2999], [1500], [40]], dtype=torch.int32)
    nv = torch.tensor([[2000], [1371], [3]], dtype=torch.int32)
    idx = synth.random_index_lists(nv.reshape(-1), k, seed=534 + h, n_pad_holes=3).reshape(bt, 1, k)
    o_s, l_s = ops.sparse_attn(q, ckv, idx.to(DEV), raw, pos.to(DEV), 128, return_lse=True)
    o_d, l_d = ops.dense_compressed_attn(q, ckv, nv.to(DEV), raw, pos.to(DEV), 128, return_lse=True)
    torch.cuda.synchronize()
    sc = 1 / math.sqrt(d)
    for b in range(bt):
        ro, rl = oracle.sparse_attention(f64(q[b]), f64(ckv[b]), idx[b].numpy(), f64(raw[b]), pos[b].numpy(), 128, sc)
        assert np.abs(f64(o_s[b]) - ro).max() < 1e-2 and np.abs(f64(l_s[b]) - rl).max() < 1e-2, b
        ro, rl = oracle.dense_compressed_attention(f64(q[b]), f64(ckv[b]), nv[b].numpy(), f64(raw[b]), pos[b].numpy(),
                                                   128, sc)
        assert np.abs(f64(o_d[b]) - ro).max() < 1e-2 and np.abs(f64(l_d[b]) - rl).max() < 1e-2, b


@pytest.mark.parametrize("h,d", [(16, 64), (32, 64), (32, 128)])
def test_sparse_multi_query_shapes(h, d):
    # Several queries per sequence (K|V through L2) in sparse attention at the
    # smaller MFMA head shapes; holes, out-of-range indices, partial windows.
    bt, nq, L, N, k = 2, 6, 1500, 900, 200
    dt = torch.bfloat16
    raw = synth.normal((bt, L, 2 * d), 561 + d, dtype=dt).to(DEV)
    ckv = synth.normal((bt, N, 2 * d), 562 + d, dtype=dt).to(DEV)
    q = synth.normal((bt, nq, h, d), 563 + h, dtype=dt).to(DEV)
    pos = torch.tensor([[0, 5, 127, 128, 900, 1499]] * bt, dtype=torch.int32)
    nv = torch.tensor([[0, 1, 30, 31, 224, 373], [900, 17, 0, 400, 2, 899]], dtype=torch.int32)
    idx = synth.random_index_lists(nv.reshape(-1), k, seed=564 + h, n_pad_holes=4).reshape(bt, nq, k)
    idx[1, 3, 10] = N + 5  # out of range: skipped
    out, lse = ops.sparse_attn(q, ckv, idx.to(DEV), raw, pos.to(DEV), 128, return_lse=True)
    torch.cuda.synchronize()
    for b in range(bt):
        ii = idx[b].numpy().copy()
        ii[ii >= N] = -1
        ro, rl = oracle.sparse_attention(f64(q[b]), f64(ckv[b]), ii, f64(raw[b]), pos[b].numpy(), 128,
                                         1 / math.sqrt(d))
        assert np.abs(f64(out[b]) - ro).max() < 1e-2 and np.abs(f64(lse[b]) - rl).max() < 1e-2, b


def test_merge_of_many_splits():
    # One query over 20,000 entries: 158 splits of 128 keys, more than the
    # fast merge holds (64), so the general merge combines them.
    h, d, N, L = 64, 128, 20000, 30000
    dt = torch.bfloat16
    raw = synth.normal((1, L, 2 * d), 541, dtype=dt).to(DEV)
    ckv = synth.normal((1, N, 2 * d), 542, dtype=dt).to(DEV)
    q = synth.normal((1, 1, h, d), 543, dtype=dt).to(DEV)
    pos = torch.tensor([[L - 1]], dtype=torch.int32)
    nv = torch.tensor([[N]], dtype=torch.int32)
    out, lse = ops.dense_compressed_attn(q, ckv, nv.to(DEV), raw, pos.to(DEV), 128, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_compressed_attention(f64(q[0]), f64(ckv[0]), nv[0].numpy(), f64(raw[0]), pos[0].numpy(),
                                               128, 1 / math.sqrt(d))
    assert np.abs(f64(out[0]) - ro).max() < 1e-2
    assert np.abs(f64(lse[0]) - rl).max() < 1e-2


def test_merge_off_grid_head_size_fp32():
    # fp32 vector attention with d = 40 (not a multiple of 64): its split-K
    # partials take the general merge.
    h, d, N, L, nq = 8, 40, 900, 1200, 2
    raw = synth.normal((1, L, 2 * d), 551).to(DEV)
    ckv = synth.normal((1, N, 2 * d), 552).to(DEV)
    q = synth.normal((1, nq, h, d), 553).to(DEV)
    pos = torch.tensor([[L - 1, 700]], dtype=torch.int32)
    nv = torch.tensor([[N, 500]], dtype=torch.int32)
    out, lse = ops.dense_compressed_attn(q, ckv, nv.to(DEV), raw, pos.to(DEV), 128, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_compressed_attention(f64(q[0]), f64(ckv[0]), nv[0].numpy(), f64(raw[0]), pos[0].numpy(),
                                               128, 1 / math.sqrt(d))
    assert np.abs(f64(out[0]) - ro).max() < 1e-4
    assert np.abs(f64(lse[0]) - rl).max() < 1e-4
