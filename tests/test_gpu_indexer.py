"""GPU parity: flat indexer top-k and HISA two-stage selection vs the oracle.

Integer-grid inputs make every fp32 score exact, so indices must be
bit-identical; float inputs are held to mean IoU >= 0.999 plus the check
that every disagreement sits at the selection boundary."""
import numpy as np
import pytest
import torch

import oracle
from compressed_attention_amd import ops, synth
from helpers import check_near_ties, f64, iou_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _nvis_entry_space(nq, N):
    # queries at the end of the entry sequence: query j sits at entry N - nq + j
    pos = torch.arange(N - nq, N, dtype=torch.int32).reshape(1, nq)
    return ops.visible_count(pos.to(DEV), 1, 1, N)


def _rows(nq, count, seed=0):
    rng = np.random.default_rng(seed)
    return sorted(set(rng.choice(nq, min(nq, count), replace=False).tolist()) | {0, nq - 1})


def test_tiny_layer_fp32_flat_exact():
    t = synth.tiny_hybrid_layer(0).tensors
    nv = ops.visible_count(t["q_pos"].to(DEV), 8, 4, 1023)
    idx, sc = ops.index_topk(t["q_i"].to(DEV), t["k_i"].to(DEV), t["w_i"].to(DEV), nv, 64, return_scores=True)
    torch.cuda.synchronize()
    nv_o = np.array([oracle.n_visible(int(p), 8, 4, 1023) for p in t["q_pos"][0]])
    assert np.array_equal(nv.cpu().numpy()[0], nv_o)
    ref, ref_sc = oracle.flat_topk(f64(t["q_i"][0]), f64(t["k_i"][0]), f64(t["w_i"][0]), nv_o, 64, return_scores=True)
    assert np.array_equal(idx.cpu().numpy()[0], ref)
    got_sc = f64(sc[0])
    assert np.array_equal(np.where(ref >= 0, got_sc, 0), np.where(ref >= 0, ref_sc, 0))


@pytest.mark.parametrize("nq,N,k,hi", [(1024, 8191, 512, 8), (37, 1000, 64, 8), (16, 70000, 700, 4)])
def test_bf16_mfma_integer_grid_exact(nq, N, k, hi):
    # 16 heads x 64 dims on the grid [-8, 8] (16 x 128 on [-4, 4]) keep every
    # fp32 partial sum an exact multiple of 2^-8 below 2^24.
    d = 64 if hi == 8 else 128
    q_i = synth.int_grid((1, nq, 16, d), 41, -hi, hi, dtype=torch.bfloat16)
    k_i = synth.int_grid((1, N, d), 42, -hi, hi, dtype=torch.bfloat16)
    w_i = synth.dyadic_uniform((1, nq, 16), 43)
    nv = _nvis_entry_space(nq, N)
    idx = ops.index_topk(q_i.to(DEV), k_i.to(DEV), w_i.to(DEV), nv, k)
    torch.cuda.synchronize()
    rows = _rows(nq, 48)
    nvh = nv.cpu().numpy()[0]
    ref = oracle.flat_topk(f64(q_i[0, rows]), f64(k_i[0]), f64(w_i[0, rows]), nvh[rows], k)
    assert np.array_equal(idx.cpu().numpy()[0, rows], ref)


def test_indexer_128k_integer_grid_exact_sampled():
    # The 128K-entry chunk at full size (multi-level selection), grid [-4, 4].
    w = synth.indexer_128k(0, integer_grid=True)
    t = w.tensors
    N, nq, k = 131072, 1024, 2048
    nv = _nvis_entry_space(nq, N)
    idx = ops.index_topk(t["q_i"].to(DEV), t["k_i"].to(DEV), t["w_i"].to(DEV), nv, k)
    torch.cuda.synchronize()
    rows = _rows(nq, 10)
    ref = oracle.flat_topk(f64(t["q_i"][0, rows]), f64(t["k_i"][0]), f64(t["w_i"][0, rows]),
                           nv.cpu().numpy()[0][rows], k)
    assert np.array_equal(idx.cpu().numpy()[0, rows], ref)


def test_float_inputs_iou_and_boundary():
    t = synth.csa_prefill_chunk(0).tensors
    N, nq, k = 8191, 1024, 512
    nv = ops.visible_count(t["q_pos"].to(DEV), 8, 4, N)
    idx = ops.index_topk(t["q_i"].to(DEV), t["k_i"].to(DEV), t["w_i"].to(DEV), nv, k)
    torch.cuda.synchronize()
    rows = _rows(nq, 96)
    nvh = nv.cpu().numpy()[0]
    q, kk, ww = f64(t["q_i"][0]), f64(t["k_i"][0]), f64(t["w_i"][0])
    ref = oracle.flat_topk(q[rows], kk, ww[rows], nvh[rows], k)
    got = idx.cpu().numpy()[0, rows]
    mean, mn = iou_rows(got, ref)
    assert mean >= 0.999, (mean, mn)

    def scores(r):
        return oracle.index_scores(q[rows[r]], kk[: nvh[rows[r]]], ww[rows[r]])

    def tol(r):  # fp32 accumulation bound: d * 2^-23 * sum_h w |q||k|
        qa = np.abs(q[rows[r]])
        return 64 * 2.0**-23 * float((ww[rows[r]][:, None] * (qa @ np.abs(kk).T)).max()) * 4

    check_near_ties(got, ref, scores, tol)


@pytest.mark.parametrize("d,lo,hi", [(32, -8, 8), (64, -8, 8), (128, -4, 4), (256, -4, 4)])
def test_flat_mfma_head_dims_exact(d, lo, hi):
    # Every bf16 MFMA flat-score head size, bit-exact on an integer grid whose
    # weighted sums stay below 2^24 units of 2^-8 (16 heads * d * hi^2 * 255):
    # ragged query count, key count off the 64-key tile, mixed visibility.
    N, nq = 3001, 37
    q_i = synth.int_grid((2, nq, 16, d), 61 + d, lo, hi, dtype=torch.bfloat16)
    k_i = synth.int_grid((2, N, d), 62 + d, lo, hi, dtype=torch.bfloat16)
    w_i = synth.dyadic_uniform((2, nq, 16), 63 + d)
    nv = synth.int_grid((2, nq), 64 + d, 0, N, dtype=torch.int32)
    nv[0, :3] = torch.tensor([0, 1, N], dtype=torch.int32)
    for k in (1, 100, 700, 4000):
        idx = ops.index_topk(q_i.to(DEV), k_i.to(DEV), w_i.to(DEV), nv.to(DEV), k).cpu().numpy()
        for b in range(2):
            ref = oracle.flat_topk(f64(q_i[b]), f64(k_i[b]), f64(w_i[b]), nv[b].numpy(), k)
            assert np.array_equal(idx[b], ref), (d, b, k)


def test_long_row_selection_boundaries_exact():
    # A flat launch with n above the LDS-resident limit: rows whose visible
    # counts straddle the in-register limit (8192), the LDS limit (16384) and
    # the full row take every selection path; bit-exact on the integer grid.
    d, N, nq = 64, 40000, 12
    q_i = synth.int_grid((1, nq, 16, d), 71, -8, 8, dtype=torch.bfloat16)
    k_i = synth.int_grid((1, N, d), 72, -8, 8, dtype=torch.bfloat16)
    w_i = synth.dyadic_uniform((1, nq, 16), 73)
    nv = torch.tensor([[0, 1, 5000, 8192, 8193, 12000, 16384, 16385, 20000, 33333, 39999, 40000]], dtype=torch.int32)
    for k in (64, 2048):
        idx = ops.index_topk(q_i.to(DEV), k_i.to(DEV), w_i.to(DEV), nv.to(DEV), k).cpu().numpy()
        ref = oracle.flat_topk(f64(q_i[0]), f64(k_i[0]), f64(w_i[0]), nv[0].numpy(), k)
        assert np.array_equal(idx[0], ref), k


def test_edge_cases():
    d, N, nq = 64, 300, 20
    q_i = synth.int_grid((2, nq, 16, d), 51, -8, 8, dtype=torch.bfloat16)
    k_i = synth.int_grid((2, N, d), 52, -8, 8, dtype=torch.bfloat16)
    w_i = synth.dyadic_uniform((2, nq, 16), 53)
    nv = torch.tensor([[0, 1, 2, 5, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 255, 256, 299, 300, 300]] * 2,
                      dtype=torch.int32)
    nv[1] = nv[1].flip(0)
    for k in (1, 7, 64, 299, 300, 512):
        idx = ops.index_topk(q_i.to(DEV), k_i.to(DEV), w_i.to(DEV), nv.to(DEV), k).cpu().numpy()
        for b in range(2):
            ref = oracle.flat_topk(f64(q_i[b]), f64(k_i[b]), f64(w_i[b]), nv[b].numpy(), k)
            assert np.array_equal(idx[b], ref), (b, k)
    # an all-zero query: every visible score is 0, the lowest indices win
    qz = torch.zeros_like(q_i)
    idx = ops.index_topk(qz.to(DEV), k_i.to(DEV), w_i.to(DEV), nv.to(DEV), 10).cpu().numpy()
    assert list(idx[0, 19]) == list(range(10)) and list(idx[0, 0]) == [-1] * 10


# ---- HISA -------------------------------------------------------------------

@pytest.mark.parametrize("B,m", [(16, 1), (16, 2), (16, 8), (128, 1), (128, 2), (128, 8)])
def test_tiny_layer_fp32_hisa_exact(B, m):
    t = synth.tiny_hybrid_layer(0).tensors
    N = 1023
    nv = ops.visible_count(t["q_pos"].to(DEV), 8, 4, N)
    k_i = t["k_i"].to(DEV)
    reps = ops.hisa_pool(k_i, B)
    idx, blk = ops.hisa_topk(t["q_i"].to(DEV), k_i, t["w_i"].to(DEV), nv, reps, B, m, 64, return_blocks=True)
    torch.cuda.synchronize()
    ref, ref_blk = oracle.hisa_topk(f64(t["q_i"][0]), f64(t["k_i"][0]), f64(t["w_i"][0]), nv.cpu().numpy()[0], B, m, 64)
    assert np.array_equal(blk.cpu().numpy()[0], ref_blk)
    assert np.array_equal(idx.cpu().numpy()[0], ref)


def _stage1_exact_bound(q, k_i, w, B, weight_bits):
    # With block sums S_b (integers), representatives S_b / B (B a power of 2)
    # and head weights v / 2^bits, every partial sum of a stage-1 score is a
    # multiple of 2^-(log2 B + bits); it is exact in fp32 when
    #     max_v * sum_h sum_c |q_hc S_bc| < 2^24      (asserted here).
    nb = -(-k_i.shape[0] // B)
    S = np.stack([k_i[j * B:(j + 1) * B].sum(0) for j in range(nb)])
    worst = (np.abs(q).reshape(-1, q.shape[-1]) @ np.abs(S).T).reshape(q.shape[0], q.shape[1], nb).sum(1).max()
    assert worst * ((1 << weight_bits) - 1) < 2**24, worst


def test_hisa_128k_bf16_integer_grid_exact_sampled():
    w = synth.indexer_128k(0, integer_grid=True, weight_bits=4)
    t = w.tensors
    N, nq, B, m, k = 131072, 1024, 128, 64, 2048
    nv = _nvis_entry_space(nq, N)
    k_i = t["k_i"].to(DEV)
    reps = ops.hisa_pool(k_i, B)
    idx, blk = ops.hisa_topk(t["q_i"].to(DEV), k_i, t["w_i"].to(DEV), nv, reps, B, m, k, return_blocks=True)
    torch.cuda.synchronize()
    rows = _rows(nq, 10)
    q, kk, ww = f64(t["q_i"][0]), f64(t["k_i"][0]), f64(t["w_i"][0])
    _stage1_exact_bound(q[rows], kk, ww, B, 4)
    ref, ref_blk = oracle.hisa_topk(q[rows], kk, ww[rows], nv.cpu().numpy()[0][rows], B, m, k)
    assert np.array_equal(blk.cpu().numpy()[0, rows], ref_blk)
    assert np.array_equal(idx.cpu().numpy()[0, rows], ref)


@pytest.mark.parametrize("N,B,m", [(4096, 128, 32), (1000, 64, 16), (8191, 128, 64)])
def test_hisa_keeping_every_block_equals_flat(N, B, m):
    nq, k = 64, 256
    q_i = synth.normal((1, nq, 16, 128), 61, dtype=torch.bfloat16).to(DEV)
    k_i = synth.normal((1, N, 128), 62, dtype=torch.bfloat16).to(DEV)
    w_i = synth.uniform((1, nq, 16), 63).to(DEV)
    nv = _nvis_entry_space(nq, N)
    reps = ops.hisa_pool(k_i, B)
    a = ops.hisa_topk(q_i, k_i, w_i, nv, reps, B, m, k)
    f = ops.index_topk(q_i, k_i, w_i, nv, k)
    torch.cuda.synchronize()
    assert torch.equal(a, f)


def test_hisa_float_inputs_vs_oracle():
    # N(0,1) indexer at the 128K chunk with needles: IoU of GPU HISA vs oracle
    # HISA on sampled rows (the selection itself is a heuristic, so it is the
    # oracle's HISA, not flat, that the GPU must match).
    w = synth.indexer_128k(0)
    t = w.tensors
    N, nq, B, m, k = 131072, 1024, 128, 64, 2048
    nv = _nvis_entry_space(nq, N)
    k_i = t["k_i"].to(DEV)
    reps = ops.hisa_pool(k_i, B)
    idx = ops.hisa_topk(t["q_i"].to(DEV), k_i, t["w_i"].to(DEV), nv, reps, B, m, k)
    torch.cuda.synchronize()
    rows = _rows(nq, 8)
    ref, _ = oracle.hisa_topk(f64(t["q_i"][0, rows]), f64(t["k_i"][0]), f64(t["w_i"][0, rows]),
                              nv.cpu().numpy()[0][rows], B, m, k)
    mean, mn = iou_rows(idx.cpu().numpy()[0, rows], ref)
    assert mean >= 0.999, (mean, mn)


@pytest.mark.parametrize("N,B,m,k", [(20000, 128, 64, 2048), (262143, 128, 64, 512), (5000, 64, 8, 300),
                                     (524287, 128, 16, 512),  # CSA2's rate-2 cache at 1M, 4,096 blocks
                                     (20000, 8, 1100, 2048),  # more chosen blocks than LDS slots
                                     (20000, 2, 64, 100)])  # over 8,192 blocks a row: the 1,024-thread block select
def test_hisa_decode_shape_exact(N, B, m, k):
    # One query per sequence (the decode launch shape), ragged last block,
    # integer grid with 4-bit weights (stage-1 scores exact, bound asserted).
    bt = 3
    q_i = synth.int_grid((bt, 1, 16, 128), 201, -4, 4, dtype=torch.bfloat16)
    k_i = synth.int_grid((bt, N, 128), 202, -4, 4, dtype=torch.bfloat16)
    w_i = synth.dyadic_uniform((bt, 1, 16), 203, bits=4)
    nv = torch.tensor([[N], [N - 77], [B * 3 + 5]], dtype=torch.int32)
    kd = k_i.to(DEV)
    reps = ops.hisa_pool(kd, B)
    idx, blk = ops.hisa_topk(q_i.to(DEV), kd, w_i.to(DEV), nv.to(DEV), reps, B, m, k, return_blocks=True)
    torch.cuda.synchronize()
    for b in range(bt):
        q, kk, ww = f64(q_i[b]), f64(k_i[b]), f64(w_i[b])
        _stage1_exact_bound(q, kk, ww, B, 4)
        ref, ref_blk = oracle.hisa_topk(q, kk, ww, nv[b].numpy(), B, m, k)
        assert np.array_equal(blk.cpu().numpy()[b], ref_blk), b
        assert np.array_equal(idx.cpu().numpy()[b], ref), b


@pytest.mark.parametrize("d,B", [(64, 64), (128, 128), (32, 128)])
def test_hisa_block_major_stage2_exact(d, B):
    # Many queries per sequence (the block-major stage-2 path: each chosen
    # block scored once for all its choosers), two sequences, ragged key
    # count, mixed visibility; integer grid, 4-bit weights, bound asserted.
    bt, nq, N, m, k = 2, 200, 5001, 8, 300
    q_i = synth.int_grid((bt, nq, 16, d), 221 + d, -4, 4, dtype=torch.bfloat16)
    k_i = synth.int_grid((bt, N, d), 222 + d, -4, 4, dtype=torch.bfloat16)
    w_i = synth.dyadic_uniform((bt, nq, 16), 223 + d, bits=4)
    nv = synth.int_grid((bt, nq), 224 + d, 1, N, dtype=torch.int32)
    nv[0, :4] = torch.tensor([1, B, B + 1, N], dtype=torch.int32)
    kd = k_i.to(DEV)
    reps = ops.hisa_pool(kd, B)
    idx, blk = ops.hisa_topk(q_i.to(DEV), kd, w_i.to(DEV), nv.to(DEV), reps, B, m, k, return_blocks=True)
    torch.cuda.synchronize()
    for b in range(bt):
        q, kk, ww = f64(q_i[b]), f64(k_i[b]), f64(w_i[b])
        _stage1_exact_bound(q, kk, ww, B, 4)
        ref, ref_blk = oracle.hisa_topk(q, kk, ww, nv[b].numpy(), B, m, k)
        assert np.array_equal(blk.cpu().numpy()[b], ref_blk), b
        assert np.array_equal(idx.cpu().numpy()[b], ref), b


def test_long_rows_ties_take_the_fallback_path():
    # All-zero queries: every visible score is exactly 0, so the sampled
    # threshold can never isolate k candidates; the exact segment + merge
    # kernels must finish those rows (lowest indices win the ties).  Row 1 is
    # ordinary float data on the fast path, row 2 a short row.
    N, k = 40000, 1000
    q_i = synth.normal((1, 3, 16, 128), 211, dtype=torch.bfloat16)
    q_i[0, 0] = 0
    k_i = synth.normal((1, N, 128), 212, dtype=torch.bfloat16)
    w_i = synth.uniform((1, 3, 16), 213)
    nv = torch.tensor([[N, N - 5, 9000]], dtype=torch.int32)
    idx, sc = ops.index_topk(q_i.to(DEV), k_i.to(DEV), w_i.to(DEV), nv.to(DEV), k, return_scores=True)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()[0]
    assert list(got[0]) == list(range(k))
    assert float(sc[0, 0].abs().max()) == 0.0
    ref = oracle.flat_topk(f64(q_i[0, 1:]), f64(k_i[0]), f64(w_i[0, 1:]), nv[0, 1:].numpy(), k)
    mean, mn = iou_rows(got[1:], ref)
    assert mean >= 0.999, (mean, mn)


def _top_rows_case(seed, N, nq, top_rows):
    # Non-negative queries; ordinary keys on [-4, 4], the listed rows all +4:
    # those keys share the largest score of every query (ties everywhere).
    d = 128
    q_i = synth.int_grid((1, nq, 16, d), seed, 0, 4, dtype=torch.bfloat16)
    k_i = synth.int_grid((1, N, d), seed + 1, -4, 4, dtype=torch.bfloat16)
    k_i[0, top_rows] = 4
    w_i = synth.dyadic_uniform((1, nq, 16), seed + 2)
    return q_i, k_i, w_i


def _flat_exact(q_i, k_i, w_i, nv, k, rows):
    idx, sc = ops.index_topk(q_i.to(DEV), k_i.to(DEV), w_i.to(DEV), nv.to(DEV), k, return_scores=True)
    torch.cuda.synchronize()
    ref, ref_sc = oracle.flat_topk(f64(q_i[0, rows]), f64(k_i[0]), f64(w_i[0, rows]), nv[0, rows].numpy(), k,
                                   return_scores=True)
    got = idx.cpu().numpy()[0, rows]
    assert np.array_equal(got, ref)
    got_sc = f64(sc[0, rows])
    assert np.array_equal(np.where(ref >= 0, got_sc, 0), np.where(ref >= 0, ref_sc, 0))


def test_fused_flat_threshold_too_high_falls_back():
    # Long rows take the fused path: a threshold from an evenly spread sample
    # of 64-key tiles (every 17th tile at N = 70,000), then only scores above
    # it are kept.  Here the first 8 keys of every sampled tile tie for the
    # top score, so the sample puts the threshold at that score although only
    # 512 keys reach it, fewer than k: the rows must take the full path.
    N, nq, k = 70000, 16, 700
    ntiles = (N + 63) // 64
    ts = ntiles // 64
    top = [t * 64 * ts + j for t in range((ntiles + ts - 1) // ts) for j in range(8) if t * 64 * ts + j < N]
    q_i, k_i, w_i = _top_rows_case(221, N, nq, top)
    nv = torch.tensor([[N] * 8 + [N - 1000 * i for i in range(1, 9)]], dtype=torch.int32)
    _flat_exact(q_i, k_i, w_i, nv, k, list(range(nq)))


def test_fused_flat_chunk_overflow_falls_back():
    # 2,000 consecutive keys tie for the top score: more candidates than a key
    # chunk's span holds, so those rows take the full path; rows that do not
    # see the cluster stay on the fused path.
    N, nq, k = 70000, 16, 2048
    q_i, k_i, w_i = _top_rows_case(231, N, nq, list(range(20000, 22000)))
    nv = torch.tensor([[N] * 6 + [21000, 20500, 20001, 19999, 19000, 50000, 60000, 65536, 69999, 100]],
                      dtype=torch.int32)
    _flat_exact(q_i, k_i, w_i, nv, k, list(range(nq)))


def test_fused_flat_float_inputs_vs_oracle():
    # Float inputs on the fused path (sample, threshold, candidates) at
    # N = 50,000: agreement with the fp64 oracle up to near ties.
    N, nq, k = 50000, 24, 2048
    q_i = synth.normal((1, nq, 16, 128), 241, dtype=torch.bfloat16)
    k_i = synth.normal((1, N, 128), 242, dtype=torch.bfloat16)
    w_i = synth.uniform((1, nq, 16), 243)
    nv = torch.tensor([[N - 7 * i for i in range(nq)]], dtype=torch.int32)
    nv[0, 5] = 3000   # between k and 2k: every key is a candidate
    nv[0, 6] = 2048   # exactly k
    idx = ops.index_topk(q_i.to(DEV), k_i.to(DEV), w_i.to(DEV), nv.to(DEV), k)
    torch.cuda.synchronize()
    q, kk, ww = f64(q_i[0]), f64(k_i[0]), f64(w_i[0])
    nvh = nv[0].numpy()
    ref = oracle.flat_topk(q, kk, ww, nvh, k)
    got = idx.cpu().numpy()[0]
    mean, mn = iou_rows(got, ref)
    assert mean >= 0.999, (mean, mn)

    def scores(r):
        return oracle.index_scores(q[r], kk[: nvh[r]], ww[r])

    def tol(r):  # fp32 accumulation bound, as in the 8K test
        qa = np.abs(q[r])
        return 128 * 2.0**-23 * float((ww[r][:, None] * (qa @ np.abs(kk).T)).max()) * 4

    check_near_ties(got, ref, scores, tol)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d_i", [16, 48, 80, 256])
def test_hisa_indexer_widths_exact(dtype, d_i):
    # Block scores on MFMA exist for d_i in {16, 32, 64, 128, 256}; other
    # widths (48, 80) must take the vector kernel.  Several queries per
    # sequence and one query per sequence, ragged key count, mixed
    # visibility; integer grid with 4-bit weights (bound asserted).
    N, B, m, k = 3001, 64, 6, 200
    for bt, nq in ((2, 40), (3, 1)):
        q_i = synth.int_grid((bt, nq, 16, d_i), 401 + d_i, -4, 4, dtype=dtype)
        k_i = synth.int_grid((bt, N, d_i), 402 + d_i, -4, 4, dtype=dtype)
        w_i = synth.dyadic_uniform((bt, nq, 16), 403 + d_i, bits=4)
        nv = synth.int_grid((bt, nq), 404 + d_i, 1, N, dtype=torch.int32)
        nv[0, 0] = N
        kd = k_i.to(DEV)
        reps = ops.hisa_pool(kd, B)
        idx, blk = ops.hisa_topk(q_i.to(DEV), kd, w_i.to(DEV), nv.to(DEV), reps, B, m, k, return_blocks=True)
        torch.cuda.synchronize()
        for b in range(bt):
            q, kk, ww = f64(q_i[b]), f64(k_i[b]), f64(w_i[b])
            _stage1_exact_bound(q, kk, ww, B, 4)
            ref, ref_blk = oracle.hisa_topk(q, kk, ww, nv[b].numpy(), B, m, k)
            assert np.array_equal(blk.cpu().numpy()[b], ref_blk), (d_i, bt, b)
            assert np.array_equal(idx.cpu().numpy()[b], ref), (d_i, bt, b)


@pytest.mark.parametrize("dtype,d_i", [(torch.bfloat16, 64), (torch.bfloat16, 128), (torch.float32, 64),
                                       (torch.bfloat16, 48)])
def test_block_sparse_exact(dtype, d_i):
    # Block-sparse baseline: HISA's block choice, then every visible entry of
    # the chosen blocks.  Many queries and one query per sequence, ragged
    # key count, mixed visibility (partly visible last blocks, fewer
    # candidate blocks than m); integer grid, 4-bit weights (bound asserted).
    N, B, m = 3001, 64, 6
    for bt, nq in ((2, 40), (3, 1)):
        q_i = synth.int_grid((bt, nq, 16, d_i), 501 + d_i, -4, 4, dtype=dtype)
        k_i = synth.int_grid((bt, N, d_i), 502 + d_i, -4, 4, dtype=dtype)
        w_i = synth.dyadic_uniform((bt, nq, 16), 503 + d_i, bits=4)
        nv = synth.int_grid((bt, nq), 504 + d_i, 0, N, dtype=torch.int32)
        nv[0, 0] = N
        if nq > 1:
            nv[0, 1:4] = torch.tensor([1, B + 3, 3 * B], dtype=torch.int32)
        kd = k_i.to(DEV)
        reps = ops.hisa_pool(kd, B)
        idx, blk = ops.block_sparse_topk(q_i.to(DEV), kd, w_i.to(DEV), nv.to(DEV), reps, B, m, return_blocks=True)
        torch.cuda.synchronize()
        for b in range(bt):
            q, kk, ww = f64(q_i[b]), f64(k_i[b]), f64(w_i[b])
            _stage1_exact_bound(q, kk, ww, B, 4)
            ref, ref_blk = oracle.block_sparse_topk(q, kk, ww, nv[b].numpy(), B, m)
            assert np.array_equal(blk.cpu().numpy()[b], ref_blk), (d_i, bt, b)
            assert np.array_equal(idx.cpu().numpy()[b], ref), (d_i, bt, b)


def test_block_sparse_128k_exact_sampled_and_same_blocks_as_hisa():
    # The 128K chunk at the attention budget of HISA's k = 2,048: 16 blocks
    # of 128.  Exact against the oracle on sampled queries; the chosen blocks
    # are those of HISA's first stage with m = 16.
    w = synth.indexer_128k(0, integer_grid=True, weight_bits=4)
    t = w.tensors
    N, nq, B, m = 131072, 1024, 128, 16
    nv = _nvis_entry_space(nq, N)
    k_i = t["k_i"].to(DEV)
    reps = ops.hisa_pool(k_i, B)
    idx, blk = ops.block_sparse_topk(t["q_i"].to(DEV), k_i, t["w_i"].to(DEV), nv, reps, B, m, return_blocks=True)
    _, hblk = ops.hisa_topk(t["q_i"].to(DEV), k_i, t["w_i"].to(DEV), nv, reps, B, m, 2048, return_blocks=True)
    torch.cuda.synchronize()
    assert torch.equal(blk, hblk)
    rows = _rows(nq, 8)
    q, kk, ww = f64(t["q_i"][0]), f64(t["k_i"][0]), f64(t["w_i"][0])
    _stage1_exact_bound(q[rows], kk, ww, B, 4)
    ref, ref_blk = oracle.block_sparse_topk(q[rows], kk, ww[rows], nv.cpu().numpy()[0][rows], B, m)
    assert np.array_equal(blk.cpu().numpy()[0, rows], ref_blk)
    assert np.array_equal(idx.cpu().numpy()[0, rows], ref)


# ---- flat top-k with one query per sequence (decode) --------------------------

@pytest.mark.parametrize("d,lo,hi", [(32, -8, 8), (64, -8, 8), (128, -4, 4)])
@pytest.mark.parametrize("N", [3001, 70000])
def test_flat_decode_exact(d, lo, hi, N):
    # One query per sequence: the decode score kernel, on the plain path
    # (N = 3001) and the fused sample / threshold / candidate path
    # (N = 70,000), bit-exact on the integer grid; visible counts around k,
    # 2k, the 64-key tile and the full row.
    bt = 8
    q_i = synth.int_grid((bt, 1, 16, d), 301 + d, lo, hi, dtype=torch.bfloat16)
    k_i = synth.int_grid((bt, N, d), 302 + d, lo, hi, dtype=torch.bfloat16)
    w_i = synth.dyadic_uniform((bt, 1, 16), 303 + d)
    for k in (1, 100, 700, 2048):
        nvl = [N, N - 1, 0, 1, min(N, k), min(N, k + 37), min(N, 2 * k + 5), 64 * (N // 128) + 13]
        nv = torch.tensor(nvl, dtype=torch.int32).reshape(bt, 1)
        idx, sc = ops.index_topk(q_i.to(DEV), k_i.to(DEV), w_i.to(DEV), nv.to(DEV), k, return_scores=True)
        idx, sc = idx.cpu().numpy(), f64(sc)
        for b in range(bt):
            ref, ref_sc = oracle.flat_topk(f64(q_i[b]), f64(k_i[b]), f64(w_i[b]), nv[b].numpy(), k,
                                           return_scores=True)
            assert np.array_equal(idx[b], ref), (d, N, k, b)
            assert np.array_equal(np.where(ref >= 0, sc[b], 0), np.where(ref >= 0, ref_sc, 0)), (d, N, k, b)


def test_flat_decode_ties_take_the_fallback_path():
    # One query per sequence on the fused path: an all-zero query (every
    # score 0, the sample cannot isolate k candidates) must be finished by
    # the exact fallback; the other rows stay on the fast path.
    N, k, bt = 40000, 1000, 4
    q_i = synth.int_grid((bt, 1, 16, 128), 311, -4, 4, dtype=torch.bfloat16)
    q_i[2] = 0
    k_i = synth.int_grid((bt, N, 128), 312, -4, 4, dtype=torch.bfloat16)
    w_i = synth.dyadic_uniform((bt, 1, 16), 313, bits=4)
    nv = torch.tensor([[N], [N - 5], [N], [9000]], dtype=torch.int32)
    idx = ops.index_topk(q_i.to(DEV), k_i.to(DEV), w_i.to(DEV), nv.to(DEV), k).cpu().numpy()
    assert list(idx[2, 0]) == list(range(k))
    for b in (0, 1, 3):
        ref = oracle.flat_topk(f64(q_i[b]), f64(k_i[b]), f64(w_i[b]), nv[b].numpy(), k)
        assert np.array_equal(idx[b], ref), b


@pytest.mark.parametrize("N,B,m", [(16000, 128, 125), (5000, 64, 80)])
def test_flat_decode_equals_hisa_keeping_every_block_float(N, B, m):
    # At decode the flat score and HISA's second stage share their
    # arithmetic, so on float inputs HISA keeping every block returns the
    # flat selection bit for bit.
    bt, k = 6, 512
    q_i = synth.normal((bt, 1, 16, 128), 321, dtype=torch.bfloat16).to(DEV)
    k_i = synth.normal((bt, N, 128), 322, dtype=torch.bfloat16).to(DEV)
    w_i = synth.uniform((bt, 1, 16), 323).to(DEV)
    nv = torch.tensor([[N], [N - 3], [N // 2], [k], [k + 1], [B * 7 + 5]], dtype=torch.int32).to(DEV)
    reps = ops.hisa_pool(k_i, B)
    a = ops.hisa_topk(q_i, k_i, w_i, nv, reps, B, m, k)
    f = ops.index_topk(q_i, k_i, w_i, nv, k)
    torch.cuda.synchronize()
    assert torch.equal(a, f)


def test_flat_decode_csa2_size_exact_sampled():
    # The CSA2 decode selection at its full size: 8 sequences of 524,287
    # compressed entries (rate 2 at 1M), one query each, top-512, on the
    # integer grid with 4-bit weights (exact scores); two rows against the
    # oracle, every row's selection checked for validity.
    bt, N, k = 8, 524287, 512
    q_i = synth.int_grid((bt, 1, 16, 128), 331, -4, 4, dtype=torch.bfloat16, device=DEV)
    k_i = synth.int_grid((bt, N, 128), 332, -4, 4, dtype=torch.bfloat16, device=DEV)
    w_i = synth.dyadic_uniform((bt, 1, 16), 333, device=DEV, bits=4)
    nv = torch.full((bt, 1), N, dtype=torch.int32, device=DEV)
    nv[5, 0] = N - 1000
    idx = ops.index_topk(q_i, k_i, w_i, nv, k).cpu().numpy()
    for b in range(bt):
        row = idx[b, 0]
        assert (np.diff(row) > 0).all() and row[0] >= 0 and row[-1] < int(nv[b, 0])
    for b in (0, 5):
        ref = oracle.flat_topk(f64(q_i[b]), f64(k_i[b]), f64(w_i[b]), nv[b].cpu().numpy(), k)
        assert np.array_equal(idx[b], ref), b
