"""GPU parity: compression, visibility and HISA pooling against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from compressed_attention_amd import ops, synth
from helpers import assert_bf16_close, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _compress_case(x, z, b, w, s, e0=0, e1=None):
    y = ops.compress(x.to(DEV), z.to(DEV) if z is not None else None, b.to(DEV) if b is not None else None, w, s,
                     e0, e1)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("branch", ["csa", "hca"])
def test_tiny_layer_fp32(branch):
    t = synth.tiny_hybrid_layer(0).tensors
    w, s, bias = (8, 4, t["b_csa"]) if branch == "csa" else (128, 128, t["b_hca"])
    y = _compress_case(t["raw_kv"], t["z"], bias, w, s)
    ref = oracle.compress(f64(t["raw_kv"][0]), f64(t["z"][0]), f64(bias), w, s)
    assert y.shape[1] == ref.shape[0] == (1023 if branch == "csa" else 32)
    np.testing.assert_allclose(f64(y[0]), ref, rtol=2e-5, atol=2e-5)


def test_prefill_csa_bf16():
    t = synth.csa_prefill_chunk(0).tensors
    y = _compress_case(t["raw_kv"], t["z"], t["b"], 8, 4)
    ref = oracle.compress(f64(t["raw_kv"][0]), f64(t["z"][0]), f64(t["b"]), 8, 4)
    assert y.shape == (1, 8191, 256)
    assert_bf16_close(f64(y[0]), ref)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("w,s,L", [(8, 4, 1001), (128, 128, 1000), (5, 3, 77), (1, 1, 33), (16, 16, 16), (12, 4, 259)])
def test_ragged_and_generic_windows(dtype, w, s, L):
    C = 64
    bt = 3
    x = synth.normal((bt, L, C), seed=11 + w, dtype=dtype)
    z = synth.normal((bt, L), seed=12 + w)
    b = synth.normal((w,), seed=13 + w, std=0.1)
    y = _compress_case(x, z, b, w, s)
    for i in range(bt):
        ref = oracle.compress(f64(x[i]), f64(z[i]), f64(b), w, s)
        if dtype == torch.float32:
            np.testing.assert_allclose(f64(y[i]), ref, rtol=2e-5, atol=2e-5)
        else:
            assert_bf16_close(f64(y[i]), ref)


def test_no_logits_no_bias_is_mean():
    x = synth.normal((2, 1024, 32), seed=5)
    y = _compress_case(x, None, None, 128, 128)
    ref = f64(x).reshape(2, 8, 128, 32).mean(axis=2)
    np.testing.assert_allclose(f64(y), ref, rtol=1e-5, atol=1e-6)


def test_entry_range_rewrites_only_that_range():
    x = synth.normal((2, 600, 64), seed=7, dtype=torch.bfloat16).to(DEV)
    z = synth.normal((2, 600), seed=8).to(DEV)
    b = synth.normal((8,), seed=9, std=0.1).to(DEV)
    full = ops.compress(x, z, b, 8, 4)
    part = torch.full_like(full, 7.0)
    ops.compress(x, z, b, 8, 4, 100, 140, out=part)
    torch.cuda.synchronize()
    assert torch.equal(part[:, 100:140], full[:, 100:140])
    assert bool((part[:, :100] == 7.0).all()) and bool((part[:, 140:] == 7.0).all())


@pytest.mark.parametrize("branch", ["csa", "hca"])
def test_one_million_tokens_sampled(branch):
    # Full-length sequences (device-generated inputs); entries sampled for the oracle.
    L, bt = 1 << 20, 2
    w, s = (8, 4) if branch == "csa" else (128, 128)
    x = synth.normal((bt, L, 256), seed=21, dtype=torch.bfloat16, device=DEV)
    z = synth.normal((bt, L), seed=22, device=DEV)
    b = synth.normal((w,), seed=23, std=0.1).to(DEV)
    y = ops.compress(x, z, b, w, s)
    torch.cuda.synchronize()
    N = y.shape[1]
    assert N == oracle.n_entries(L, w, s)
    rng = np.random.default_rng(0)
    for bi in range(bt):
        for e in sorted(set(rng.integers(0, N, 24).tolist()) | {0, N - 1}):
            lo, hi = e * s, e * s + w
            ref = oracle.compress(f64(x[bi, lo:hi]), f64(z[bi, lo:hi]), f64(b), w, s)
            assert_bf16_close(f64(y[bi, e]), ref[0])


def test_visible_count_matches_definition():
    for w, s, N in [(8, 4, 1023), (128, 128, 32), (1, 1, 131072), (8, 4, 262143), (5, 3, 50)]:
        pos = torch.tensor(list(range(0, 400)) + [N * s + w - 2, N * s + w + 5, 2**20 - 1], dtype=torch.int32)
        got = ops.visible_count(pos.to(DEV), w, s, N).cpu().numpy()
        for p, g in zip(pos.tolist(), got.tolist()):
            if p < 3000:
                assert g == oracle.n_visible(p, w, s, N), (w, s, p)
            else:  # beyond a brute-force count: the definition at the far end
                assert g == min(N, (p - w + 1) // s + 1)


@pytest.mark.parametrize("dtype,B,n", [(torch.float32, 16, 1023), (torch.bfloat16, 128, 131072),
                                       (torch.bfloat16, 128, 262143), (torch.bfloat16, 64, 1000)])
def test_hisa_pool(dtype, B, n):
    k_i = synth.int_grid((2, n, 128), seed=31, lo=-4, hi=4, dtype=dtype)
    reps = ops.hisa_pool(k_i.to(DEV), B)
    torch.cuda.synchronize()
    for i in range(2):
        ref = oracle.hisa_pool(f64(k_i[i]), B)
        np.testing.assert_array_equal(f64(reps[i]), ref)  # sums of small integers / 2^k: exact
    # refreshing the last block alone reproduces it
    part = torch.zeros_like(reps)
    nb = reps.shape[1]
    ops.hisa_pool(k_i.to(DEV), B, nb - 1, nb, out=part)
    torch.cuda.synchronize()
    assert torch.equal(part[:, nb - 1], reps[:, nb - 1]) and bool((part[:, : nb - 1] == 0).all())


def _append_positions(L, w, s, N):
    """Decode positions covering: an entry completed at the start, in the
    middle and at the end; a position inside a window (no entry completed);
    one before the first window closes; one past the last entry."""
    return [w - 1, w - 1 + s * (N // 2), w - 1 + s * (N - 1), w - 1 + s * (N // 3) + (1 if s > 1 else 0),
            max(0, w - 3), w - 1 + s * N + (s - 1)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("w,s,L,C,pool", [(8, 4, 1001, 256, 16), (128, 128, 1000, 256, 0), (5, 3, 77, 64, 8),
                                          (1, 1, 300, 32, 128), (12, 4, 259, 512, 0)])
def test_decode_append(dtype, w, s, L, C, pool):
    """The fused per-token step against the oracle's compression, block mean
    and visible count: only the entry the token completes (and the block
    holding it) is written; everything else keeps its previous value."""
    N = (L - w) // s + 1
    pos = _append_positions(L, w, s, N)
    if s == 1:
        pos[3] = w - 1 + (N // 3)  # every position past w - 2 completes an entry
    bt = len(pos)
    x = synth.normal((bt, L, C), seed=41 + w, dtype=dtype)
    z = synth.normal((bt, L), seed=42 + w)
    b = synth.normal((w,), seed=43 + w, std=0.1)
    q_pos = torch.tensor(pos, dtype=torch.int32)
    ckv = torch.full((bt, N, C), 7.0, dtype=dtype, device=DEV)
    k_i = reps = None
    if pool:
        d_i = 128
        k_i = synth.int_grid((bt, N, d_i), seed=44, lo=-4, hi=4, dtype=dtype)
        reps = torch.full((bt, -(-N // pool), d_i), -3.0, dtype=torch.float32, device=DEV)
    nv = ops.decode_append(x.to(DEV), z.to(DEV), b.to(DEV), w, s, q_pos.to(DEV), ckv,
                           k_i.to(DEV) if pool else None, reps, pool or 1)
    torch.cuda.synchronize()
    nv = nv.cpu().numpy()
    ckv = f64(ckv)
    reps = f64(reps) if pool else None
    for i, p in enumerate(pos):
        assert nv[i] == oracle.n_visible(p, w, s, N), (i, p)
        done = p >= w - 1 and (p - w + 1) % s == 0 and (p - w + 1) // s < N
        e = (p - w + 1) // s if done else -1
        for row in range(N):
            if row != e:
                assert (ckv[i, row] == 7.0).all(), (i, row)
        if done:
            ref = oracle.compress(f64(x[i, e * s : e * s + w]), f64(z[i, e * s : e * s + w]), f64(b), w, s)[0]
            if dtype == torch.float32:
                np.testing.assert_allclose(ckv[i, e], ref, rtol=2e-5, atol=2e-5)
            else:
                assert_bf16_close(ckv[i, e], ref)
        if pool:
            ref_reps = oracle.hisa_pool(f64(k_i[i]), pool)
            for j in range(reps.shape[1]):
                if done and j == e // pool:
                    np.testing.assert_array_equal(reps[i, j], ref_reps[j])  # small integers / 2^k: exact
                else:
                    assert (reps[i, j] == -3.0).all(), (i, j)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("w,s,L", [(8, 4, 1001), (128, 128, 1000), (5, 3, 77)])
def test_compress_with_index(dtype, w, s, L):
    # K|V entries and their indexer keys from one pass with the entries'
    # own weights; each output against the oracle's compression of its raw
    # rows, and the K|V output equals hattn_compress's where the two share a
    # kernel and its per-thread arithmetic (the w = 2s and generic kernels).
    bt, C, Ci = 2, 256, 128
    x = synth.normal((bt, L, C), seed=31 + w, dtype=dtype)
    xi = synth.normal((bt, L, Ci), seed=32 + w, dtype=dtype)
    z = synth.normal((bt, L), seed=33 + w)
    b = synth.normal((w,), seed=34 + w, std=0.1)
    y, yi = ops.compress_with_index(x.to(DEV), xi.to(DEV), z.to(DEV), b.to(DEV), w, s)
    y_ref_gpu = ops.compress(x.to(DEV), z.to(DEV), b.to(DEV), w, s)
    torch.cuda.synchronize()
    for i in range(bt):
        r, ri = oracle.compress_with_index(f64(x[i]), f64(xi[i]), f64(z[i]), f64(b), w, s)
        for got, ref in ((y[i], r), (yi[i], ri)):
            if dtype == torch.float32:
                np.testing.assert_allclose(f64(got), ref, rtol=2e-5, atol=2e-5)
            else:
                assert_bf16_close(f64(got), ref)
    if w < 32:
        assert torch.equal(y, y_ref_gpu)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("w,s,L", [(8, 4, 1001), (128, 128, 1024), (5, 3, 77), (1, 1, 9)])
def test_compress_channel_logits(dtype, w, s, L):
    bt, C = 2, 64
    x = synth.normal((bt, L, C), seed=41 + w, dtype=dtype)
    Z = synth.normal((bt, L, C), seed=42 + w)
    b = synth.normal((w,), seed=43 + w, std=0.1)
    y = ops.compress_channel_logits(x.to(DEV), Z.to(DEV), b.to(DEV), w, s)
    # the same logit in every channel reproduces the per-token compression
    z1 = synth.normal((bt, L), seed=44 + w)
    y1 = ops.compress_channel_logits(x.to(DEV), z1[:, :, None].expand(bt, L, C).contiguous().to(DEV), b.to(DEV), w, s)
    torch.cuda.synchronize()
    for i in range(bt):
        ref = oracle.compress_channel_logits(f64(x[i]), f64(Z[i]), f64(b), w, s)
        ref1 = oracle.compress(f64(x[i]), f64(z1[i]), f64(b), w, s)
        for got, r in ((y[i], ref), (y1[i], ref1)):
            if dtype == torch.float32:
                np.testing.assert_allclose(f64(got), r, rtol=2e-5, atol=2e-5)
            else:
                assert_bf16_close(f64(got), r)


def test_compress_channel_logits_decode_entry_only():
    # a decode step rewrites just the entry the new token completes
    bt, L, C, w, s = 3, 2048, 256, 8, 4
    N = oracle.n_entries(L, w, s)
    x = synth.normal((bt, L, C), seed=51, dtype=torch.bfloat16)
    Z = synth.normal((bt, L, C), seed=52)
    y = torch.zeros((bt, N, C), dtype=torch.bfloat16, device=DEV)
    ops.compress_channel_logits(x.to(DEV), Z.to(DEV), None, w, s, N - 1, N, out=y)
    torch.cuda.synchronize()
    assert (y[:, : N - 1] == 0).all()
    for i in range(bt):
        ref = oracle.compress_channel_logits(f64(x[i, L - w:]), f64(Z[i, L - w:]), None, w, s)
        assert_bf16_close(f64(y[i, N - 1:]), ref)
