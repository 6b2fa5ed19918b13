"""Pins for the attention oracles (CPU)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(7)


def sdpa(q, keys, vals, mask=None):
    """Library attention in float64 on the CPU: q [H][d], keys/vals [U][d]."""
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, :, None, :]  # [1][H][1][d]
    kt = torch.from_numpy(np.ascontiguousarray(keys))[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(np.ascontiguousarray(vals))[None, None].expand(1, q.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o[0, :, 0, :].numpy()


def test_worked_example():
    e = json.load(open(os.path.join(GOLD, "worked_examples.json")))["attention"]
    o, lse = oracle.attend(np.array(e["q"]), np.array(e["keys"]), np.array(e["vals"]), e["scale"])
    np.testing.assert_allclose(o, np.array(e["o"]), rtol=1e-14)
    np.testing.assert_allclose(lse, np.array(e["lse"]), rtol=1e-14)


def _layer(L=700, d=16, H=4, nq=5, w=8, s=4):
    raw = rng.standard_normal((L, 2 * d))
    z = rng.standard_normal(L)
    b = 0.1 * rng.standard_normal(w)
    ckv = oracle.compress(raw, z, b, w, s)
    q = rng.standard_normal((nq, H, d))
    q_pos = np.sort(rng.choice(np.arange(w, L), nq, replace=False))
    n_vis = np.array([oracle.n_visible(int(p), w, s, ckv.shape[0]) for p in q_pos])
    return raw, ckv, q, q_pos, n_vis


def test_dense_matches_library_sdpa_on_gathered_keys():
    d = 16
    raw, ckv, q, q_pos, n_vis = _layer(d=d)
    W = 128
    out, lse = oracle.dense_compressed_attention(q, ckv, n_vis, raw, q_pos, W, 1 / np.sqrt(d))
    for i, p in enumerate(q_pos):
        lo = max(0, p - W + 1)
        keys = np.concatenate([ckv[: n_vis[i], :d], raw[lo : p + 1, :d]])
        vals = np.concatenate([ckv[: n_vis[i], d:], raw[lo : p + 1, d:]])
        np.testing.assert_allclose(out[i], sdpa(q[i], keys, vals), rtol=1e-12, atol=1e-12)
        logits = (q[i] @ keys.T) / np.sqrt(d)
        np.testing.assert_allclose(lse[i], np.log(np.exp(logits).sum(1)), rtol=1e-12)


def test_sparse_with_all_entries_equals_dense_and_matches_sdpa():
    d = 16
    raw, ckv, q, q_pos, n_vis = _layer(d=d)
    k = int(n_vis.max()) + 3
    idx = np.full((len(q_pos), k), -1)
    for i in range(len(q_pos)):
        idx[i, : n_vis[i]] = np.arange(n_vis[i])
    sc = 1 / np.sqrt(d)
    o1, l1 = oracle.sparse_attention(q, ckv, idx, raw, q_pos, 128, sc)
    o2, l2 = oracle.dense_compressed_attention(q, ckv, n_vis, raw, q_pos, 128, sc)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)
    # a random subset: compare with the library over the explicit list
    sub = np.full((len(q_pos), 6), -1)
    for i in range(len(q_pos)):
        pick = np.sort(rng.choice(n_vis[i], min(5, n_vis[i]), replace=False))
        sub[i, : pick.size] = pick
    o3, _ = oracle.sparse_attention(q, ckv, sub, raw, q_pos, 16, sc)
    for i, p in enumerate(q_pos):
        ent = sub[i][sub[i] >= 0]
        rows = np.arange(max(0, p - 15), p + 1)
        keys = np.concatenate([ckv[ent, :d], raw[rows, :d]])
        vals = np.concatenate([ckv[ent, d:], raw[rows, d:]])
        np.testing.assert_allclose(o3[i], sdpa(q[i], keys, vals), rtol=1e-12, atol=1e-12)


def test_hca_is_dense_over_L_over_128_entries():
    d, L = 8, 1024
    raw = rng.standard_normal((L, 2 * d))
    ckv = oracle.compress(raw, rng.standard_normal(L), 0.1 * rng.standard_normal(128), 128, 128)
    assert ckv.shape[0] == L // 128
    q = rng.standard_normal((1, 2, d))
    p = L - 1
    out, _ = oracle.dense_compressed_attention(q, ckv, np.array([L // 128]), raw, np.array([p]), 128, 1 / np.sqrt(d))
    keys = np.concatenate([ckv[:, :d], raw[p - 127 : p + 1, :d]])
    vals = np.concatenate([ckv[:, d:], raw[p - 127 : p + 1, d:]])
    np.testing.assert_allclose(out[0], sdpa(q[0], keys, vals), rtol=1e-12, atol=1e-12)


def test_no_compressed_entries_is_sliding_window_attention():
    d, L, W = 8, 300, 128
    raw = rng.standard_normal((L, 2 * d))
    q_pos = np.array([0, 5, 127, 128, 299])
    q = rng.standard_normal((len(q_pos), 3, d))
    out, _ = oracle.sparse_attention(q, np.zeros((0, 2 * d)), np.full((len(q_pos), 4), -1), raw, q_pos, W,
                                     1 / np.sqrt(d))
    # textbook banded attention over the raw sequence
    qq = torch.zeros(1, 3, L, d, dtype=torch.float64)
    for i, p in enumerate(q_pos):
        qq[0, :, p] = torch.from_numpy(q[i])
    kk = torch.from_numpy(raw[:, :d])[None, None].expand(1, 3, L, d)
    vv = torch.from_numpy(raw[:, d:])[None, None].expand(1, 3, L, d)
    i = torch.arange(L)[:, None]
    j = torch.arange(L)[None, :]
    band = (j <= i) & (j > i - W)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=band)
    for n, p in enumerate(q_pos):
        np.testing.assert_allclose(out[n], ref[0, :, p].numpy(), rtol=1e-12, atol=1e-12)


def test_single_key_returns_its_value():
    d = 4
    raw = rng.standard_normal((1, 2 * d))
    q = rng.standard_normal((1, 5, d))
    out, lse = oracle.dense_compressed_attention(q, np.zeros((0, 2 * d)), np.array([0]), raw, np.array([0]), 128, 0.5)
    np.testing.assert_allclose(out[0], np.tile(raw[0, d:], (5, 1)), rtol=1e-15)
    np.testing.assert_allclose(lse[0], 0.5 * q[0] @ raw[0, :d], rtol=1e-14)


def test_lse_merge_identity():
    d, H = 8, 3
    q = rng.standard_normal((H, d))
    keys = rng.standard_normal((50, d))
    vals = rng.standard_normal((50, d))
    o, l = oracle.attend(q, keys, vals, 0.3)
    parts = [(0, 7), (7, 8), (8, 31), (31, 50)]
    os_, ls_ = zip(*[oracle.attend(q, keys[a:b], vals[a:b], 0.3) for a, b in parts])
    om, lm = oracle.lse_merge(os_, ls_)
    np.testing.assert_allclose(om, o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lm, l, rtol=1e-13, atol=1e-13)


def test_causality_future_tokens_do_not_matter():
    # Perturbing every raw token after p leaves query p's compressed entries,
    # indexer selection and both attention outputs bit-identical.
    d, L, w, s = 8, 400, 8, 4
    raw = rng.standard_normal((L, 2 * d))
    z = rng.standard_normal(L)
    b = 0.1 * rng.standard_normal(w)
    k_i = rng.integers(-8, 9, (oracle.n_entries(L, w, s), 4)).astype(float)
    q_i = rng.integers(-8, 9, (1, 2, 4)).astype(float)
    w_i = np.array([[0.5, 0.25]])
    q = rng.standard_normal((1, 2, d))
    for p in (7, 100, 203, 398):
        raw2, z2 = raw.copy(), z.copy()
        raw2[p + 1 :] += 10 * rng.standard_normal((L - p - 1, 2 * d))
        z2[p + 1 :] -= 3.0
        outs = []
        for rr, zz in ((raw, z), (raw2, z2)):
            ckv = oracle.compress(rr, zz, b, w, s)
            nv = oracle.n_visible(p, w, s, ckv.shape[0])
            idx = oracle.flat_topk(q_i, k_i, w_i, np.array([nv]), 6)
            o_s, _ = oracle.sparse_attention(q, ckv, idx, rr, np.array([p]), 128, 0.3)
            o_d, _ = oracle.dense_compressed_attention(q, ckv, np.array([nv]), rr, np.array([p]), 128, 0.3)
            outs.append((ckv[:nv], idx, o_s, o_d))
        for a, bb in zip(*outs):
            np.testing.assert_array_equal(a, bb)


# ---- CSA2: one compression level, a selection shared by a group of layers ---

def _csa2_inputs(L=300, d=8, H=3, G=2, nq=4, DI=4, HI=2):
    raw = rng.standard_normal((L, 2 * d))
    raw_ki = rng.integers(-3, 4, (L, DI)).astype(float)
    z = rng.standard_normal(L)
    q = rng.standard_normal((G, nq, H, d))
    q_i = rng.integers(-3, 4, (nq, HI, DI)).astype(float)
    w_i = rng.integers(0, 4, (nq, HI)).astype(float) / 4
    q_pos = np.sort(rng.choice(np.arange(8, L), nq, replace=False))
    return raw, raw_ki, z, q, q_i, w_i, q_pos


@pytest.mark.parametrize("w,s", [(4, 2), (1, 1)])
def test_csa2_keeping_every_entry_is_library_attention(w, s):
    # k at least the visible count: each layer attends to every visible
    # entry (compressed from its raw rows here with explicit window slices)
    # plus the window, in one library softmax
    d, W = 8, 16
    raw, raw_ki, z, q, q_i, w_i, q_pos = _csa2_inputs(d=d)
    b = 0.1 * rng.standard_normal(w)
    out, lse, idx = oracle.csa2_layer_group(q, raw, raw_ki, z, b, q_i, w_i, q_pos, 400, W, w, s, 1 / np.sqrt(d))
    for j, p in enumerate(q_pos):
        nv = (p - w + 1) // s + 1
        assert list(idx[j][:nv]) == list(range(nv)) and (idx[j][nv:] == -1).all()
        ents = []
        for i in range(nv):
            a = z[i * s:i * s + w] + b
            al = np.exp(a - a.max())
            al /= al.sum()
            ents.append(al @ raw[i * s:i * s + w])
        ents = np.array(ents)
        lo = max(0, p - W + 1)
        keys = np.concatenate([ents[:, :d], raw[lo:p + 1, :d]])
        vals = np.concatenate([ents[:, d:], raw[lo:p + 1, d:]])
        for g in range(q.shape[0]):
            # torch's SDPA scales by 1/sqrt(d), the scale passed above
            np.testing.assert_allclose(out[g, j], sdpa(q[g, j], keys, vals), rtol=1e-10, atol=1e-12)


def test_csa2_uncompressed_cache_is_the_raw_rows():
    raw, raw_ki, z, q, q_i, w_i, q_pos = _csa2_inputs()
    ckv, k_i = oracle.compress_with_index(raw, raw_ki, z, None, 1, 1)
    np.testing.assert_array_equal(ckv, raw)
    np.testing.assert_array_equal(k_i, raw_ki)


def test_csa2_layers_fold_into_heads():
    # MQA: every head attends to the same keys, so a group's layers sharing
    # one cache and one selection are one attention with G*H heads (the
    # layout the GPU uses: head g*H + h is head h of layer g)
    d = 8
    raw, raw_ki, z, q, q_i, w_i, q_pos = _csa2_inputs(d=d)
    G, nq, H, _ = q.shape
    b = 0.1 * rng.standard_normal(4)
    out, lse, idx = oracle.csa2_layer_group(q, raw, raw_ki, z, b, q_i, w_i, q_pos, 20, 16, 4, 2, 1 / np.sqrt(d))
    ckv, _ = oracle.compress_with_index(raw, raw_ki, z, b, 4, 2)
    folded = q.transpose(1, 0, 2, 3).reshape(nq, G * H, d)
    of, lf = oracle.sparse_attention(folded, ckv, idx, raw, q_pos, 16, 1 / np.sqrt(d))
    np.testing.assert_allclose(of.reshape(nq, G, H, d).transpose(1, 0, 2, 3), out, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lf.reshape(nq, G, H).transpose(1, 0, 2), lse, rtol=1e-13, atol=1e-14)
    # the layers really share a sparse set: some query sees more entries
    # than it selects
    nvis = (q_pos - 4 + 1) // 2 + 1
    assert (nvis > 20).any() and ((idx >= 0).sum(axis=1) == np.minimum(nvis, 20)).all()
