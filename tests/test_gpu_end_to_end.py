"""GPU parity of the whole tiny hybrid layer chain (fp32, seed 0):
compress -> visibility -> flat / HISA selection -> sparse attention (CSA)
and compress -> dense attention (HCA), against the same chain in the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from compressed_attention_amd import ops, synth
from helpers import f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_tiny_hybrid_layer_chain():
    w = synth.tiny_hybrid_layer(0)
    t, P = w.tensors, w.params
    g = {k: v.to(DEV) for k, v in t.items()}
    sc = 1 / math.sqrt(P["d"])
    # CSA branch
    ckv = ops.compress(g["raw_kv"], g["z"], g["b_csa"], 8, 4)
    nv = ops.visible_count(g["q_pos"], 8, 4, ckv.shape[1])
    idx = ops.index_topk(g["q_i"], g["k_i"], g["w_i"], nv, P["k"])
    o_csa = ops.sparse_attn(g["q"], ckv, idx, g["raw_kv"], g["q_pos"], P["window"])
    reps = ops.hisa_pool(g["k_i"], 128)
    idx_h = ops.hisa_topk(g["q_i"], g["k_i"], g["w_i"], nv, reps, 128, 2, P["k"])
    # HCA branch
    hkv = ops.compress(g["raw_kv"], g["z"], g["b_hca"], 128, 128)
    nvh = ops.visible_count(g["q_pos"], 128, 128, hkv.shape[1])
    o_hca = ops.dense_compressed_attn(g["q"], hkv, nvh, g["raw_kv"], g["q_pos"], P["window"])
    torch.cuda.synchronize()

    raw, z, pos = f64(t["raw_kv"][0]), f64(t["z"][0]), t["q_pos"][0].numpy()
    r_ckv = oracle.compress(raw, z, f64(t["b_csa"]), 8, 4)
    r_nv = np.array([oracle.n_visible(int(p), 8, 4, r_ckv.shape[0]) for p in pos])
    r_idx = oracle.flat_topk(f64(t["q_i"][0]), f64(t["k_i"][0]), f64(t["w_i"][0]), r_nv, P["k"])
    assert np.array_equal(idx.cpu().numpy()[0], r_idx)
    r_o, _ = oracle.sparse_attention(f64(t["q"][0]), r_ckv, r_idx, raw, pos, P["window"], sc)
    assert np.abs(f64(o_csa[0]) - r_o).max() < 1e-4
    r_idx_h, _ = oracle.hisa_topk(f64(t["q_i"][0]), f64(t["k_i"][0]), f64(t["w_i"][0]), r_nv, 128, 2, P["k"])
    assert np.array_equal(idx_h.cpu().numpy()[0], r_idx_h)
    r_hkv = oracle.compress(raw, z, f64(t["b_hca"]), 128, 128)
    r_nvh = np.array([oracle.n_visible(int(p), 128, 128, r_hkv.shape[0]) for p in pos])
    r_oh, _ = oracle.dense_compressed_attention(f64(t["q"][0]), r_hkv, r_nvh, raw, pos, P["window"], sc)
    assert np.abs(f64(o_hca[0]) - r_oh).max() < 1e-4


def test_decode_step_hybrid_pair_reduced():
    # The decode step that bench.py times, at 2 sequences of 65536 tokens:
    # compress the windows the last token completes, refresh the last HISA
    # block mean, HISA selection, sparse (CSA) and dense (HCA) attention.
    # Oracle: the same step on the host from the same inputs.
    bt, L = 2, 65536
    N = oracle.n_entries(L, 8, 4)
    Nh = oracle.n_entries(L, 128, 128)
    w = synth.hybrid_pair_decode(0, device="cpu", bt=bt, L=L, N_csa=N)
    t = w.tensors
    # integer-grid indexer (4-bit weights): exact selection on both sides
    t["q_i"] = synth.int_grid((bt, 1, 16, 128), 301, -4, 4, dtype=torch.bfloat16)
    t["k_i"] = synth.int_grid((bt, N, 128), 302, -4, 4, dtype=torch.bfloat16)
    t["w_i"] = synth.dyadic_uniform((bt, 1, 16), 303, bits=4)
    g = {k_: v.to(DEV) for k_, v in t.items()}
    B, m, k = 128, 64, 512
    # caches built from all but the last token's windows (as before the step)
    ckv = ops.compress(g["csa_raw_kv"], g["csa_z"], g["csa_b"], 8, 4)
    hkv = ops.compress(g["hca_raw_kv"], g["hca_z"], g["hca_b"], 128, 128)
    ckv[:, N - 1] = 0
    hkv[:, Nh - 1] = 0
    reps = ops.hisa_pool(g["k_i"], B)
    reps[:, -1] = 0
    # the step
    ops.compress(g["csa_raw_kv"], g["csa_z"], g["csa_b"], 8, 4, N - 1, N, out=ckv)
    ops.compress(g["hca_raw_kv"], g["hca_z"], g["hca_b"], 128, 128, Nh - 1, Nh, out=hkv)
    nb = reps.shape[1]
    ops.hisa_pool(g["k_i"], B, nb - 1, nb, out=reps)
    nv = ops.visible_count(g["q_pos"], 8, 4, N)
    nvh = ops.visible_count(g["q_pos"], 128, 128, Nh)
    idx = ops.hisa_topk(g["q_i"], g["k_i"], g["w_i"], nv, reps, B, m, k)
    o1 = ops.sparse_attn(g["csa_q"], ckv, idx, g["csa_raw_kv"], g["q_pos"], 128)
    o2 = ops.dense_compressed_attn(g["hca_q"], hkv, nvh, g["hca_raw_kv"], g["q_pos"], 128)
    torch.cuda.synchronize()
    sc = 1 / math.sqrt(128)
    for b in range(bt):
        raw_c, raw_h = f64(t["csa_raw_kv"][b]), f64(t["hca_raw_kv"][b])
        r_ckv = oracle.compress(raw_c, f64(t["csa_z"][b]), f64(t["csa_b"]), 8, 4)
        r_hkv = oracle.compress(raw_h, f64(t["hca_z"][b]), f64(t["hca_b"]), 128, 128)
        p = int(t["q_pos"][b, 0])
        assert int(nv[b, 0]) == oracle.n_visible(p, 8, 4, N) == N
        assert int(nvh[b, 0]) == oracle.n_visible(p, 128, 128, Nh) == Nh
        r_idx, _ = oracle.hisa_topk(f64(t["q_i"][b]), f64(t["k_i"][b]), f64(t["w_i"][b]), np.array([N]), B, m, k)
        assert np.array_equal(idx[b].cpu().numpy(), r_idx)
        # GPU caches are bf16 roundings of the oracle's fp64 entries
        r_o1, _ = oracle.sparse_attention(f64(t["csa_q"][b]), r_ckv, r_idx, raw_c, np.array([p]), 128, sc)
        r_o2, _ = oracle.dense_compressed_attention(f64(t["hca_q"][b]), r_hkv, [Nh], raw_h, np.array([p]), 128, sc)
        assert np.abs(f64(o1[b]) - r_o1).max() < 1e-2
        assert np.abs(f64(o2[b]) - r_o2).max() < 1e-2


def test_decode_plan_matches_separate_calls_and_oracle():
    # The native decode-step plan (both branches, one host call) against the
    # separate entry points on copies of the same caches (identical kernels:
    # bit-exact), and against the oracle's step; then a second run on another
    # stream reproduces the first.
    bt, L = 2, 65536
    N = oracle.n_entries(L, 8, 4)
    Nh = oracle.n_entries(L, 128, 128)
    w = synth.hybrid_pair_decode(1, device="cpu", bt=bt, L=L, N_csa=N)
    t = w.tensors
    t["q_i"] = synth.int_grid((bt, 1, 16, 128), 311, -4, 4, dtype=torch.bfloat16)
    t["k_i"] = synth.int_grid((bt, N, 128), 312, -4, 4, dtype=torch.bfloat16)
    t["w_i"] = synth.dyadic_uniform((bt, 1, 16), 313, bits=4)
    g = {k_: v.to(DEV) for k_, v in t.items()}
    B, m, k = 128, 64, 512
    ckv = ops.compress(g["csa_raw_kv"], g["csa_z"], g["csa_b"], 8, 4)
    hkv = ops.compress(g["hca_raw_kv"], g["hca_z"], g["hca_b"], 128, 128)
    ckv[:, N - 1] = 0
    hkv[:, Nh - 1] = 0
    reps = ops.hisa_pool(g["k_i"], B)
    reps[:, -1] = 0
    ckv2, hkv2, reps2 = ckv.clone(), hkv.clone(), reps.clone()
    plan = ops.DecodePlan(q_pos=g["q_pos"], csa_raw_kv=g["csa_raw_kv"], csa_logits=g["csa_z"], csa_pos_bias=g["csa_b"],
                          csa_ckv=ckv, k_i=g["k_i"], reps=reps, q_i=g["q_i"], w_i=g["w_i"], csa_q=g["csa_q"],
                          hca_raw_kv=g["hca_raw_kv"], hca_logits=g["hca_z"], hca_pos_bias=g["hca_b"], hca_ckv=hkv,
                          hca_q=g["hca_q"], B=B, m=m, k=k, return_lse=True)
    o1, o2 = plan.run()
    # the same step through the separate calls
    nv = ops.decode_append(g["csa_raw_kv"], g["csa_z"], g["csa_b"], 8, 4, g["q_pos"], ckv2, g["k_i"], reps2, B)
    idx = ops.hisa_topk(g["q_i"], g["k_i"], g["w_i"], nv, reps2, B, m, k)
    s1, l1 = ops.sparse_attn(g["csa_q"], ckv2, idx, g["csa_raw_kv"], g["q_pos"], 128, return_lse=True)
    nvh = ops.decode_append(g["hca_raw_kv"], g["hca_z"], g["hca_b"], 128, 128, g["q_pos"], hkv2)
    s2, l2 = ops.dense_compressed_attn(g["hca_q"], hkv2, nvh, g["hca_raw_kv"], g["q_pos"], 128, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(ckv, ckv2) and torch.equal(hkv, hkv2) and torch.equal(reps, reps2)
    assert torch.equal(o1, s1) and torch.equal(o2, s2)
    assert torch.equal(plan.csa_lse, l1) and torch.equal(plan.hca_lse, l2)
    first = (o1.clone(), o2.clone())
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        plan.run()
    torch.cuda.synchronize()
    assert torch.equal(plan.csa_out, first[0]) and torch.equal(plan.hca_out, first[1])
    sc = 1 / math.sqrt(128)
    for b in range(bt):
        raw_c, raw_h = f64(t["csa_raw_kv"][b]), f64(t["hca_raw_kv"][b])
        r_ckv = oracle.compress(raw_c, f64(t["csa_z"][b]), f64(t["csa_b"]), 8, 4)
        r_hkv = oracle.compress(raw_h, f64(t["hca_z"][b]), f64(t["hca_b"]), 128, 128)
        p = int(t["q_pos"][b, 0])
        r_idx, _ = oracle.hisa_topk(f64(t["q_i"][b]), f64(t["k_i"][b]), f64(t["w_i"][b]), np.array([N]), B, m, k)
        r_o1, _ = oracle.sparse_attention(f64(t["csa_q"][b]), r_ckv, r_idx, raw_c, np.array([p]), 128, sc)
        r_o2, _ = oracle.dense_compressed_attention(f64(t["hca_q"][b]), r_hkv, [Nh], raw_h, np.array([p]), 128, sc)
        assert np.abs(f64(o1[b]) - r_o1).max() < 1e-2
        assert np.abs(f64(o2[b]) - r_o2).max() < 1e-2
    plan.close()
