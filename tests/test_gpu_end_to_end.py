"""GPU parity of the whole tiny hybrid layer chain (fp32, seed 0):
compress -> visibility -> flat / HISA selection -> sparse attention (CSA)
and compress -> dense attention (HCA), against the same chain in the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from compressed_attention_amd import ops, synth
from helpers import assert_bf16_close, f64

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


@pytest.mark.parametrize("h,d", [(16, 64), (16, 128), (32, 64), (32, 128), (64, 64)])
def test_decode_plan_head_shapes(h, d):
    """The decode plan's paired attention launch for other head counts and
    sizes (16 or 32 heads per query, d = 64): bit-exact against the separate
    calls, and within 1e-2 of the oracle (integer-grid indexer, so that both
    select the same entries)."""
    bt, L = 2, 8192
    N = oracle.n_entries(L, 8, 4)
    Nh = oracle.n_entries(L, 128, 128)
    bf = torch.bfloat16
    t = {
        "csa_raw_kv": synth.normal((bt, L, 2 * d), 401, dtype=bf),
        "csa_z": synth.normal((bt, L), 402),
        "csa_b": synth.tiled_bias(4, 8, 403),
        "csa_q": synth.normal((bt, 1, h, d), 404, dtype=bf),
        "q_i": synth.int_grid((bt, 1, 16, 128), 405, -4, 4, dtype=bf),
        "k_i": synth.int_grid((bt, N, 128), 406, -4, 4, dtype=bf),
        "w_i": synth.dyadic_uniform((bt, 1, 16), 407, bits=4),
        "hca_raw_kv": synth.normal((bt, L, 2 * d), 408, dtype=bf),
        "hca_z": synth.normal((bt, L), 409),
        "hca_b": synth.tiled_bias(128, 128, 410),
        "hca_q": synth.normal((bt, 1, h, d), 411, dtype=bf),
        "q_pos": torch.tensor([[L - 1], [L - 3]], dtype=torch.int32),
    }
    g = {k_: v.to(DEV) for k_, v in t.items()}
    B, m, k = 128, 4, 128
    ckv = ops.compress(g["csa_raw_kv"], g["csa_z"], g["csa_b"], 8, 4)
    hkv = ops.compress(g["hca_raw_kv"], g["hca_z"], g["hca_b"], 128, 128)
    ckv[:, N - 1] = 0  # completed by the step
    hkv[:, Nh - 1] = 0
    reps = ops.hisa_pool(g["k_i"], B)
    ckv2, hkv2, reps2 = ckv.clone(), hkv.clone(), reps.clone()
    plan = ops.DecodePlan(q_pos=g["q_pos"], csa_raw_kv=g["csa_raw_kv"], csa_logits=g["csa_z"], csa_pos_bias=g["csa_b"],
                          csa_ckv=ckv, k_i=g["k_i"], reps=reps, q_i=g["q_i"], w_i=g["w_i"], csa_q=g["csa_q"],
                          hca_raw_kv=g["hca_raw_kv"], hca_logits=g["hca_z"], hca_pos_bias=g["hca_b"], hca_ckv=hkv,
                          hca_q=g["hca_q"], B=B, m=m, k=k, return_lse=True)
    o1, o2 = plan.run()
    nv = ops.decode_append(g["csa_raw_kv"], g["csa_z"], g["csa_b"], 8, 4, g["q_pos"], ckv2, g["k_i"], reps2, B)
    idx = ops.hisa_topk(g["q_i"], g["k_i"], g["w_i"], nv, reps2, B, m, k)
    s1, l1 = ops.sparse_attn(g["csa_q"], ckv2, idx, g["csa_raw_kv"], g["q_pos"], 128, return_lse=True)
    nvh = ops.decode_append(g["hca_raw_kv"], g["hca_z"], g["hca_b"], 128, 128, g["q_pos"], hkv2)
    s2, l2 = ops.dense_compressed_attn(g["hca_q"], hkv2, nvh, g["hca_raw_kv"], g["q_pos"], 128, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(ckv, ckv2) and torch.equal(hkv, hkv2) and torch.equal(reps, reps2)
    assert torch.equal(o1, s1) and torch.equal(o2, s2)
    assert torch.equal(plan.csa_lse, l1) and torch.equal(plan.hca_lse, l2)
    sc = 1 / math.sqrt(d)
    for b in range(bt):
        raw_c, raw_h = f64(t["csa_raw_kv"][b]), f64(t["hca_raw_kv"][b])
        p = int(t["q_pos"][b, 0])
        r_ckv = oracle.compress(raw_c, f64(t["csa_z"][b]), f64(t["csa_b"]), 8, 4)
        r_hkv = oracle.compress(raw_h, f64(t["hca_z"][b]), f64(t["hca_b"]), 128, 128)
        nv_c = oracle.n_visible(p, 8, 4, N)
        nv_h = oracle.n_visible(p, 128, 128, Nh)
        r_idx, _ = oracle.hisa_topk(f64(t["q_i"][b]), f64(t["k_i"][b]), f64(t["w_i"][b]), np.array([nv_c]), B, m, k)
        assert np.array_equal(idx[b].cpu().numpy(), r_idx)
        r_o1, _ = oracle.sparse_attention(f64(t["csa_q"][b]), r_ckv, r_idx, raw_c, np.array([p]), 128, sc)
        r_o2, _ = oracle.dense_compressed_attention(f64(t["hca_q"][b]), r_hkv, [nv_h], raw_h, np.array([p]), 128, sc)
        assert np.abs(f64(o1[b]) - r_o1).max() < 1e-2
        assert np.abs(f64(o2[b]) - r_o2).max() < 1e-2
    plan.close()


@pytest.mark.parametrize("dtype,d_i", [(torch.bfloat16, 48), (torch.float32, 48), (torch.bfloat16, 16),
                                       (torch.bfloat16, 32), (torch.bfloat16, 64), (torch.bfloat16, 256),
                                       (torch.float32, 128)])
def test_decode_plan_indexer_widths(dtype, d_i):
    # The decode plan at indexer widths that take each stage-1 path: 48 has no
    # MFMA instantiation (vector kernels), 16 has one but its LDS tile is too
    # small for the fused front kernel's cache-maintenance scratch, 32, 64 and
    # 256 run the fused front kernel; fp32 runs every step on the vector
    # kernels.
    # Integer-grid indexer with 4-bit weights: the selection is exact.
    bt, L = 2, 16384
    N, Nh = oracle.n_entries(L, 8, 4), oracle.n_entries(L, 128, 128)
    B, m, k = 128, 8, 256
    t = dict(synth.hybrid_pair_decode(2, device="cpu", bt=bt, L=L, N_csa=N).tensors)
    t["q_i"] = synth.int_grid((bt, 1, 16, d_i), 341 + d_i, -4, 4)
    t["k_i"] = synth.int_grid((bt, N, d_i), 342 + d_i, -4, 4)
    t["w_i"] = synth.dyadic_uniform((bt, 1, 16), 343 + d_i, bits=4)
    for name in ("csa_raw_kv", "csa_q", "hca_raw_kv", "hca_q", "q_i", "k_i"):
        t[name] = t[name].to(dtype)
    g = {k_: v.to(DEV) for k_, v in t.items()}
    ckv = ops.compress(g["csa_raw_kv"], g["csa_z"], g["csa_b"], 8, 4)
    hkv = ops.compress(g["hca_raw_kv"], g["hca_z"], g["hca_b"], 128, 128)
    ckv[:, N - 1] = 0
    hkv[:, Nh - 1] = 0
    reps = ops.hisa_pool(g["k_i"], B)
    reps[:, -1] = 0
    plan = ops.DecodePlan(q_pos=g["q_pos"], csa_raw_kv=g["csa_raw_kv"], csa_logits=g["csa_z"], csa_pos_bias=g["csa_b"],
                          csa_ckv=ckv, k_i=g["k_i"], reps=reps, q_i=g["q_i"], w_i=g["w_i"], csa_q=g["csa_q"],
                          hca_raw_kv=g["hca_raw_kv"], hca_logits=g["hca_z"], hca_pos_bias=g["hca_b"], hca_ckv=hkv,
                          hca_q=g["hca_q"], B=B, m=m, k=k, return_idx=True)
    o1, o2 = plan.run()
    torch.cuda.synchronize()
    tol = 1e-2 if dtype == torch.bfloat16 else 1e-4
    sc = 1 / math.sqrt(128)
    for b in range(bt):
        raw_c, raw_h = f64(t["csa_raw_kv"][b]), f64(t["hca_raw_kv"][b])
        r_ckv = oracle.compress(raw_c, f64(t["csa_z"][b]), f64(t["csa_b"]), 8, 4)
        r_hkv = oracle.compress(raw_h, f64(t["hca_z"][b]), f64(t["hca_b"]), 128, 128)
        p = int(t["q_pos"][b, 0])
        r_idx, _ = oracle.hisa_topk(f64(t["q_i"][b]), f64(t["k_i"][b]), f64(t["w_i"][b]), np.array([N]), B, m, k)
        assert np.array_equal(plan.csa_idx[b].cpu().numpy(), r_idx), b
        r_o1, _ = oracle.sparse_attention(f64(t["csa_q"][b]), r_ckv, r_idx, raw_c, np.array([p]), 128, sc)
        r_o2, _ = oracle.dense_compressed_attention(f64(t["hca_q"][b]), r_hkv, [Nh], raw_h, np.array([p]), 128, sc)
        assert np.abs(f64(o1[b]) - r_o1).max() < tol, b
        assert np.abs(f64(o2[b]) - r_o2).max() < tol, b
    # the appended block mean is the oracle's mean of the last block
    r_reps = oracle.hisa_pool(f64(t["k_i"][0]), B)
    assert np.array_equal(f64(reps[0, -1]), r_reps[-1])
    plan.close()


@pytest.mark.parametrize("nq,w,s", [(1, 4, 2), (64, 4, 2), (1, 1, 1)])
def test_csa2_layer_group(nq, w, s):
    # CSA2: the K|V cache and its indexer keys compressed at the group's one
    # rate (or left uncompressed: w = s = 1), one flat top-512 selection, and
    # two layers' 64 query heads each attending to the shared selection plus
    # their window: the layers fold into 128 MFMA heads (two head groups).
    bt, L, G, H, d, DI, k = 2, 8192, 2, 64, 128, 64, 512
    names = synth.tensor_seeds(7, ["raw", "raw_ki", "z", "b", "q", "q_i", "w_i"])
    raw = synth.normal((bt, L, 2 * d), names["raw"], dtype=torch.bfloat16)
    raw_ki = synth.int_grid((bt, L, DI), names["raw_ki"], -8, 8, dtype=torch.bfloat16)
    z = synth.normal((bt, L), names["z"])
    b = synth.tiled_bias(2, w, names["b"]) if w > 1 else torch.zeros(1)
    q = synth.normal((bt, nq, G * H, d), names["q"], dtype=torch.bfloat16)
    q_i = synth.int_grid((bt, nq, 16, DI), names["q_i"], -8, 8, dtype=torch.bfloat16)
    w_i = synth.dyadic_uniform((bt, nq, 16), names["w_i"])
    q_pos = torch.arange(L - nq, L, dtype=torch.int32).reshape(1, nq).repeat(bt, 1)
    N = oracle.n_entries(L, w, s)
    g = {n: t.to(DEV) for n, t in dict(raw=raw, raw_ki=raw_ki, z=z, b=b, q=q, q_i=q_i, w_i=w_i, q_pos=q_pos).items()}
    if w > 1:
        # integer-grid keys merged with softmax weights are not integers:
        # the selection stays exact only with uniform weights, so the
        # indexer keys get no logits; K|V use the real ones
        ckv, _ = ops.compress_with_index(g["raw"], g["raw_ki"], g["z"], g["b"], w, s)
        _, k_i = ops.compress_with_index(g["raw"], g["raw_ki"], None, None, w, s)
    else:
        ckv, k_i = ops.compress_with_index(g["raw"], g["raw_ki"], g["z"], None, w, s)
    nv = ops.visible_count(g["q_pos"], w, s, N)
    idx = ops.index_topk(g["q_i"], k_i, g["w_i"], nv, k)
    out = ops.sparse_attn(g["q"], ckv, idx, g["raw"], g["q_pos"], 128)
    torch.cuda.synchronize()
    sc = 1 / math.sqrt(d)
    for bb in range(bt):
        qq = f64(q[bb]).reshape(nq, G, H, d).transpose(1, 0, 2, 3)
        if w > 1:
            r_o, _, r_idx = oracle.csa2_layer_group(qq, f64(raw[bb]), f64(raw_ki[bb]), f64(z[bb]), f64(b), f64(q_i[bb]),
                                                    f64(w_i[bb]), q_pos[bb].numpy(), k, 128, w, s, sc)
            # the reference's selection over the same uniform-weight keys
            r_ki = oracle.compress(f64(raw_ki[bb]), None, None, w, s)
            nvh = np.array([oracle.n_visible(int(p), w, s, N) for p in q_pos[bb]])
            r_idx = oracle.flat_topk(f64(q_i[bb]), r_ki, f64(w_i[bb]), nvh, k)
            ckv_r = oracle.compress(f64(raw[bb]), f64(z[bb]), f64(b), w, s)
            r_o = np.stack([oracle.sparse_attention(qq[gg], ckv_r, r_idx, f64(raw[bb]), q_pos[bb].numpy(), 128, sc)[0]
                            for gg in range(G)])
        else:
            r_o, _, r_idx = oracle.csa2_layer_group(qq, f64(raw[bb]), f64(raw_ki[bb]), f64(z[bb]), None, f64(q_i[bb]),
                                                    f64(w_i[bb]), q_pos[bb].numpy(), k, 128, w, s, sc)
        assert np.array_equal(idx[bb].cpu().numpy(), r_idx), bb
        got = f64(out[bb]).reshape(nq, G, H, d).transpose(1, 0, 2, 3)
        assert np.abs(got - r_o).max() < 1e-2, (bb, float(np.abs(got - r_o).max()))


@pytest.mark.parametrize("graph", [False, True])
def test_decode_plan_ring_multi_step(graph):
    # A decode loop of 130 steps (positions 3500 .. 3629): both layers' raw
    # K|V rows and logits live in 128-row rings (before each step the
    # caller writes the new token's rows at slot p % 128), and the caches
    # grow by the plan's own appends.  The run crosses CSA-entry (every 4
    # tokens), HCA-entry (p = 3583) and HISA-block (entry 896, p = 3591)
    # boundaries.  Checked against the oracle on the whole raw prefix every
    # 8 steps and at the boundaries; a second plan on the full raw arrays
    # must give the same bits at every step.  With graph=True the ring plan
    # runs each step as one launch of its captured graph (replayed 130 times,
    # with eager writes and copies between the replays).
    bt, L, R, B, m, k = 2, 4096, 128, 128, 4, 128
    N, Nh = oracle.n_entries(L, 8, 4), oracle.n_entries(L, 128, 128)
    w = synth.hybrid_pair_decode(3, device="cpu", bt=bt, L=L, N_csa=N)
    t = dict(w.tensors)
    t["q_i"] = synth.int_grid((bt, 1, 16, 128), 351, -4, 4, dtype=torch.bfloat16)
    t["k_i"] = synth.int_grid((bt, N, 128), 352, -4, 4, dtype=torch.bfloat16)
    t["w_i"] = synth.dyadic_uniform((bt, 1, 16), 353, bits=4)
    g = {k_: v.to(DEV) for k_, v in t.items()}
    p0, T = 3500, 130
    nv0, nvh0 = oracle.n_visible(p0 - 1, 8, 4, N), oracle.n_visible(p0 - 1, 128, 128, Nh)
    caches = []
    for _ in range(2):  # ring plan, full plan
        ckv = ops.compress(g["csa_raw_kv"], g["csa_z"], g["csa_b"], 8, 4)
        hkv = ops.compress(g["hca_raw_kv"], g["hca_z"], g["hca_b"], 128, 128)
        ckv[:, nv0:] = 0
        hkv[:, nvh0:] = 0
        caches.append((ckv, hkv, ops.hisa_pool(g["k_i"], B)))
    rings = {n: torch.zeros((bt, R) + tuple(g[n].shape[2:]), dtype=g[n].dtype, device=DEV)
             for n in ("csa_raw_kv", "hca_raw_kv", "csa_z", "hca_z")}
    for r in range(p0 - R, p0):
        for n, ring in rings.items():
            ring[:, r % R] = g[n][:, r]
    q_pos = torch.full((bt, 1), p0, dtype=torch.int32, device=DEV)
    common = dict(csa_pos_bias=g["csa_b"], hca_pos_bias=g["hca_b"], k_i=g["k_i"], q_i=g["q_i"], w_i=g["w_i"],
                  csa_q=g["csa_q"], hca_q=g["hca_q"], B=B, m=m, k=k, return_idx=True, q_pos=q_pos)
    ring_plan = ops.DecodePlan(csa_raw_kv=rings["csa_raw_kv"], csa_logits=rings["csa_z"], hca_raw_kv=rings["hca_raw_kv"],
                               hca_logits=rings["hca_z"], csa_ckv=caches[0][0], hca_ckv=caches[0][1], reps=caches[0][2],
                               L=L, **common)
    full_plan = ops.DecodePlan(csa_raw_kv=g["csa_raw_kv"], csa_logits=g["csa_z"], hca_raw_kv=g["hca_raw_kv"],
                               hca_logits=g["hca_z"], csa_ckv=caches[1][0], hca_ckv=caches[1][1], reps=caches[1][2],
                               **common)
    sc = 1 / math.sqrt(128)
    r_ckv = [oracle.compress(f64(t["csa_raw_kv"][b]), f64(t["csa_z"][b]), f64(t["csa_b"]), 8, 4) for b in range(bt)]
    r_hkv = [oracle.compress(f64(t["hca_raw_kv"][b]), f64(t["hca_z"][b]), f64(t["hca_b"]), 128, 128) for b in range(bt)]
    checked = 0
    for p in range(p0, p0 + T):
        for n, ring in rings.items():
            ring[:, p % R] = g[n][:, p]
        q_pos.fill_(p)
        o_r = [x.clone() for x in (ring_plan.run_graph() if graph else ring_plan.run())] + [ring_plan.csa_idx.clone()]
        o_f = [x.clone() for x in full_plan.run()] + [full_plan.csa_idx.clone()]
        for a, b_ in zip(o_r, o_f):
            assert torch.equal(a, b_), p
        if (p - p0) % 8 and p not in (3503, 3583, 3591):
            continue
        torch.cuda.synchronize()
        nv, nvh = oracle.n_visible(p, 8, 4, N), oracle.n_visible(p, 128, 128, Nh)
        for b in range(bt):
            r_idx, _ = oracle.hisa_topk(f64(t["q_i"][b]), f64(t["k_i"][b]), f64(t["w_i"][b]), np.array([nv]), B, m, k)
            assert np.array_equal(o_r[2][b].cpu().numpy(), r_idx), (p, b)
            r_o1, _ = oracle.sparse_attention(f64(t["csa_q"][b]), r_ckv[b], r_idx, f64(t["csa_raw_kv"][b]),
                                              np.array([p]), 128, sc)
            r_o2, _ = oracle.dense_compressed_attention(f64(t["hca_q"][b]), r_hkv[b], [nvh], f64(t["hca_raw_kv"][b]),
                                                        np.array([p]), 128, sc)
            assert np.abs(f64(o_r[0][b]) - r_o1).max() < 1e-2, (p, b)
            assert np.abs(f64(o_r[1][b]) - r_o2).max() < 1e-2, (p, b)
        checked += 1
    torch.cuda.synchronize()
    # the entries the loop completed, appended from the rings
    nv_end, nvh_end = oracle.n_visible(p0 + T - 1, 8, 4, N), oracle.n_visible(p0 + T - 1, 128, 128, Nh)
    assert nvh_end == nvh0 + 1 and nv_end > nv0 + 30
    for b in range(bt):
        assert_bf16_close(f64(caches[0][0][b, nv0:nv_end]), r_ckv[b][nv0:nv_end])
        assert_bf16_close(f64(caches[0][1][b, nvh0:nvh_end]), r_hkv[b][nvh0:nvh_end])
    assert checked >= 18
    ring_plan.close()
    full_plan.close()
