"""GPU parity of the decode step at the size the benchmark times.

Hybrid layer pair at 1M context: 8 sequences of 2^20 raw tokens, one query
each at position L - 1, the raw rows either whole or as 128-row rings; CSA
262,143 entries (HISA B = 128, m = 64, k in {2048, 512}) and HCA 8,192
entries; 64 heads x 128, window 128.  The native decode plan runs the step
(cache maintenance of both layers, HISA, sparse and dense attention); its
outputs are checked against the oracle:

  - the CSA selection, bit-exact: the indexer is drawn on the integer grid
    [-4, 4] with 4-bit dyadic head weights, so every fp32 score on both sides
    is exact (the stage-1 bound is asserted on the drawn data);
  - both attention outputs within 1e-2 max-abs, the oracle computing the
    selected entries (and, for HCA, all 8,192 entries) from the raw rows in
    float64, plus the 128 window rows.

Inputs are drawn on the device (seeded); the oracle receives copies of the
same tensors.  Before the step, the caches hold every entry except the ones
the new token completes (zeroed), so the plan's appends are checked too.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from compressed_attention_amd import ops, synth
from helpers import f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BT, L = 8, 1 << 20
N, NH = 262143, 8192
B, M = 128, 64


def _say(*a):
    print("[decode-full]", *a, flush=True)


@pytest.fixture(scope="module")
def full():
    _say(f"drawing inputs on the device: {BT} x {L} tokens, two layers")
    t = dict(synth.hybrid_pair_decode(0, device=DEV, bt=BT, L=L, N_csa=N).tensors)
    t["q_i"] = synth.int_grid((BT, 1, 16, 128), 331, -4, 4, dtype=torch.bfloat16, device=DEV)
    t["k_i"] = synth.int_grid((BT, N, 128), 332, -4, 4, dtype=torch.bfloat16, device=DEV)
    t["w_i"] = synth.dyadic_uniform((BT, 1, 16), 333, device=DEV, bits=4)
    ckv = ops.compress(t["csa_raw_kv"], t["csa_z"], t["csa_b"], 8, 4)
    hkv = ops.compress(t["hca_raw_kv"], t["hca_z"], t["hca_b"], 128, 128)
    reps = ops.hisa_pool(t["k_i"], B)
    torch.cuda.synchronize()
    assert ckv.shape[1] == N and hkv.shape[1] == NH and reps.shape[1] == 2048
    return dict(t=t, ckv=ckv, hkv=hkv, reps=reps, hca_ref=None)


def _ring(x, R):
    """The newest R rows of x [BT, L, ...] at slots r % R."""
    rows = torch.arange(L - R, L, device=x.device)
    out = torch.empty((x.shape[0], R) + tuple(x.shape[2:]), dtype=x.dtype, device=x.device)
    out[:, rows % R] = x[:, rows]
    return out


def _run_plan(F, k, ring=0):
    t = F["t"]
    ckv, hkv, reps = F["ckv"], F["hkv"], F["reps"]
    # the state before the step: the entries (and block mean) that the new
    # token completes are not there yet
    ckv[:, N - 1] = 0
    hkv[:, NH - 1] = 0
    reps[:, -1] = 0
    raw = {n: (_ring(t[n], ring) if ring else t[n]) for n in ("csa_raw_kv", "csa_z", "hca_raw_kv", "hca_z")}
    plan = ops.DecodePlan(q_pos=t["q_pos"], csa_raw_kv=raw["csa_raw_kv"], csa_logits=raw["csa_z"],
                          csa_pos_bias=t["csa_b"], csa_ckv=ckv, k_i=t["k_i"], reps=reps, q_i=t["q_i"], w_i=t["w_i"],
                          csa_q=t["csa_q"], hca_raw_kv=raw["hca_raw_kv"], hca_logits=raw["hca_z"],
                          hca_pos_bias=t["hca_b"], hca_ckv=hkv, hca_q=t["hca_q"], B=B, m=M, k=k, return_idx=True,
                          L=L if ring else None)
    plan.run()
    torch.cuda.synchronize()
    out = (plan.csa_idx[:, 0].cpu().numpy(), f64(plan.csa_out[:, 0]), f64(plan.hca_out[:, 0]))
    plan.close()
    return out


def _stage1_exact_bound(q, k_i, weight_bits):
    # Block sums S_b are integers, block means S_b / 128 and head weights
    # v / 2^bits: every partial sum of a block score is a multiple of
    # 2^-(7 + bits), exact in fp32 while max_v * sum_h sum_c |q_hc S_bc| < 2^24.
    nb = -(-k_i.shape[0] // B)
    pad = np.zeros((nb * B - k_i.shape[0], k_i.shape[1]))
    S = np.concatenate([k_i, pad]).reshape(nb, B, -1).sum(1)
    worst = (np.abs(q) @ np.abs(S).T).sum(0).max()
    assert worst * ((1 << weight_bits) - 1) < 2**24, worst


def _selected_entries(raw_kv_b, z_b, bias, ent):
    """The oracle's compression of the listed CSA entries, from their raw rows
    (each entry's 8-row window, windows laid end to end)."""
    rows = (4 * torch.as_tensor(ent, dtype=torch.int64)[:, None] + torch.arange(8)[None, :]).reshape(-1)
    x = f64(raw_kv_b[rows.to(raw_kv_b.device)])
    z = f64(z_b[rows.to(z_b.device)])
    return oracle.compress(x, z, bias, 8, 8)


@pytest.mark.parametrize("k,ring", [(2048, 0), (512, 0), (2048, 128)])
def test_decode_plan_full_size_matches_oracle(full, k, ring):
    """ring=128: the plan reads only the newest 128 raw rows of each layer,
    kept at slots r % 128 (the configuration the benchmark times)."""
    t = full["t"]
    _say(f"k={k} ring={ring}: running the decode plan")
    idx, o_csa, o_hca = _run_plan(full, k, ring)
    sc = 1 / math.sqrt(128)
    p = L - 1
    assert (t["q_pos"].cpu().numpy() == p).all()
    bias_c, bias_h = f64(t["csa_b"]), f64(t["hca_b"])
    for b in range(BT):
        q_i, w_i = f64(t["q_i"][b]), f64(t["w_i"][b])
        k_i = f64(t["k_i"][b])
        _stage1_exact_bound(q_i[0], k_i, 4)
        r_idx, _ = oracle.hisa_topk(q_i, k_i, w_i, np.array([N]), B, M, k)
        del k_i
        assert np.array_equal(idx[b], r_idx[0]), f"sequence {b}: selection differs"
        # CSA attention: the selected entries, compressed from their raw rows,
        # then the window (the last 128 raw rows, the query being the last)
        ent = r_idx[0][r_idx[0] >= 0]
        sel = _selected_entries(t["csa_raw_kv"][b], t["csa_z"][b], bias_c, ent)
        win = f64(t["csa_raw_kv"][b, L - 128:])
        r_o, _ = oracle.sparse_attention(f64(t["csa_q"][b]), sel, np.arange(len(ent))[None, :], win,
                                         np.array([127]), 128, sc)
        err = float(np.abs(o_csa[b] - r_o[0]).max())
        assert err < 1e-2, (b, err)
        _say(f"k={k} sequence {b}: selection exact, CSA max|err| {err:.2e}")
    # HCA: every entry, compressed from the whole raw sequence in the oracle
    # (independent of k, so computed once)
    if full["hca_ref"] is None:
        refs = []
        for b in range(BT):
            raw = f64(t["hca_raw_kv"][b])
            r_hkv = oracle.compress(raw, f64(t["hca_z"][b]), bias_h, 128, 128)
            assert r_hkv.shape[0] == NH
            r_o, _ = oracle.dense_compressed_attention(f64(t["hca_q"][b]), r_hkv, [NH], raw[L - 128:],
                                                       np.array([127]), 128, sc)
            del raw
            refs.append(r_o[0])
            _say(f"oracle HCA sequence {b} done")
        full["hca_ref"] = refs
    for b in range(BT):
        err = float(np.abs(o_hca[b] - full["hca_ref"][b]).max())
        assert err < 1e-2, (b, err)
    _say(f"k={k}: HCA outputs within 1e-2 of the oracle")
