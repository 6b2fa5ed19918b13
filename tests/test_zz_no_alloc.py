"""The entry point that allocates nothing: hattn_sparse_attn_noalloc (split-K
partials in the library's static device scratch) against hattn_sparse_attn
(partials in a caller workspace), through the C ABI.  The two run the same
kernels on the same split plan, so the outputs must be bit-identical; two
calls in a row, the second smaller, show that nothing left in the shared
scratch by one call leaks into the next."""
import math

import numpy as np
import pytest
import torch

import oracle
from compressed_attention_amd import ops, synth
from helpers import f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(seed, bt, nq, N, L, k, dtype, h=64, d=128):
    g = torch.Generator().manual_seed(seed)
    q = synth.normal((bt, nq, h, d), seed + 1, dtype=dtype)
    ckv = synth.normal((bt, N, 2 * d), seed + 2, dtype=dtype)
    raw = synth.normal((bt, L, 2 * d), seed + 3, dtype=dtype)
    q_pos = torch.randint(0, L, (bt, nq), generator=g, dtype=torch.int32)
    nv = torch.full((bt * nq,), N, dtype=torch.int32)
    idx = synth.random_index_lists(nv, k, seed + 4, n_pad_holes=3).reshape(bt, nq, k)
    return q, ckv, idx, raw, q_pos


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_call_twice(dtype):
    # the vector (fp32) path splits finer, so its first case has fewer queries
    # (its partials must fit the 32 MiB scratch)
    nq = 300 if dtype == torch.bfloat16 else 100
    cases = [
        _case(500, 1, nq, 8191, 32768, 512, dtype),  # several chunks per query
        _case(600, 3, 1, 4000, 9000, 200, dtype),    # smaller: decode shape, different split plan
    ]
    for n, (q, ckv, idx, raw, q_pos) in enumerate(cases):
        g = [x.to(DEV) for x in (q, ckv, idx, raw, q_pos)]
        bt, nq, h, d = q.shape
        out = torch.empty((bt, nq, h, d), dtype=torch.float32, device=DEV)
        lse = torch.empty((bt, nq, h), dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        ops.sparse_attn_noalloc(*g, 128, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before  # nothing allocated through torch either
        ref, ref_lse = ops.sparse_attn(*g, 128, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), n
        assert torch.equal(lse, ref_lse), n
        # and against the oracle on two queries
        sc = 1 / math.sqrt(d)
        for r in (0, bt * nq - 1):
            b, qi = divmod(r, nq)
            r_o, _ = oracle.sparse_attention(f64(q[b, qi:qi + 1]), f64(ckv[b]), idx[b, qi:qi + 1].numpy(),
                                             f64(raw[b]), q_pos[b, qi:qi + 1].numpy(), 128, sc)
            tol = 1e-2 if dtype == torch.bfloat16 else 1e-4
            assert np.abs(f64(out[b, qi]) - r_o[0]).max() < tol, (n, r)
