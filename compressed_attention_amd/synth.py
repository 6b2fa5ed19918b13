"""Seeded synthetic inputs for the hybrid compressed-attention workloads.

This module holds input recipes only -- shapes, distributions and seeds -- and
none of the method's arithmetic (no windows, visibility, scores, selection or
attention).  It is the one module that both the HIP path (tests, bench) and
the CPU oracle are fed from.  Quantities that depend on the method (such as
the number of entries a query may see) are computed by each side itself; the
entry counts below are the ones the workload descriptions state, and the
oracle tests check them against the window geometry.

Every tensor comes from its own ``torch.Generator`` whose seed is spawned from
``numpy.random.SeedSequence(seed)`` in a fixed order of tensor names, so any
tensor can be regenerated alone.  ``device`` selects where the draw happens:
the CPU generator (used for every size the oracle runs in full) or the device
generator (used for the 1M-token caches, where host generation would take
minutes); the two give different values for the same seed, and each workload
fixes which one it uses.  bf16 tensors are drawn in fp32 and rounded once,
round-to-nearest-even.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


# ----------------------------------------------------------------------------
# seeds and primitive draws
# ----------------------------------------------------------------------------


def tensor_seeds(seed: int, names: list[str]) -> dict[str, int]:
    """One 63-bit seed per tensor name, spawned in the given order."""
    kids = np.random.SeedSequence(seed).spawn(len(names))
    return {n: int(k.generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1) for n, k in zip(names, kids)}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed & ((1 << 63) - 1))
    return g


def normal(shape, seed: int, std: float = 1.0, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """N(0, std^2) draw in fp32, then cast once (RNE) to ``dtype``."""
    t = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def uniform(shape, seed: int, device="cpu") -> torch.Tensor:
    """U[0, 1) in fp32."""
    return torch.rand(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)


def dyadic_uniform(shape, seed: int, device="cpu", bits: int = 8) -> torch.Tensor:
    """U[0,1) snapped down to a multiple of 2^-bits (exact in fp32 products)."""
    scale = float(1 << bits)
    return torch.floor(uniform(shape, seed, device) * scale) / scale


def int_grid(shape, seed: int, lo: int, hi: int, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """Integers drawn uniformly from {lo, ..., hi}, stored as ``dtype``."""
    t = torch.randint(lo, hi + 1, shape, generator=_gen(seed, device), device=device)
    return t.to(dtype)


def tiled_bias(r: int, w: int, seed: int, std: float = 0.1) -> torch.Tensor:
    """A length-r position bias ~ N(0, std^2) repeated to cover a window of w."""
    br = normal((r,), seed, std=std)
    reps = -(-w // r)
    return br.repeat(reps)[:w].contiguous()


def random_index_lists(n_vis, k: int, seed: int, n_pad_holes: int = 0) -> torch.Tensor:
    """Per query, a random ascending set of min(k, n_vis[q]) distinct entries.

    Padded with -1 to length k.  ``n_pad_holes`` extra -1 values are spliced in
    at random places (the attention must skip -1 wherever it appears).
    Returns int32 [nq][k] on the CPU.
    """
    g = _gen(seed, "cpu")
    n_vis = [int(v) for v in n_vis]
    out = torch.full((len(n_vis), k), -1, dtype=torch.int32)
    for q, n in enumerate(n_vis):
        c = min(k, n)
        if c:
            pick = torch.randperm(n, generator=g)[:c].sort().values.to(torch.int32)
            if n_pad_holes and c > n_pad_holes:
                drop = torch.randperm(c, generator=g)[:n_pad_holes]
                pick[drop] = -1
            out[q, :c] = pick
    return out


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    """Widen any tensor (bf16/fp32/int) to a float64 NumPy array on the host."""
    return t.detach().to("cpu", torch.float64).numpy()


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------


@dataclass
class Workload:
    name: str
    tensors: dict = field(default_factory=dict)
    params: dict = field(default_factory=dict)


def tiny_hybrid_layer(seed: int = 0, device="cpu") -> Workload:
    """Tiny hybrid layer, fp32: L=4096, d=64, H=8, 64 queries at 2048 + 32 j.

    CSA: 8-token windows at stride 4 (1023 entries, as stated), bias of length
    r=4 tiled to 8; indexer 4 heads x 32 dims on the integer grid [-8, 8] with
    dyadic U(0,1) head weights; top-k = 64.  HCA: 128-token disjoint windows
    (32 entries), bias of length 128.  Window 128.  Both branches read the same
    raw q/k/v.
    """
    L, d, H, nq, HI, DI = 4096, 64, 8, 64, 4, 32
    N_csa, N_hca = 1023, 32
    names = ["raw_kv", "z", "b_csa", "b_hca", "q", "q_i", "k_i", "w_i"]
    s = tensor_seeds(seed, names)
    t = {
        "raw_kv": normal((1, L, 2 * d), s["raw_kv"], device=device),
        "z": normal((1, L), s["z"], device=device),
        "b_csa": tiled_bias(4, 8, s["b_csa"]).to(device),
        "b_hca": tiled_bias(128, 128, s["b_hca"]).to(device),
        "q": normal((1, nq, H, d), s["q"], device=device),
        "q_i": int_grid((1, nq, HI, DI), s["q_i"], -8, 8, device=device),
        "k_i": int_grid((1, N_csa, DI), s["k_i"], -8, 8, device=device),
        "w_i": dyadic_uniform((1, nq, HI), s["w_i"], device=device),
        "q_pos": (2048 + 32 * torch.arange(nq, dtype=torch.int32)).reshape(1, nq).to(device),
    }
    p = dict(L=L, d=d, H=H, nq=nq, h_i=HI, d_i=DI, N_csa=N_csa, N_hca=N_hca, k=64, window=128,
             w_csa=8, s_csa=4, w_hca=128, s_hca=128, dtype="f32", bt=1)
    return Workload("tiny_hybrid_layer_fp32", t, p)


def csa_prefill_chunk(seed: int = 0, device="cpu", integer_indexer: bool = False) -> Workload:
    """CSA prefill chunk, bf16: L=32768, the last 1024 positions as queries.

    H=64, d=128; 8-token windows at stride 4 (8191 entries, as stated); indexer
    16 heads x 64 dims (N(0,1) bf16, head weights U(0,1)), or on the integer
    grid [-8, 8] with dyadic weights when ``integer_indexer``; k=512; window 128.
    """
    L, d, H, nq, HI, DI, N = 32768, 128, 64, 1024, 16, 64, 8191
    names = ["raw_kv", "z", "b", "q", "q_i", "k_i", "w_i"]
    s = tensor_seeds(seed, names)
    bf = torch.bfloat16
    if integer_indexer:
        q_i = int_grid((1, nq, HI, DI), s["q_i"], -8, 8, dtype=bf, device=device)
        k_i = int_grid((1, N, DI), s["k_i"], -8, 8, dtype=bf, device=device)
        w_i = dyadic_uniform((1, nq, HI), s["w_i"], device=device)
    else:
        q_i = normal((1, nq, HI, DI), s["q_i"], dtype=bf, device=device)
        k_i = normal((1, N, DI), s["k_i"], dtype=bf, device=device)
        w_i = uniform((1, nq, HI), s["w_i"], device=device)
    t = {
        "raw_kv": normal((1, L, 2 * d), s["raw_kv"], dtype=bf, device=device),
        "z": normal((1, L), s["z"], device=device),
        "b": tiled_bias(4, 8, s["b"]).to(device),
        "q": normal((1, nq, H, d), s["q"], dtype=bf, device=device),
        "q_i": q_i, "k_i": k_i, "w_i": w_i,
        "q_pos": torch.arange(L - nq, L, dtype=torch.int32).reshape(1, nq).to(device),
    }
    p = dict(L=L, d=d, H=H, nq=nq, h_i=HI, d_i=DI, N=N, k=512, window=128, w=8, s=4, dtype="bf16", bt=1)
    return Workload("csa_prefill_chunk_32k_bf16", t, p)


def hca_decode(seed: int = 0, device="cpu", bt: int = 32, L: int = 1 << 20) -> Workload:
    """HCA dense decode, bf16: bt sequences of L raw tokens, one query each at L-1.

    128-token disjoint windows (8192 entries at L = 2^20, as stated), bias of
    length 128; H=64, d=128; window 128.  Per-sequence tensors come from one
    generator each so a single sequence can be regenerated alone.
    """
    d, H = 128, 64
    names = ["raw_kv", "z", "b", "q"]
    s = tensor_seeds(seed, names)
    bf = torch.bfloat16
    t = {
        "raw_kv": normal((bt, L, 2 * d), s["raw_kv"], dtype=bf, device=device),
        "z": normal((bt, L), s["z"], device=device),
        "b": tiled_bias(128, 128, s["b"]).to(device),
        "q": normal((bt, 1, H, d), s["q"], dtype=bf, device=device),
        "q_pos": torch.full((bt, 1), L - 1, dtype=torch.int32).to(device),
    }
    p = dict(L=L, d=d, H=H, nq=1, bt=bt, window=128, w=128, s=128, dtype="bf16")
    return Workload(f"hca_decode_{bt}x{L}_bf16", t, p)


def indexer_128k(seed: int = 0, device="cpu", N: int = 131072, nq: int = 1024, n_needles: int = 64,
                 integer_grid: bool = False, weight_bits: int = 8) -> Workload:
    """Indexer chunk over 131072 entries, 1024 queries at the end, 16 x 128 heads.

    Keys N(0,1) bf16 with ``n_needles`` rows at distinct random positions
    scaled by 4 (their own draw times 4); queries N(0,1) bf16; head weights
    U(0,1).  Query j of the chunk sits at entry position N - nq + j.  HISA:
    B=128, m=64, k=2048.  ``integer_grid`` swaps in grid values in [-4, 4]
    (dyadic weights on a 2^-weight_bits grid) so that fp32 scores are exact;
    4-bit weights also keep the block-mean (HISA stage 1) scores exact.
    """
    HI, DI = 16, 128
    names = ["q_i", "k_i", "w_i", "needles"]
    s = tensor_seeds(seed, names)
    bf = torch.bfloat16
    if integer_grid:
        k_i = int_grid((1, N, DI), s["k_i"], -4, 4, device=device)
        q_i = int_grid((1, nq, HI, DI), s["q_i"], -4, 4, dtype=bf, device=device)
        w_i = dyadic_uniform((1, nq, HI), s["w_i"], device=device, bits=weight_bits)
    else:
        k_i = normal((1, N, DI), s["k_i"], device=device)
        q_i = normal((1, nq, HI, DI), s["q_i"], dtype=bf, device=device)
        w_i = uniform((1, nq, HI), s["w_i"], device=device)
    needles = torch.randperm(N, generator=_gen(s["needles"], "cpu"))[:n_needles].sort().values
    if not integer_grid:
        k_i[0, needles.to(k_i.device)] *= 4.0
    t = {
        "q_i": q_i, "k_i": k_i.to(bf), "w_i": w_i,
        "entry_pos": torch.arange(N - nq, N, dtype=torch.int32).reshape(1, nq).to(device),
        "needles": needles,
    }
    p = dict(N=N, nq=nq, h_i=HI, d_i=DI, k=2048, B=128, m=64, dtype="bf16", bt=1)
    return Workload(f"indexer_{N}_chunk{nq}_bf16", t, p)


def hybrid_pair_decode(seed: int = 0, device="cpu", bt: int = 8, L: int = 1 << 20, N_csa: int = 262143) -> Workload:
    """Full hybrid layer pair at 1M context, bf16: bt decode queries at L-1.

    CSA layer: raw K|V, logits, bias of length 4 tiled to 8, queries (64 x 128),
    indexer 16 x 128 over 262143 entries (as stated at L = 2^20), head weights
    U(0,1); HISA B=128, m=64, k in {512, 2048}.  HCA layer: its own raw K|V,
    logits, bias of length 128 and queries.  Window 128 in both.  A smaller L
    must come with the matching CSA entry count ``N_csa`` (the indexer keys
    are drawn per entry).
    """
    d, H, HI, DI = 128, 64, 16, 128
    names = ["csa_raw_kv", "csa_z", "csa_b", "csa_q", "q_i", "k_i", "w_i",
             "hca_raw_kv", "hca_z", "hca_b", "hca_q"]
    s = tensor_seeds(seed, names)
    bf = torch.bfloat16
    t = {
        "csa_raw_kv": normal((bt, L, 2 * d), s["csa_raw_kv"], dtype=bf, device=device),
        "csa_z": normal((bt, L), s["csa_z"], device=device),
        "csa_b": tiled_bias(4, 8, s["csa_b"]).to(device),
        "csa_q": normal((bt, 1, H, d), s["csa_q"], dtype=bf, device=device),
        "q_i": normal((bt, 1, HI, DI), s["q_i"], dtype=bf, device=device),
        "k_i": normal((bt, N_csa, DI), s["k_i"], dtype=bf, device=device),
        "w_i": uniform((bt, 1, HI), s["w_i"], device=device),
        "hca_raw_kv": normal((bt, L, 2 * d), s["hca_raw_kv"], dtype=bf, device=device),
        "hca_z": normal((bt, L), s["hca_z"], device=device),
        "hca_b": tiled_bias(128, 128, s["hca_b"]).to(device),
        "hca_q": normal((bt, 1, H, d), s["hca_q"], dtype=bf, device=device),
        "q_pos": torch.full((bt, 1), L - 1, dtype=torch.int32).to(device),
    }
    p = dict(L=L, d=d, H=H, h_i=HI, d_i=DI, bt=bt, nq=1, N_csa=N_csa, B=128, m=64,
             ks=(512, 2048), window=128, dtype="bf16")
    return Workload(f"hybrid_pair_decode_{bt}x{L}_bf16", t, p)
