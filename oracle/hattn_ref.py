"""fp64 definitions of every step of the hybrid compressed-attention path.

TEST INFRASTRUCTURE (see the package docstring): nothing in the product may
import this module.

Conventions shared by all functions (all arrays are NumPy, computed in
float64; inputs that the GPU receives as bf16 are passed here already rounded
to bf16 and widened, so both sides see identical values):

  raw_kv  [L][2d]   one shared K|V head per raw token, K = [:d], V = [d:]
  ckv     [N][2d]   compressed entries in the same K|V packing
  q       [nq][H][d]
  q_i     [nq][H_I][d_I], k_i [N][d_I], w_i [nq][H_I]  (indexer)
  n_vis   [nq]      number of visible entries per query
  idx     [nq][k]   int64, ascending, padded with -1
"""

from __future__ import annotations


import numpy as np

# ----------------------------------------------------------------------------
# 1. Window geometry and visibility
# ----------------------------------------------------------------------------


def n_entries(L: int, w: int, s: int) -> int:
    """Number of complete windows of width ``w`` at stride ``s`` over ``L`` tokens.

    Entry i covers raw tokens [i*s, i*s + w).  Only complete windows exist.
    [HCA] section 怎么压: every compressed entry is a weighted merge of a run of
    raw entries; HCA's runs are 128 long and do not overlap.  CSA's overlapping
    runs of 8 at stride 4 are a design choice (the pages only say HCA differs
    by being disjoint and by its larger rate; CSA's rate is 4 per [HCA] table
    in section 它补的正是 CSA 的短板 and [TRDM] section 2.1).
    """
    if L < w:
        return 0
    return (L - w) // s + 1


def entry_span(i: int, w: int, s: int) -> tuple[int, int]:
    """Half-open raw-token range [start, end) merged into entry i."""
    return i * s, i * s + w


def n_visible(p: int, w: int, s: int, N: int) -> int:
    """How many entries a query at raw position ``p`` may see.

    Causal reading: entry i is visible iff its last raw token i*s + w - 1 is
    at or before p (a query never sees a summary that mixes in its future).
    Written as a direct count over entries so that the closed forms used by
    the kernels are checked against it, not the other way round.
    """
    count = 0
    for i in range(N):
        start, end = entry_span(i, w, s)
        if end - 1 <= p:
            count += 1
        else:
            break  # ends grow with i
    return count


# ----------------------------------------------------------------------------
# 2. Sequence-dimension compression
# ----------------------------------------------------------------------------


def compress(x: np.ndarray, z: np.ndarray | None, b: np.ndarray | None, w: int, s: int) -> np.ndarray:
    """Softmax-weighted merge of each window of raw rows.

    [HCA] section 怎么压: the raw KV and a compression weight are computed per
    raw entry; each compressed entry is their sum weighted by a softmax of
    (weight + learnable position bias).  Here:

        a_ij  = z[i*s + j] + b[j]                  j = 0 .. w-1
        alpha = softmax_j(a_i.)
        y_i   = sum_j alpha_ij * x[i*s + j]        (every channel, K and V alike)

    z=None means all logits 0; b=None means zero bias.
    """
    x = np.asarray(x, dtype=np.float64)
    L, C = x.shape
    z = np.zeros(L) if z is None else np.asarray(z, dtype=np.float64)
    b = np.zeros(w) if b is None else np.asarray(b, dtype=np.float64)
    assert z.shape == (L,) and b.shape == (w,)
    N = n_entries(L, w, s)
    y = np.empty((N, C), dtype=np.float64)
    # Entries are independent; evaluate them in groups only to bound memory.
    group = max(1, (1 << 22) // max(1, w * C))
    offs = np.arange(w)
    for e0 in range(0, N, group):
        e1 = min(N, e0 + group)
        tok = (np.arange(e0, e1) * s)[:, None] + offs[None, :]  # [g][w] raw token ids
        a = z[tok] + b[None, :]
        a = a - a.max(axis=1, keepdims=True)
        alpha = np.exp(a)
        alpha /= alpha.sum(axis=1, keepdims=True)
        y[e0:e1] = np.einsum("gj,gjc->gc", alpha, x[tok])
    return y


def compress_channel_logits(x: np.ndarray, Z: np.ndarray, b: np.ndarray | None, w: int, s: int) -> np.ndarray:
    """Compression with one logit per raw token and channel.

    The variant of ``compress`` in which the compression weight is computed
    per channel ([HCA] section 怎么压 computes a compression weight for each
    raw entry and merges each window with a softmax over weight + position
    bias; here that weight is a vector, one value per channel):

        a_ijc  = Z[i*s + j][c] + b[j]
        alpha  = softmax over j of a_i.c           (separately for each c)
        y_ic   = sum_j alpha_ijc * x[i*s + j][c]

    x [L][C], Z [L][C] -> y [N][C].  b=None means zero bias.
    """
    x = np.asarray(x, dtype=np.float64)
    Z = np.asarray(Z, dtype=np.float64)
    L, C = x.shape
    assert Z.shape == (L, C)
    b = np.zeros(w) if b is None else np.asarray(b, dtype=np.float64)
    N = n_entries(L, w, s)
    y = np.empty((N, C), dtype=np.float64)
    group = max(1, (1 << 22) // max(1, w * C))
    offs = np.arange(w)
    for e0 in range(0, N, group):
        e1 = min(N, e0 + group)
        tok = (np.arange(e0, e1) * s)[:, None] + offs[None, :]  # [g][w]
        a = Z[tok] + b[None, :, None]  # [g][w][C]
        a = a - a.max(axis=1, keepdims=True)
        alpha = np.exp(a)
        alpha /= alpha.sum(axis=1, keepdims=True)
        y[e0:e1] = (alpha * x[tok]).sum(axis=1)
    return y


def compress_with_index(x, x_i, z, b, w: int, s: int):
    """Compressed K|V entries and the indexer keys of the same entries.

    The indexer keys K_I are not an independent input here: each entry's
    indexer key is the merge of the raw indexer keys of its window with the
    entry's own softmax weights ([TRDM] section 2.1: the indexer picks the
    most important compressed KV blocks, so it scores the entries that
    ``compress`` builds; [HCA] section 怎么压 for the weights).  x [L][C] K|V
    rows, x_i [L][d_I] raw indexer keys, per-token logits z [L].
    Returns (ckv [N][C], k_i [N][d_I]).
    """
    return compress(x, z, b, w, s), compress(x_i, z, b, w, s)


# ----------------------------------------------------------------------------
# 3. Lightning-indexer score and top-k
# ----------------------------------------------------------------------------


def index_scores(q_i: np.ndarray, keys: np.ndarray, w_i: np.ndarray) -> np.ndarray:
    """Indexer score of one query against a list of candidate keys.

    [HISA] section 01: the indexer scores every prefix candidate of a query and
    the top-k survive.  Score form (design choice; the pages print none):

        S[j] = sum_h w_i[h] * max(0, q_i[h] . keys[j])

    q_i [H_I][d_I], keys [n][d_I], w_i [H_I]  ->  S [n]
    """
    q_i = np.asarray(q_i, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    w_i = np.asarray(w_i, dtype=np.float64)
    dots = q_i @ keys.T  # [H_I][n]
    return w_i @ np.maximum(dots, 0.0)


def topk_select(scores: np.ndarray, n_valid: int, k: int) -> np.ndarray:
    """Positions of the k largest of scores[:n_valid], ascending, -1 padded.

    Order: larger score first, equal scores broken by the lower position
    (design choice).  Returns int64 [k].
    """
    scores = np.asarray(scores, dtype=np.float64)[:n_valid]
    pos = np.arange(n_valid)
    order = np.lexsort((pos, -scores))  # last key is primary: score descending
    chosen = np.sort(pos[order[: min(k, n_valid)]])
    out = np.full(k, -1, dtype=np.int64)
    out[: chosen.size] = chosen
    return out


def flat_topk(q_i, k_i, w_i, n_vis, k: int, return_scores: bool = False):
    """Flat (DSA-style) selection: score every visible entry, keep the top-k.

    [HISA] section 01 (the original token-level indexer scans the whole
    prefix).  q_i [nq][H_I][d_I], k_i [N][d_I], w_i [nq][H_I], n_vis [nq].
    Returns idx [nq][k] (and the selected scores, NaN where idx == -1).
    """
    nq = q_i.shape[0]
    idx = np.full((nq, k), -1, dtype=np.int64)
    sc = np.full((nq, k), np.nan)
    for q in range(nq):
        n = int(n_vis[q])
        s = index_scores(q_i[q], k_i[:n], w_i[q])
        pos = topk_select(s, n, k)
        idx[q] = pos
        sel = pos >= 0
        sc[q, sel] = s[pos[sel]]
    return (idx, sc) if return_scores else idx


# ----------------------------------------------------------------------------
# 4. HISA: hierarchical two-stage selection
# ----------------------------------------------------------------------------


def hisa_pool(k_i: np.ndarray, B: int) -> np.ndarray:
    """Block representatives: the mean of each run of B consecutive keys.

    [HISA] section 第一阶段 (block-level coarse filter): the prefix is cut into
    blocks of B, each summarised by one pooled vector.  A short last block is
    zero-padded, i.e. divided by B rather than by its own count (design choice).
    Returns float64 [ceil(N/B)][d_I].
    """
    k_i = np.asarray(k_i, dtype=np.float64)
    N, d = k_i.shape
    nb = -(-N // B)
    reps = np.zeros((nb, d))
    for blk in range(nb):
        reps[blk] = k_i[blk * B : min(N, blk * B + B)].sum(axis=0) / B
    return reps


def hisa_topk(q_i, k_i, w_i, n_vis, B: int, m: int, k: int, reps=None):
    """Two-stage HISA selection.

    [HISA] section 第一阶段: score each block representative with the query and
    keep the top-m blocks.  Section 第二阶段: run the token indexer only over
    the entries of those blocks and keep the top-k.  Section 05, Step 3: the
    result has the same form as the flat indexer's (k entry indices per
    query), so the attention downstream does not change.

    Readings: block b is a candidate iff its first entry is visible; entries
    of a chosen block that the query cannot see are not candidates; ties go
    to the lower block / lower entry.

    Returns (idx [nq][k], blk [nq][m]), both ascending and -1 padded.
    """
    k_i = np.asarray(k_i, dtype=np.float64)
    reps = hisa_pool(k_i, B) if reps is None else np.asarray(reps, dtype=np.float64)
    nq = q_i.shape[0]
    idx = np.full((nq, k), -1, dtype=np.int64)
    blk = np.full((nq, m), -1, dtype=np.int64)
    for q in range(nq):
        n = int(n_vis[q])
        nbq = -(-n // B)  # blocks whose first entry is visible
        r = index_scores(q_i[q], reps[:nbq], w_i[q])
        chosen = topk_select(r, nbq, m)
        blk[q] = chosen
        chosen = chosen[chosen >= 0]
        cand = (
            np.concatenate([np.arange(c * B, min(n, c * B + B)) for c in chosen])
            if chosen.size
            else np.zeros(0, dtype=np.int64)
        )
        s = index_scores(q_i[q], k_i[cand], w_i[q])
        pos = topk_select(s, cand.size, k)
        sel = pos >= 0
        idx[q, sel] = cand[pos[sel]]
    return idx, blk


def block_sparse_topk(q_i, k_i, w_i, n_vis, B: int, m: int, reps=None):
    """Block-sparse (MoBA/NSA-style) selection, the baseline HISA is compared with.

    [HISA] section 04: block-sparse methods choose at block granularity, and
    every token of a chosen block takes part in attention (HISA's block level
    is only a first filter before its token-level top-k).  Here the blocks are
    chosen exactly as HISA's first stage chooses them (same representatives,
    same block score, candidates are the blocks whose first entry is
    visible, ties to the lower block), and the selection is every visible
    entry of the m chosen blocks, so the attention budget is m*B entries.

    Returns (idx [nq][m*B], blk [nq][m]), both ascending and -1 padded.
    """
    k_i = np.asarray(k_i, dtype=np.float64)
    reps = hisa_pool(k_i, B) if reps is None else np.asarray(reps, dtype=np.float64)
    nq = q_i.shape[0]
    idx = np.full((nq, m * B), -1, dtype=np.int64)
    blk = np.full((nq, m), -1, dtype=np.int64)
    for q in range(nq):
        n = int(n_vis[q])
        nbq = -(-n // B)
        r = index_scores(q_i[q], reps[:nbq], w_i[q])
        chosen = topk_select(r, nbq, m)
        blk[q] = chosen
        chosen = chosen[chosen >= 0]
        ent = [e for c in chosen for e in range(c * B, min(n, c * B + B))]
        idx[q, : len(ent)] = ent
    return idx, blk


# ----------------------------------------------------------------------------
# 5. Attention
# ----------------------------------------------------------------------------


def window_rows(p: int, W: int) -> np.ndarray:
    """Raw rows of the sliding-window branch of a query at position p.

    [HCA] section 怎么压: besides the compressed entries, each query also
    attends to the most recent 128 raw tokens.  Here: max(0, p-W+1) .. p.
    """
    return np.arange(max(0, p - W + 1), p + 1)


def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float):
    """Softmax attention of H query heads over one shared K/V list (MQA).

    [HCA] section 怎么压: all query heads share one K/V (MQA).
    q [H][d], keys/vals [U][d] -> (o [H][d], lse [H]); lse = log sum exp.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    vals = np.asarray(vals, dtype=np.float64)
    logits = scale * (q @ keys.T)  # [H][U]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    den = e.sum(axis=1, keepdims=True)
    o = (e @ vals) / den
    lse = (mx + np.log(den))[:, 0]
    return o, lse


def _attend_union(q, ckv, entries, raw_kv, p, W, scale):
    d = q.shape[-1]
    rows = window_rows(p, W)
    keys = np.concatenate([ckv[entries, :d], raw_kv[rows, :d]])
    vals = np.concatenate([ckv[entries, d:], raw_kv[rows, d:]])
    return attend(q, keys, vals, scale)


def sparse_attention(q, ckv, idx, raw_kv, q_pos, W: int, scale: float):
    """CSA attention: each query attends to its selected entries plus its window.

    [HYB] section Compressed Sparse Attention and [HCA] section 怎么压.  One
    softmax runs over the union of {ckv[j] : j in idx[q], j != -1} and the
    window rows (design choice: no de-duplication).
    Returns (out [nq][H][d], lse [nq][H]).
    """
    ckv = np.asarray(ckv, dtype=np.float64)
    raw_kv = np.asarray(raw_kv, dtype=np.float64)
    nq, H, d = q.shape
    out = np.empty((nq, H, d))
    lse = np.empty((nq, H))
    for qi in range(nq):
        ent = np.asarray(idx[qi])
        ent = ent[ent >= 0]
        out[qi], lse[qi] = _attend_union(q[qi], ckv, ent, raw_kv, int(q_pos[qi]), W, scale)
    return out, lse


def dense_compressed_attention(q, ckv, n_vis, raw_kv, q_pos, W: int, scale: float):
    """HCA attention: each query attends to all its visible entries plus its window.

    [HCA] sections 128 倍是什么概念 and 怎么压: no selection; every query looks
    at every compressed entry it may see, with the same window branch.
    """
    ckv = np.asarray(ckv, dtype=np.float64)
    raw_kv = np.asarray(raw_kv, dtype=np.float64)
    nq, H, d = q.shape
    out = np.empty((nq, H, d))
    lse = np.empty((nq, H))
    for qi in range(nq):
        ent = np.arange(int(n_vis[qi]))
        out[qi], lse[qi] = _attend_union(q[qi], ckv, ent, raw_kv, int(q_pos[qi]), W, scale)
    return out, lse


def csa2_layer_group(q, raw_kv, raw_ki, z, b, q_i, w_i, q_pos, k: int, W: int, w: int, s: int, scale: float):
    """CSA2 (V4.1-Flash) for a group of layers that share one global cache.

    [HCA] section V4.1 为什么不要它了: V4.1 keeps a single global branch,
    one compression level plus cross-layer sharing, and every query sees the
    global context only through a top-512 selection, beside the 128-token
    sliding window.  Here (readings: the compression is ``compress`` at the
    group's one rate, w = 2s as for CSA, or w = s = 1 for an uncompressed
    cache; the indexer keys are compressed from raw indexer keys with the
    entries' own weights; the group of layers shares the cache, the
    visibility and the selected indices, and each layer has its own
    queries):

        ckv, K_I = compress_with_index(raw_kv, raw_ki, z, b, w, s)
        idx      = flat_topk(q_i, K_I, w_i, n_vis, k)            once per group
        out[g]   = sparse_attention(q[g], ckv, idx, raw_kv, q_pos, W, scale)

    q [G][nq][H][d] (layer g's queries), raw_kv [L][2d], raw_ki [L][d_I],
    z [L] per-token logits, q_i [nq][H_I][d_I], w_i [nq][H_I].
    Returns (out [G][nq][H][d], lse [G][nq][H], idx [nq][k]).
    """
    ckv, k_i = compress_with_index(raw_kv, raw_ki, z, b, w, s)
    N = ckv.shape[0]
    n_vis = np.array([n_visible(int(p), w, s, N) for p in q_pos])
    idx = flat_topk(q_i, k_i, w_i, n_vis, k)
    outs, lses = [], []
    for g in range(q.shape[0]):
        o, lse = sparse_attention(q[g], ckv, idx, raw_kv, q_pos, W, scale)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses), idx


def lse_merge(outs, lses):
    """Combine attention over disjoint key lists from their (o, lse) pairs.

    o = sum_s exp(lse_s - lse) * o_s with lse = log sum_s exp(lse_s).  This
    is an identity of softmax, used to check the split-key design.
    """
    lses = np.stack([np.asarray(x, dtype=np.float64) for x in lses])  # [S][...]
    outs = np.stack([np.asarray(x, dtype=np.float64) for x in outs])  # [S][...][d]
    mx = lses.max(axis=0)
    wts = np.exp(lses - mx)
    lse = mx + np.log(wts.sum(axis=0))
    o = (np.exp(lses - lse)[..., None] * outs).sum(axis=0)
    return o, lse
