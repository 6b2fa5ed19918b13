"""Comparison helpers shared by the GPU parity tests (no method arithmetic)."""
import numpy as np
import torch


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def bf16_half_ulp(v):
    """Half a bf16 unit in the last place at |v| (8-bit significand)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def assert_bf16_close(gpu, ref, extra_abs=2e-5, extra_rel=2e-5):
    """|gpu - ref| <= half a bf16 ulp (one final rounding) + fp32 accumulation slack."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    tol = np.maximum(bf16_half_ulp(ref), bf16_half_ulp(gpu)) + extra_abs + extra_rel * np.abs(ref)
    bad = np.abs(gpu - ref) > tol
    assert not bad.any(), f"{bad.sum()} of {bad.size} outside bf16 tolerance; worst {np.abs(gpu - ref).max():.3g}"


def iou_rows(a, b):
    """Mean and min IoU over rows of two -1-padded index lists."""
    vals = []
    for ra, rb in zip(np.asarray(a), np.asarray(b)):
        sa, sb = set(int(x) for x in ra if x >= 0), set(int(x) for x in rb if x >= 0)
        u = sa | sb
        vals.append(1.0 if not u else len(sa & sb) / len(u))
    return float(np.mean(vals)), float(np.min(vals))


def check_near_ties(gpu_idx, ora_idx, ora_scores_row_fn, tol_fn):
    """Where two selections differ, every differing element must sit at the
    selection boundary: its oracle score within tol of the k-th largest."""
    for r, (ga, oa) in enumerate(zip(np.asarray(gpu_idx), np.asarray(ora_idx))):
        sg, so = set(int(x) for x in ga if x >= 0), set(int(x) for x in oa if x >= 0)
        if sg == so:
            continue
        assert len(sg) == len(so), (r, len(sg), len(so))
        scores = ora_scores_row_fn(r)
        thr = min(scores[i] for i in so)
        tol = tol_fn(r)
        for i in sg ^ so:
            assert abs(scores[i] - thr) <= tol, (r, i, scores[i], thr, tol)
