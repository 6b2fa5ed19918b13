"""The shared input generator: reproducible, bf16 rounding is RNE, stated shapes."""
import numpy as np
import torch

from compressed_attention_amd import synth


def test_reproducible_and_independent_streams():
    a = synth.tiny_hybrid_layer(0).tensors
    b = synth.tiny_hybrid_layer(0).tensors
    for k in a:
        assert torch.equal(a[k], b[k]), k
    c = synth.tiny_hybrid_layer(1).tensors
    assert not torch.equal(a["raw_kv"], c["raw_kv"])
    # different names draw from different streams
    assert not torch.equal(a["raw_kv"].reshape(-1)[:512], a["q"].reshape(-1)[:512])


def test_bf16_rounding_is_round_to_nearest_even():
    x = torch.tensor([1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -(1.0 + 2**-8)], dtype=torch.float32)
    y = x.to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(y, [1.0, 1.0 + 2**-6, 1.0 + 2**-7, -1.0])


def test_integer_grid_and_dyadic_weights():
    w = synth.tiny_hybrid_layer(0).tensors
    qi = w["q_i"].numpy()
    assert qi.min() >= -8 and qi.max() <= 8 and np.all(qi == np.round(qi))
    wi = w["w_i"].numpy() * 256
    assert np.all(wi == np.round(wi)) and wi.min() >= 0 and wi.max() <= 255
    assert list(w["q_pos"][0, :3]) == [2048, 2080, 2112] and int(w["q_pos"][0, -1]) == 2048 + 32 * 63


def test_tiled_bias_and_index_lists():
    b = synth.tiled_bias(4, 8, 5)
    assert torch.equal(b[:4], b[4:])
    idx = synth.random_index_lists([0, 3, 100], 8, seed=3)
    assert list(idx[0]) == [-1] * 8 and list(idx[1]) == [0, 1, 2, -1, -1, -1, -1, -1]
    row = idx[2].tolist()
    assert row == sorted(row) and len(set(row)) == 8 and max(row) < 100


def test_needles_are_scaled_rows():
    w = synth.indexer_128k(0, N=4096, nq=8, n_needles=16)
    k = w.tensors["k_i"][0].float()
    norms = k.norm(dim=1)
    needles = w.tensors["needles"]
    assert needles.numel() == 16 and len(set(needles.tolist())) == 16
    assert norms[needles].mean() > 3.0 * norms.mean()
