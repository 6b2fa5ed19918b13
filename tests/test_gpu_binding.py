"""The binding refuses buffers whose shape or device disagrees with the call
before anything is launched: the library sees only addresses, so a short
output or cache would otherwise be written out of bounds."""
import pytest
import torch

from compressed_attention_amd import ops, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _attn_inputs(bt=2, nq=3, h=64, d=128, n=300, L=500, k=32):
    dt = torch.bfloat16
    q = synth.normal((bt, nq, h, d), 901, dtype=dt).to(DEV)
    ckv = synth.normal((bt, n, 2 * d), 902, dtype=dt).to(DEV)
    raw = synth.normal((bt, L, 2 * d), 903, dtype=dt).to(DEV)
    pos = torch.full((bt, nq), L - 1, dtype=torch.int32, device=DEV)
    nv = torch.full((bt, nq), n, dtype=torch.int32, device=DEV)
    idx = torch.arange(k, dtype=torch.int32, device=DEV).repeat(bt, nq, 1)
    return q, ckv, raw, pos, nv, idx


def test_attention_rejects_mismatched_buffers():
    q, ckv, raw, pos, nv, idx = _attn_inputs()
    bt, nq, h, d = q.shape
    with pytest.raises(ValueError, match="n_vis"):
        ops.dense_compressed_attn(q, ckv, nv[:, :2].contiguous(), raw, pos, 128)
    with pytest.raises(ValueError, match="out"):
        ops.sparse_attn_noalloc(q, ckv, idx, raw, pos, 128,
                                out=torch.empty((bt, nq, h // 2, d), dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError, match="lse"):
        ops.sparse_attn_noalloc(q, ckv, idx, raw, pos, 128,
                                out=torch.empty((bt, nq, h, d), dtype=torch.float32, device=DEV),
                                lse=torch.empty((bt, nq, 1), dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError, match="idx"):
        ops.sparse_attn(q, ckv, idx.cpu(), raw, pos, 128)
    with pytest.raises(ValueError, match="CUDA"):
        ops.sparse_attn(q, ckv.cpu(), idx, raw, pos, 128)


def test_cache_ops_reject_mismatched_buffers():
    bt, L, C, w, s = 2, 64, 256, 8, 4
    x = synth.normal((bt, L, C), 911, dtype=torch.bfloat16).to(DEV)
    z = synth.normal((bt, L), 912).to(DEV)
    N = (L - w) // s + 1
    with pytest.raises(ValueError, match="pos_bias"):
        ops.compress_channel_logits(x, torch.zeros((bt, L, C), device=DEV), torch.zeros(w - 1, device=DEV), w, s)
    with pytest.raises(ValueError, match="out"):
        ops.compress_with_index(x, x[..., :32].contiguous(), z, None, w, s,
                                out=torch.empty((bt, N - 1, C), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="logits"):
        ops.compress_with_index(x, x[..., :32].contiguous(), z[:, :-1].contiguous(), None, w, s)
    k_i = synth.normal((bt, 1000, 128), 913, dtype=torch.bfloat16).to(DEV)
    with pytest.raises(ValueError, match="out"):
        ops.hisa_pool(k_i, 128, out=torch.empty((bt, 7, 128), dtype=torch.float32, device=DEV))
    pos = torch.tensor([5, 9], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="out"):
        ops.visible_count(pos, w, s, N, out=torch.empty(1, dtype=torch.int32, device=DEV))
    ckv = torch.empty((bt, N, C), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="logits"):
        ops.decode_append(x, z[:, :10].contiguous(), None, w, s, pos.reshape(bt, 1), ckv)
    with pytest.raises(ValueError, match="n_vis"):
        ops.decode_append(x, z, None, w, s, pos.reshape(bt, 1), ckv,
                          n_vis=torch.empty((bt, 2), dtype=torch.int32, device=DEV))


def test_decode_plan_rejects_mismatched_caches():
    bt, L, h, d, h_i, d_i, B = 2, 1024, 64, 128, 16, 128, 128
    dt = torch.bfloat16
    n_csa, n_hca = (L - 8) // 4 + 1, L // 128

    def t(*shape, dtype=dt):
        return torch.zeros(shape, dtype=dtype, device=DEV)

    args = dict(q_pos=t(bt, 1, dtype=torch.int32), csa_raw_kv=t(bt, L, 2 * d), csa_logits=None, csa_pos_bias=None,
                csa_ckv=t(bt, n_csa, 2 * d), k_i=t(bt, n_csa, d_i), reps=t(bt, -(-n_csa // B), d_i, dtype=torch.float32),
                q_i=t(bt, 1, h_i, d_i), w_i=t(bt, 1, h_i, dtype=torch.float32), csa_q=t(bt, 1, h, d),
                hca_raw_kv=t(bt, L, 2 * d), hca_logits=None, hca_pos_bias=None, hca_ckv=t(bt, n_hca, 2 * d),
                hca_q=t(bt, 1, h, d), B=B, m=4, k=128)
    for name, bad in [("csa_ckv", t(bt, n_csa - 1, 2 * d)), ("hca_ckv", t(bt, n_hca + 1, 2 * d)),
                      ("k_i", t(bt, n_csa, d_i // 2)), ("reps", t(bt, 1, d_i, dtype=torch.float32)),
                      ("csa_logits", t(bt, L - 1, dtype=torch.float32)),
                      ("hca_pos_bias", t(127, dtype=torch.float32))]:
        with pytest.raises(ValueError, match=name):
            ops.DecodePlan(**{**args, name: bad})
    with pytest.raises(TypeError, match="k_i"):
        ops.DecodePlan(**{**args, "k_i": t(bt, n_csa, d_i, dtype=torch.float32)})
