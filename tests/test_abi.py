"""C-ABI checks that need no GPU: the library loads, exports every function
include/hattn.h declares, and rejects bad arguments before launching."""
import ctypes
import os
import re

import pytest

from compressed_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "hattn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hattn_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libhattn.so is not built (run __graft_entry__.build())")
    return _lib.lib()


def test_exports_match_header(L):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
        assert n in _lib.SIGNATURES, f"{n} has no binding signature"


def test_status_strings(L):
    for s in range(5):
        assert L.hattn_status_string(s).startswith(b"HATTN_")
    assert L.hattn_abi_version() == _lib.ABI_VERSION


def test_compress_validation(L):
    f = L.hattn_compress
    assert f(7, None, 1, 100, 256, None, None, 8, 4, 0, 1, None, None) == 1
    assert f(1, None, 1, 100, 250, None, None, 8, 4, 0, 1, None, None) == 1  # C not multiple of 8
    assert f(0, None, 1, 100, 6, None, None, 8, 4, 0, 1, None, None) == 1    # fp32 C not multiple of 4
    assert f(1, None, 1, 5, 256, None, None, 8, 4, 0, 1, None, None) == 1    # L < w
    assert f(1, None, 1, 100, 256, None, None, 8, 4, 0, 30, None, None) == 1  # e_end > N = 24
    assert f(1, None, 1, 100, 256, None, None, 0, 4, 0, 1, None, None) == 1  # w = 0
    assert f(1, None, 1, 100, 256, None, None, 8, 4, 0, 1, None, None) == 1  # NULL x
    assert b"NULL" in L.hattn_last_error()
    assert f(1, None, 0, 100, 256, None, None, 8, 4, 0, 24, None, None) == 0  # bt = 0: nothing to do
    # vector-accessed arrays must be 16-byte aligned (checked before any launch)
    assert f(1, ctypes.c_void_p(20), 1, 100, 256, None, None, 8, 4, 0, 1, ctypes.c_void_p(32), None) == 1
    assert b"aligned" in L.hattn_last_error()


def test_decode_append_validation(L):
    f = L.hattn_decode_append
    p = ctypes.c_void_p(16)
    args = lambda **kw: [kw.get(n, d) for n, d in [
        ("dt", 1), ("x", p), ("bt", 2), ("L", 100), ("R", 0), ("C", 256), ("z", None), ("b", None), ("w", 8), ("s", 4),
        ("qp", p), ("y", p), ("nv", p), ("ki", None), ("di", 0), ("B", 0), ("reps", None), ("st", None)]]
    assert f(*args(dt=5)) == 1
    assert f(*args(C=250)) == 1                      # not a multiple of 8 bf16 elements
    assert f(*args(C=4096)) == 1                     # more than 256 16-byte slots
    assert f(*args(w=0)) == 1
    assert f(*args(w=5000, L=6000)) == 1             # window above 4096
    assert f(*args(s=0)) == 1
    assert f(*args(L=7)) == 1                        # shorter than the window
    assert f(*args(ki=p)) == 1                       # k_i without reps
    assert f(*args(ki=p, reps=p, di=128, B=0)) == 1  # B = 0
    assert f(*args(ki=p, reps=p, di=12, B=16)) == 1  # d_i not a multiple of 8
    assert f(*args(y=None)) == 1
    assert b"NULL" in L.hattn_last_error()
    assert f(*args(bt=0, x=None, qp=None, y=None, nv=None)) == 0  # nothing to do
    # a ring of raw rows must hold the window and no more than L rows
    assert f(*args(R=4)) == 1
    assert b"ring" in L.hattn_last_error()
    assert f(*args(R=101)) == 1
    assert f(*args(R=-1)) == 1
    assert f(*args(R=8, bt=0, x=None, qp=None, y=None, nv=None)) == 0


def _sz():
    return ctypes.c_size_t(0)


def test_index_topk_validation_and_size_query(L):
    p = ctypes.c_void_p(16)  # never dereferenced: every call below returns before launching
    sz = _sz()
    # bad k, bad heads, NULL pointer
    assert L.hattn_index_topk(1, p, p, p, p, 1, 4, 16, 128, 1000, 0, p, None, None, ctypes.byref(sz), None) == 1
    assert L.hattn_index_topk(1, p, p, p, p, 1, 4, 16, 128, 1000, 9000, p, None, None, ctypes.byref(sz), None) == 1
    assert L.hattn_index_topk(1, p, p, p, p, 1, 4, 65, 128, 1000, 8, p, None, None, ctypes.byref(sz), None) == 1
    assert L.hattn_index_topk(1, None, p, p, p, 1, 4, 16, 128, 1000, 8, p, None, None, ctypes.byref(sz), None) == 1
    # size query: rows * round4(n) * 4 bytes of scores (n below the LDS cap)
    assert L.hattn_index_topk(1, p, p, p, p, 2, 8, 16, 128, 1000, 8, p, None, None, ctypes.byref(sz), None) == 0
    assert sz.value >= 16 * 1000 * 4
    # a long row needs candidate lists too
    big = _sz()
    assert L.hattn_index_topk(1, p, p, p, p, 1, 1, 16, 128, 131072, 2048, p, None, None, ctypes.byref(big), None) == 0
    assert big.value > 131072 * 4
    # too small a workspace, or none at all
    small = ctypes.c_size_t(sz.value - 1)
    assert L.hattn_index_topk(1, p, p, p, p, 2, 8, 16, 128, 1000, 8, p, None, p, ctypes.byref(small), None) == 3
    assert L.hattn_index_topk(1, p, p, p, p, 2, 8, 16, 128, 1000, 8, p, None, None, None, None) == 3


def test_hisa_validation(L):
    p = ctypes.c_void_p(16)
    sz = _sz()
    assert L.hattn_hisa_topk(1, p, p, p, p, 1, 4, 16, 128, 4096, p, 128, 200, 64, p, None, None,
                             ctypes.byref(sz), None) == 1  # m*B > 16384
    assert L.hattn_hisa_topk(1, p, p, p, p, 1, 4, 16, 128, 4096, None, 128, 8, 64, p, None, None,
                             ctypes.byref(sz), None) == 1  # NULL reps
    assert L.hattn_hisa_topk(1, p, p, p, p, 1, 4, 16, 128, 4096, p, 128, 8, 64, p, None, None,
                             ctypes.byref(sz), None) == 0 and sz.value > 0
    assert L.hattn_hisa_pool(1, p, 1, 100, 12, 16, 0, 7, p, None) == 1  # d_i not multiple of 8
    assert L.hattn_hisa_pool(1, p, 1, 100, 16, 16, 0, 8, p, None) == 1  # block range past ceil(100/16) = 7


def test_attention_validation(L):
    p = ctypes.c_void_p(16)
    sz = _sz()
    f = L.hattn_dense_compressed_attn
    # arguments: dtype q ckv n n_vis raw_kv L raw_rows q_pos window scale bt nq h d out lse ws ws_bytes stream
    assert f(1, p, p, 100, p, p, 1000, 0, p, 0, 0.1, 1, 1, 64, 128, p, None, None, ctypes.byref(sz), None) == 1  # window
    assert f(1, p, p, 100, p, p, 1000, 0, p, 128, -1.0, 1, 1, 64, 128, p, None, None, ctypes.byref(sz), None) == 1
    assert f(1, p, p, 100, p, p, 1000, 0, p, 128, 0.1, 1, 1, 64, 12, p, None, None, ctypes.byref(sz), None) == 1
    assert f(1, p, p, 100, None, p, 1000, 0, p, 128, 0.1, 1, 1, 64, 128, p, None, None, ctypes.byref(sz), None) == 1
    assert f(1, p, p, 100, p, p, 1000, 0, p, 128, 0.1, 1, 1, 2048, 128, p, None, None, ctypes.byref(sz), None) == 2
    # long key lists are split: the partials need a workspace
    assert f(1, p, p, 8192, p, p, 1 << 20, 0, p, 128, 0.1, 32, 1, 64, 128, p, None, None, ctypes.byref(sz), None) == 0
    assert sz.value > 0
    # a raw ring must hold at least the window and at most L rows
    assert f(1, p, p, 8192, p, p, 1 << 20, 127, p, 128, 0.1, 32, 1, 64, 128, p, None, None, ctypes.byref(sz),
             None) == 1
    assert b"ring" in L.hattn_last_error()
    assert f(1, p, p, 100, p, p, 1000, 1001, p, 128, 0.1, 1, 1, 64, 128, p, None, None, ctypes.byref(sz), None) == 1
    assert f(1, p, p, 100, p, p, 1000, -1, p, 128, 0.1, 1, 1, 64, 128, p, None, None, ctypes.byref(sz), None) == 1
    assert f(1, p, p, 8192, p, p, 1 << 20, 1 << 40, p, 128, 0.1, 32, 1, 64, 128, p, None, None, ctypes.byref(sz),
             None) == 1
    assert f(1, p, p, 8192, p, p, 1 << 20, 128, p, 128, 0.1, 32, 1, 64, 128, p, None, None, ctypes.byref(sz),
             None) == 0
    g = L.hattn_sparse_attn
    assert g(1, p, p, 100, None, 8, p, 1000, 0, p, 128, 0.1, 1, 1, 64, 128, p, None, None, ctypes.byref(sz), None) == 1
    assert g(1, p, p, 100, p, 8, p, 1000, 64, p, 128, 0.1, 1, 1, 64, 128, p, None, None, ctypes.byref(sz), None) == 1
    assert g(1, p, p, 100, p, 8, p, 1000, 200, p, 128, 0.1, 1, 1, 64, 128, p, None, None, ctypes.byref(sz), None) == 0
    n = L.hattn_sparse_attn_noalloc
    assert n(1, p, p, 100, p, 8, p, 1000, 64, p, 128, ctypes.c_float(0.1), 1, 1, 64, 128, p, None, None) == 1
    assert b"ring" in L.hattn_last_error()


def test_decode_plan_validation(L):
    from compressed_attention_amd._lib import DecodeDesc
    assert L.hattn_decode_desc_size() == ctypes.sizeof(DecodeDesc)
    plan = ctypes.c_void_p()
    sz = ctypes.c_size_t(0)
    assert L.hattn_decode_plan_create(None, ctypes.byref(plan)) == 1
    assert L.hattn_decode_plan_ws_bytes(None, ctypes.byref(sz)) == 1
    p = ctypes.c_void_p(256)
    d = DecodeDesc(dtype=1, h=64, d=128, window=128, bt=2, L=4096, scale=0.088, h_i=16, d_i=128, B=128, m=8, k=64,
                   csa_w=8, csa_stride=4, hca_w=128, hca_stride=128, q_pos=p, csa_raw_kv=p, csa_ckv=p, k_i=p,
                   reps=p, q_i=p, w_i=p, csa_q=p, csa_out=p, hca_raw_kv=p, hca_ckv=p, hca_q=p, hca_out=p)
    assert L.hattn_decode_plan_ws_bytes(ctypes.byref(d), ctypes.byref(sz)) == 0 and sz.value > 0
    d.k_i = None  # the CSA branch needs the indexer keys and block means
    d.reps = None
    assert L.hattn_decode_plan_ws_bytes(ctypes.byref(d), ctypes.byref(sz)) == 1
    d.k_i, d.reps = p, p
    d.bt = 0
    assert L.hattn_decode_plan_ws_bytes(ctypes.byref(d), ctypes.byref(sz)) == 1
    d.bt = 2
    d.csa_w = 0
    assert L.hattn_decode_plan_ws_bytes(ctypes.byref(d), ctypes.byref(sz)) == 1
    d.csa_w = 8
    d.csa_q = ctypes.c_void_p(264)  # misaligned
    assert L.hattn_decode_plan_ws_bytes(ctypes.byref(d), ctypes.byref(sz)) == 1
    assert b"aligned" in L.hattn_last_error()
    d.csa_q = p
    # raw rings: at least the window and both compression windows, at most L rows
    for rows, ok in ((128, True), (4096, True), (64, False), (127, False), (4097, False), (-1, False)):
        d.raw_rows = rows
        st = L.hattn_decode_plan_ws_bytes(ctypes.byref(d), ctypes.byref(sz))
        assert (st == 0) == ok, (rows, st, L.hattn_last_error())
        if not ok:
            assert b"raw_rows" in L.hattn_last_error() or b"ring" in L.hattn_last_error()
    d.hca_w, d.hca_stride, d.raw_rows = 256, 256, 128  # the HCA window does not fit the ring
    assert L.hattn_decode_plan_ws_bytes(ctypes.byref(d), ctypes.byref(sz)) == 1
    d.hca_w, d.hca_stride, d.raw_rows = 128, 128, 0
    d.ws, d.ws_bytes = p, 16  # too small: refused before any device work
    assert L.hattn_decode_plan_create(ctypes.byref(d), ctypes.byref(plan)) == 3
    assert L.hattn_decode_plan_destroy(None) == 0
    assert L.hattn_decode_plan_run(None, None) == 1
    assert L.hattn_decode_plan_run_graph(None, None) == 1


def test_sparse_attn_noalloc_rejects_oversize(L):
    # 600 bf16 queries with 30,000 + 128 keys split in 15 chunks of 2,048
    # need 600 * 15 * 64 * 128 * 2 bytes (147 MB) of fp16 partials, more than
    # the 32 MiB static scratch: refused before any launch.
    f = L.hattn_sparse_attn_noalloc
    p = ctypes.c_void_p(256)
    st = f(1, p, p, 4000, p, 30000, p, 9000, 0, p, 128, ctypes.c_float(0.088), 1, 600, 64, 128, p, None, None)
    assert st == 3, L.hattn_last_error()
    assert b"static" in L.hattn_last_error()
    # the same call with a workspace would need more than 32 MiB
    sz = ctypes.c_size_t(0)
    assert L.hattn_sparse_attn(1, p, p, 4000, p, 30000, p, 9000, 0, p, 128, ctypes.c_float(0.088), 1, 600, 64, 128,
                               p, None, None, ctypes.byref(sz), None) == 0
    assert sz.value > 32 << 20


def test_empty_shapes_launch_nothing(L):
    # With no rows (bt * nq == 0) every compute call asks for no workspace,
    # accepts NULL buffers and returns HATTN_OK without touching a device.
    f32 = ctypes.c_float(0.088)
    sz = ctypes.c_size_t(123)
    assert L.hattn_index_topk(1, None, None, None, None, 0, 4, 16, 128, 1000, 8, None, None, None,
                              ctypes.byref(sz), None) == 0 and sz.value == 0
    assert L.hattn_index_topk(1, None, None, None, None, 2, 0, 16, 128, 1000, 8, None, None, None, None, None) == 0
    sz.value = 123
    assert L.hattn_hisa_topk(1, None, None, None, None, 2, 0, 16, 128, 4096, None, 128, 8, 64, None, None, None,
                             ctypes.byref(sz), None) == 0 and sz.value == 0
    sz.value = 123
    assert L.hattn_block_sparse_topk(1, None, None, None, None, 0, 4, 16, 128, 4096, None, 128, 8, None, None, None,
                                     ctypes.byref(sz), None) == 0 and sz.value == 0
    assert L.hattn_hisa_pool(1, None, 0, 100, 16, 16, 0, 7, None, None) == 0
    assert L.hattn_hisa_pool(1, None, 2, 100, 16, 16, 3, 3, None, None) == 0  # empty block range
    assert L.hattn_visible_count(None, 0, 8, 4, 1023, None, None) == 0
    for bt, nq in ((0, 1), (3, 0)):
        sz.value = 123
        assert L.hattn_sparse_attn(1, None, None, 100, None, 8, None, 1000, 0, None, 128, f32, bt, nq, 64, 128,
                                   None, None, None, ctypes.byref(sz), None) == 0 and sz.value == 0
        sz.value = 123
        assert L.hattn_dense_compressed_attn(1, None, None, 100, None, None, 1000, 0, None, 128, f32, bt, nq, 64, 128,
                                             None, None, None, ctypes.byref(sz), None) == 0 and sz.value == 0
        assert L.hattn_sparse_attn_noalloc(1, None, None, 100, None, 8, None, 1000, 0, None, 128, f32, bt, nq, 64,
                                           128, None, None, None) == 0
    assert L.hattn_last_error() == b""
