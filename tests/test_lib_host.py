"""CPU-side checks of the C-ABI library: it loads, exports every symbol that
include/msa.h declares, and its host logic (chunk plan, argument validation,
workspace sizing) behaves as documented. No GPU compute is launched here:
every validation case below fails before anything is enqueued."""
import ctypes
import os
import re
import struct

import numpy as np
import pytest

import routed_sparse_attention_amd as msa
from oracle import msa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "msa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(msa.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = msa.lib()
    for name in _declared():
        assert hasattr(L, name), f"libmsa.so does not export {name}"
    assert L.msa_abi_version() == 6


def test_default_dims_follow_the_pages():
    d = msa.dims()
    assert (d.n_kv_heads, d.n_router_heads, d.head_dim, d.chunk, d.top_k) == \
        (O.N_KV_HEADS, O.N_ROUTER_HEADS, O.HEAD_DIM, O.CHUNK, O.TOP_K)
    assert d.n_q_heads == 32 and d.rope_theta == 1e6 and d.token_reduce == 0 and d.doc_rope_mode == 0


def test_plan_chunks_matches_oracle():
    rng = np.random.default_rng(3)
    for chunk in (1, 7, 64, 100):
        lengths = rng.integers(1, 500, size=200)
        offs = np.concatenate([[0], np.cumsum(lengths)])
        assert np.array_equal(msa.plan_chunks(offs, chunk), O.plan_chunks(offs, chunk))


def test_plan_chunks_rejects_empty_document():
    with pytest.raises(msa.MsaError) as e:
        msa.plan_chunks(np.array([0, 3, 3, 9]))
    assert e.value.code == -2 and "document 1" in str(e.value)


def _route(d, B=1, M=1, n_docs=4, n_chunks=8, ptr=16, accumulate=0, ws_bytes=0):
    L = msa.lib()
    p = ctypes.c_void_p(ptr)
    return L.msa_route_topk(ctypes.byref(d), p, B, M, p, p, n_docs, n_chunks, p, accumulate, p, p, p,
                            p, ws_bytes, None)


def test_validation_codes():
    L = msa.lib()
    assert _route(msa.dims(head_dim=64)) == -5
    assert b"head_dim" in L.msa_last_error()
    assert _route(msa.dims(n_q_heads=30)) == -2
    assert _route(msa.dims(top_k=0)) == -2
    assert _route(msa.dims(token_reduce=3)) == -1
    assert _route(msa.dims(rope_theta=float("nan"))) == -1
    assert _route(msa.dims(), B=0) == -2
    assert _route(msa.dims(), n_docs=9, n_chunks=8) == -2
    assert _route(msa.dims(), ptr=0) == -1
    assert _route(msa.dims(token_reduce=1), accumulate=1) == -5
    assert _route(msa.dims(), ws_bytes=0) == -3       # the workspace check precedes any launch
    d = msa.dims()
    p = ctypes.c_void_p(16)
    rc = L.msa_sparse_attend(ctypes.byref(d), p, 5, p, p, 4, 0, p, p, 0, 8, p, 2, p, p, 8, -1, p,
                             None, p, 1 << 30, None)
    assert rc == -2 and b"M_loc" in L.msa_last_error()
    rc = L.msa_encode_pool(ctypes.byref(d), p, p, p, p, p, 3, 2, 3, p, p, p, None, 0, None)
    assert rc == -2
    rc = L.msa_encode_pool(ctypes.byref(d), None, p, p, p, p, 1, 2, 1, p, None, None, None, 0, None)
    assert rc == -1


def test_workspace_sizes():
    d = msa.dims()
    a = msa.route_topk_workspace(1, 1, 1_562_500, 46_000, d)
    b = msa.route_topk_workspace(64, 1, 250_000, 7_350, d)
    assert a >= 1_562_500 * 4 and b >= 64 * 250_000 * 4
    assert msa.sparse_attend_workspace(1, 129, 1024, d) > 0
    assert msa.lib().msa_route_topk_workspace(ctypes.byref(d), 0, 1, 10, 2) == 0


def _header(n_docs=3, chunk=64, n_chunks=7, heads=8, head_dim=128, mask=7, magic=b"MSASTOR1",
            version=1, hbytes=64):
    return struct.pack("<8sIIiiqiiIif12x", magic, version, hbytes, n_docs, chunk, n_chunks, heads,
                       head_dim, mask, 0, 1e6)


def test_store_header_layout_is_64_bytes():
    assert len(_header()) == 64


def test_store_file_info_reads_the_header(tmp_path):
    f = tmp_path / "ok.msastore"
    f.write_bytes(_header(n_docs=5, n_chunks=11, mask=5) + bytes(48))
    assert msa.store_file_info(str(f)) == (5, 11, 5)


@pytest.mark.parametrize("kw,why", [
    (dict(magic=b"NOTSTORE"), "bad magic"),
    (dict(version=2), "unsupported version"),
    (dict(hbytes=80), "unsupported version"),
    (dict(n_docs=4, n_chunks=3), "malformed"),
    (dict(mask=9), "malformed"),
    (dict(chunk=0), "malformed"),
])
def test_store_file_info_rejects_malformed_headers(tmp_path, kw, why):
    f = tmp_path / "bad.msastore"
    f.write_bytes(_header(**kw))
    with pytest.raises(msa.MsaError) as e:
        msa.store_file_info(str(f))
    assert e.value.code == -6 and why in str(e.value)


def test_store_file_info_io_errors(tmp_path):
    with pytest.raises(msa.MsaError) as e:
        msa.store_file_info(str(tmp_path / "missing"))
    assert e.value.code == -6
    f = tmp_path / "short"
    f.write_bytes(_header()[:40])
    with pytest.raises(msa.MsaError) as e:
        msa.store_file_info(str(f))
    assert e.value.code == -6 and "header" in str(e.value)


def test_store_validation_before_any_gpu_work():
    """Store calls reject bad arguments before touching the GPU."""
    L = msa.lib()
    d = msa.dims()
    dco_h = (ctypes.c_int64 * 5)(0, 2, 5, 0, 0)
    st = msa._lib.StoreC(None, None, None, 16, ctypes.addressof(dco_h), 10, 4, 2, 5)
    dto_h = (ctypes.c_int64 * 3)(0, 100, 180)
    p = ctypes.c_void_p(16)
    # one 700-token document is 11 chunks; the store has room for 10 - 5
    big = (ctypes.c_int64 * 2)(0, 700)
    rc = L.msa_store_append(ctypes.byref(d), ctypes.byref(st), p, p, p, p, big, 1, 700, None)
    assert rc == -2 and b"do not fit" in L.msa_last_error() and st.n_docs == 2
    rc = L.msa_store_append(ctypes.byref(d), ctypes.byref(st), p, p, p, p, dto_h, 2, 999, None)
    assert rc == -2 and b"run from 0" in L.msa_last_error()
    bad = (ctypes.c_int64 * 3)(0, 100, 100)
    rc = L.msa_store_append(ctypes.byref(d), ctypes.byref(st), p, p, p, p, bad, 2, 100, None)
    assert rc == -2 and b"document 1" in L.msa_last_error()
    st.n_chunks = 4   # mirror ends at 5: inconsistent fill
    rc = L.msa_store_append(ctypes.byref(d), ctypes.byref(st), p, p, p, p, dto_h, 2, 180, None)
    assert rc == -2 and b"not at n_chunks" in L.msa_last_error()
    st.n_chunks = 5
    rc = L.msa_store_save(ctypes.byref(d), ctypes.byref(st), b"/tmp/x", None, 0)
    assert rc == -1 and b"staging" in L.msa_last_error()


def test_attend_batch_validation_and_workspace():
    """msa_sparse_attend_batch checks its arguments on the host like
    msa_sparse_attend (an empty batch, a context shorter than the query, too
    small a workspace) and touches no device memory; its workspace grows with
    the batch, one query's equal to msa_sparse_attend's."""
    L = msa.lib()
    d = msa.dims()
    p = ctypes.c_void_p(16)
    args = lambda B, M, M_loc, ws_bytes: (ctypes.byref(d), p, B, M, p, p, M_loc, 0, p, p, 0, 8, p, 2,
                                          p, p, 8, -1, p, None, p, ws_bytes, None)
    assert L.msa_sparse_attend_batch(*args(0, 1, 4, 1 << 30)) == -2
    assert b"B=0" in L.msa_last_error()
    assert L.msa_sparse_attend_batch(*args(2, 5, 4, 1 << 30)) == -2
    assert b"M_loc" in L.msa_last_error()
    assert L.msa_sparse_attend_batch(*args(2, 1, 4, 16)) == -3
    one = msa.sparse_attend_workspace(1, 129, 1024, d)
    w = [L.msa_sparse_attend_batch_workspace(ctypes.byref(d), B, 1, 129, 1024) for B in (1, 2, 8)]
    assert w[0] == one and w[0] < w[1] < w[2]
    assert L.msa_sparse_attend_batch_workspace(ctypes.byref(d), 0, 1, 129, 1024) == 0
    assert L.msa_sparse_attend_batch_workspace(ctypes.byref(d), 4, 64, 768, 2048) > \
        msa.sparse_attend_workspace(64, 768, 2048, d)


def test_attend_workspace_covers_every_smaller_context():
    """A workspace sized for cap_loc local tokens serves every smaller context
    (interleave rounds reuse one): the size is monotone in M_loc."""
    d = msa.dims()
    for M in (1, 8, 64, 256):
        for max_sel in (16, 1024, 2048):
            cap = 3 * 256 + M
            top = msa.sparse_attend_workspace(M, cap, max_sel, d)
            prev = 0
            for M_loc in range(M, cap + 1, 7):
                w = msa.sparse_attend_workspace(M, M_loc, max_sel, d)
                assert prev <= w <= top, (M, max_sel, M_loc)
                prev = w


def test_route_topk_noalloc_rejects_calls_beyond_its_scratch():
    """The no-allocation routing call refuses, before touching the GPU, a
    shape whose workspace exceeds its fixed scratch, and says how large each
    is; other argument errors are those of msa_route_topk."""
    L = msa.lib()
    d = msa.dims()
    p = ctypes.c_void_p(16)
    C = 5_000_000                          # 20 MB of chunk scores for one query
    need = msa.route_topk_workspace(1, 1, C, 1000, d)
    assert need > msa.NOALLOC_SCRATCH_BYTES
    rc = L.msa_route_topk_noalloc(ctypes.byref(d), p, 1, 1, p, p, 1000, C, p, 0, p, p, p, None)
    assert rc == -3
    msg = L.msa_last_error().decode()
    assert str(need) in msg and str(msa.NOALLOC_SCRATCH_BYTES) in msg
    rc = L.msa_route_topk_noalloc(ctypes.byref(d), None, 1, 1, p, p, 4, 8, p, 0, p, p, p, None)
    assert rc == -1
    rc = L.msa_route_topk_noalloc(ctypes.byref(d), p, 0, 1, p, p, 4, 8, p, 0, p, p, p, None)
    assert rc == -2


def test_interleave_batch_rejects_bad_states_before_the_gpu():
    """The batched interleave calls check the state and shapes on the host:
    a batch of no queries or of more than 65,535, a round past the local
    capacity and missing buffers fail with their codes and touch no device
    memory."""
    L = msa.lib()
    d = msa.dims()
    p = ctypes.c_void_p(16)
    st = msa._lib.InterleaveBatchC(p, p, p, 0, 64, 0, p, p, p, -1)
    assert L.msa_interleave_batch_reset(ctypes.byref(st), 10, None) == -2
    args = (p, p, p, p, 8, p, p, p, 0, 100, p, 10, 64, p, p, 1 << 20, None)
    assert L.msa_interleave_batch_step(ctypes.byref(d), ctypes.byref(st), *args) == -2
    st.B = 65536                           # one launch appends every query's rows: B <= 65535
    assert L.msa_interleave_batch_step(ctypes.byref(d), ctypes.byref(st), *args) == -2
    assert b"65535" in L.msa_last_error()
    st.B, st.n_loc = 2, 60                 # 60 + 8 tokens exceed cap_loc = 64
    assert L.msa_interleave_batch_step(ctypes.byref(d), ctypes.byref(st), *args) == -2
    assert b"cap_loc" in L.msa_last_error()
    assert st.n_loc == 60
    st.n_loc, st.doc_scores = 0, None
    assert L.msa_interleave_batch_step(ctypes.byref(d), ctypes.byref(st), *args) == -1
    assert L.msa_interleave_batch_step_workspace(ctypes.byref(d), 0, 8, 64, 100, 10, 64) == 0
    one = L.msa_interleave_step_workspace(ctypes.byref(d), 8, 64, 100, 10, 64)
    two = L.msa_interleave_batch_step_workspace(ctypes.byref(d), 2, 8, 64, 100, 10, 64)
    assert two >= one > 0


def test_misaligned_bf16_tensors_are_rejected_before_the_gpu():
    """Kernels move bf16 tensors in 16-byte vectors, so each must start at a
    16-byte aligned address: a misaligned one fails with MSA_ERR_INVALID_ARG
    naming the argument, before any device work (aligned fake addresses pass
    these checks and fail later, on the workspace check)."""
    L = msa.lib()
    d = msa.dims()
    p = ctypes.c_void_p(256)
    bad = ctypes.c_void_p(258)

    def scores(qr, kr):
        return L.msa_route_scores(ctypes.byref(d), qr, 2, 1, kr, 100, p, None, 0, None)

    assert scores(bad, p) == -1 and b"QR must start at a 16-byte" in L.msa_last_error()
    assert scores(p, bad) == -1 and b"KRbar" in L.msa_last_error()
    assert _route(d, ptr=258) == -1 and b"route: QR" in L.msa_last_error()

    def attend(q=p, kl=p, vl=p, kb=p, vb=p, out=p):
        return L.msa_sparse_attend(ctypes.byref(d), q, 4, kl, vl, 8, 0, kb, vb, 0, 8, p, 2, p, p,
                                   8, -1, out, None, p, 0, None)

    assert attend() == -3                           # aligned: reaches the workspace check
    for name in ("q", "kl", "vl", "kb", "vb", "out"):
        assert attend(**{name: bad}) == -1, name
    assert b"attend: V_loc" in (attend(vl=bad), L.msa_last_error())[1]
    rc = L.msa_encode_pool(ctypes.byref(d), p, bad, p, p, p, 1, 64, 1, p, p, p, None, 0, None)
    assert rc == -1 and b"encode_pool: V must" in L.msa_last_error()
