"""msa_route_topk_noalloc, the routing call that takes no workspace, against
msa_route_topk with a caller workspace: the same kernels, so the outputs must
be identical. Two calls in a row on the fixed scratch, the second smaller than
the first (the scratch keeps the first call's contents), then a call that
max-merges into running scores. Both entry points are called through the C
ABI directly."""
import ctypes

import numpy as np
import pytest
import torch

import routed_sparse_attention_amd as msa
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _call(noalloc, d, QR, KR, dco, n_docs, ds, accumulate, k):
    L = msa.lib()
    B, M, C = QR.shape[0], QR.shape[1], KR.shape[0]
    ids = torch.full((B, k), -7, dtype=torch.int32, device=DEV)
    sc = torch.full((B, k), 7.0, dtype=torch.float32, device=DEV)
    ns = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        rc = L.msa_route_topk_noalloc(ctypes.byref(d), QR.data_ptr(), B, M, KR.data_ptr(),
                                      dco.data_ptr(), n_docs, C, ds.data_ptr(), int(accumulate),
                                      ids.data_ptr(), sc.data_ptr(), ns.data_ptr(), stream)
    else:
        need = L.msa_route_topk_workspace(ctypes.byref(d), B, M, C, n_docs)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        rc = L.msa_route_topk(ctypes.byref(d), QR.data_ptr(), B, M, KR.data_ptr(), dco.data_ptr(),
                              n_docs, C, ds.data_ptr(), int(accumulate), ids.data_ptr(),
                              sc.data_ptr(), ns.data_ptr(), ws.data_ptr(), need, stream)
    assert rc == 0, L.msa_last_error().decode()
    return ds, ids, sc, ns


def _case(seed, n_chunks, B, M, lo, hi):
    rng = synth.np_rng(seed, 0)
    counts = synth.counts_until(rng, n_chunks, lo, hi)
    st = synth.pooled_store(counts, seed, DEV)
    QR = synth.randn_bf16((B, M, 8, 128), synth.torch_gen(seed, 3, DEV), DEV)
    dco = torch.from_numpy(st.doc_chunk_offsets).to(DEV)
    return st, QR, dco


def _same(a, b, what):
    for x, y, n in zip(a, b, ("doc_scores", "ids", "scores", "n_sel")):
        assert torch.equal(x, y), f"{what}: {n} differ"


def test_noalloc_matches_route_topk_on_two_calls_then_accumulate():
    d = msa.dims()
    # 1) a decode query over 1,200,000 chunks (the VALU scan; 4.8 MB of scores)
    print("[case] noalloc: 1 query x 1,200,000 chunks", flush=True)
    st, QR, dco = _case(901, 1_200_000, 1, 1, 4, 64)
    N = st.n_docs
    a = _call(True, d, QR, st.KRbar, dco, N, torch.empty((1, N), device=DEV), 0, 16)
    b = _call(False, d, QR, st.KRbar, dco, N, torch.empty((1, N), device=DEV), 0, 16)
    torch.cuda.synchronize()
    _same(a, b, "first call")
    # 2) right after it, a smaller call: 2 queries of 13 tokens over 30,000
    #    chunks (the MFMA scan with per-part maxima in the scratch)
    print("[case] noalloc: 2 queries x 13 tokens x 30,000 chunks", flush=True)
    st2, QR2, dco2 = _case(902, 30_000, 2, 13, 1, 40)
    N2 = st2.n_docs
    a2 = _call(True, d, QR2, st2.KRbar, dco2, N2, torch.empty((2, N2), device=DEV), 0, 16)
    b2 = _call(False, d, QR2, st2.KRbar, dco2, N2, torch.empty((2, N2), device=DEV), 0, 16)
    torch.cuda.synchronize()
    _same(a2, b2, "second call")
    # 3) max-merge into the running scores of the second call
    print("[case] noalloc: accumulate", flush=True)
    QR3 = synth.randn_bf16((2, 5, 8, 128), synth.torch_gen(903, 3, DEV), DEV)
    a3 = _call(True, d, QR3, st2.KRbar, dco2, N2, a2[0].clone(), 1, 16)
    b3 = _call(False, d, QR3, st2.KRbar, dco2, N2, b2[0].clone(), 1, 16)
    torch.cuda.synchronize()
    _same(a3, b3, "accumulate")
    assert torch.all(a3[0] >= a2[0])


def test_noalloc_refuses_a_call_beyond_its_scratch():
    print("[case] noalloc: too large", flush=True)
    d = msa.dims()
    st, QR, dco = _case(904, 5_000_000, 1, 1, 4, 64)
    N = st.n_docs
    ds = torch.full((1, N), 3.0, device=DEV)
    L = msa.lib()
    ids = torch.full((1, 16), -7, dtype=torch.int32, device=DEV)
    rc = L.msa_route_topk_noalloc(ctypes.byref(d), QR.data_ptr(), 1, 1, st.KRbar.data_ptr(),
                                  dco.data_ptr(), N, st.n_chunks, ds.data_ptr(), 0, ids.data_ptr(),
                                  ds.data_ptr(), ids.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == -3 and b"scratch" in L.msa_last_error()
    assert torch.all(ds == 3.0) and torch.all(ids == -7)
