"""Concurrent decode queries on separate streams (the pipelined form of the
layer loop): each query's route → select → attend chain runs in order on its
own stream while other queries' chains overlap it. Results must be bit-identical
to running the same chains one after another on one stream."""
import numpy as np
import pytest
import torch

import routed_sparse_attention_amd as msa
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_concurrent_queries_match_sequential():
    print("[case] 3 queries × 4 layers on 3 streams vs one stream", flush=True)
    L, Qn = 4, 3
    store, queries, atts = synth.cfg4_100m(DEV, seed=81, n_chunks=30_000, n_layers=L,
                                           kv_pinned=True)
    d = msa.dims()
    dco = torch.from_numpy(store.doc_chunk_offsets).to(DEV)
    max_sel = d.top_k * int(np.diff(store.doc_chunk_offsets).max())
    C, N = store.n_chunks, store.n_docs

    def lane():
        return {
            "S": torch.empty((1, C), dtype=torch.float32, device=DEV),
            "ds": torch.empty((1, N), dtype=torch.float32, device=DEV),
            "outs": (torch.empty((1, 16), dtype=torch.int32, device=DEV),
                     torch.empty((1, 16), dtype=torch.float32, device=DEV),
                     torch.empty((1,), dtype=torch.int32, device=DEV)),
            "out": [torch.empty((1, 32, 128), dtype=torch.bfloat16, device=DEV) for _ in range(L)],
            "ids": [None] * L,
        }

    def layer(st, q, l):
        # query q reads layer l's inputs shifted by q, so the chains differ
        ql = (l + q) % L
        msa.route_scores(queries[ql].QR, store.KRbar[ql], d, out=st["S"])
        msa.select_topk(st["S"], dco, d, doc_scores=st["ds"], outs=st["outs"])
        st["ids"][l] = st["outs"][0].clone()
        msa.sparse_attend(atts[ql].Q, atts[ql].K_loc, atts[ql].V_loc, store.Kbar, store.Vbar, dco,
                          st["outs"][0][0], st["outs"][2], max_sel, d=d, out=st["out"][l])

    seq = [lane() for _ in range(Qn)]
    for q in range(Qn):
        for l in range(L):
            layer(seq[q], q, l)
    torch.cuda.synchronize()

    conc = [lane() for _ in range(Qn)]
    streams = [torch.cuda.Stream() for _ in range(Qn)]
    for l in range(L):
        for q in range(Qn):
            with torch.cuda.stream(streams[q]):
                layer(conc[q], q, l)
    torch.cuda.synchronize()
    for q in range(Qn):
        for l in range(L):
            assert torch.equal(seq[q]["ids"][l], conc[q]["ids"][l]), (q, l)
            assert torch.equal(seq[q]["out"][l].view(torch.int16), conc[q]["out"][l].view(torch.int16))
            ql = (l + q) % L
            assert set(queries[ql].planted_docs[0]) <= set(conc[q]["ids"][l][0].cpu().tolist())
