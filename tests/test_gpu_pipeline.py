"""Concurrent decode queries on separate streams (the pipelined form of the
layer loop): each query's route → select → attend chain runs in order on its
own stream while other queries' chains overlap it. Every lane's document
scores, selection and attention output are checked against the oracle, and
the concurrent results must be bit-identical to running the same chains one
after another on one stream."""
import numpy as np
import pytest
import torch

import routed_sparse_attention_amd as msa
import synth
from oracle import msa_oracle as O
from tests._util import assert_attn_close, assert_scores_close, assert_topk_matches, u16

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
            "ds_l": [None] * L,
        }

    def layer(st, q, l):
        # query q reads layer l's inputs shifted by q, so the chains differ
        ql = (l + q) % L
        msa.route_scores(queries[ql].QR, store.KRbar[ql], d, out=st["S"])
        msa.select_topk(st["S"], dco, d, doc_scores=st["ds"], outs=st["outs"])
        st["ids"][l] = st["outs"][0].clone()
        st["ds_l"][l] = st["ds"].clone()
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

    # every lane against the oracle: document scores of all 30K chunks, the
    # top-16 rule, and the decode attention over the lane's own selection
    # read from pinned host memory
    dco_h = store.doc_chunk_offsets
    kb_h, vb_h = u16(store.Kbar), u16(store.Vbar)
    oracle_s = {}
    for ql in range(L):
        oracle_s[ql] = O.doc_scores(O.chunk_scores(u16(queries[ql].QR[0]), u16(store.KRbar[ql])),
                                    dco_h)
    for q in range(Qn):
        for l in range(L):
            ql = (l + q) % L
            ids = conc[q]["ids"][l][0].cpu().numpy()
            assert_scores_close(conc[q]["ds_l"][l][0].cpu().numpy(), oracle_s[ql],
                                f"lane {q} layer {l} doc scores")
            assert_topk_matches(ids, 16, oracle_s[ql], 16)
            a = atts[ql]
            ref = O.sparse_attend(u16(a.Q), u16(a.K_loc), u16(a.V_loc), kb_h, vb_h, dco_h,
                                  [int(x) for x in ids])
            assert_attn_close(O.bf16_to_f64(u16(conc[q]["out"][l])), ref,
                              f"lane {q} layer {l} attention")


def test_batched_concurrent_queries_match_oracle():
    """The batched schedule of concurrent decode queries: per layer the
    queries are routed together (one scan of the layer's router keys and one
    selection for all), then each attends over its own selection, and the next
    layer follows. Query q's router rows at layer l are those of input layer
    (l + q) % L, so the rows of a batch differ. Every query's document scores,
    top-16 and attention are checked against the oracle."""
    print("[case] 3 queries × 4 layers routed together per layer", flush=True)
    L, Qn = 4, 3
    store, queries, atts = synth.cfg4_100m(DEV, seed=82, n_chunks=30_000, n_layers=L,
                                           kv_pinned=True)
    d = msa.dims()
    dco = torch.from_numpy(store.doc_chunk_offsets).to(DEV)
    max_sel = d.top_k * int(np.diff(store.doc_chunk_offsets).max())
    C, N = store.n_chunks, store.n_docs
    S = torch.empty((Qn, C), dtype=torch.float32, device=DEV)
    ds = torch.empty((Qn, N), dtype=torch.float32, device=DEV)
    outs = (torch.empty((Qn, 16), dtype=torch.int32, device=DEV),
            torch.empty((Qn, 16), dtype=torch.float32, device=DEV),
            torch.empty((Qn,), dtype=torch.int32, device=DEV))
    res = []
    for l in range(L):
        QR = torch.cat([queries[(l + q) % L].QR for q in range(Qn)])
        msa.route_scores(QR, store.KRbar[l], d, out=S)
        msa.select_topk(S, dco, d, doc_scores=ds, outs=outs)
        out = [msa.sparse_attend(atts[l].Q, atts[l].K_loc, atts[l].V_loc, store.Kbar, store.Vbar,
                                 dco, outs[0][q], outs[2][q:q + 1], max_sel, d=d)
               for q in range(Qn)]
        res.append((ds.clone(), outs[0].clone(), out))
    torch.cuda.synchronize()
    dco_h = store.doc_chunk_offsets
    kb_h, vb_h = u16(store.Kbar), u16(store.Vbar)
    a_ref = {}
    for l in range(L):
        ds_l, ids_l, out_l = res[l]
        for q in range(Qn):
            ref_s = O.doc_scores(O.chunk_scores(u16(queries[(l + q) % L].QR[0]),
                                                u16(store.KRbar[l])), dco_h)
            ids = ids_l[q].cpu().numpy()
            assert_scores_close(ds_l[q].cpu().numpy(), ref_s, f"query {q} layer {l} doc scores")
            assert_topk_matches(ids, 16, ref_s, 16)
            a = atts[l]
            key = (l, tuple(int(x) for x in ids))
            if key not in a_ref:
                a_ref[key] = O.sparse_attend(u16(a.Q), u16(a.K_loc), u16(a.V_loc), kb_h, vb_h,
                                             dco_h, list(key[1]))
            assert_attn_close(O.bf16_to_f64(u16(out_l[q])), a_ref[key],
                              f"query {q} layer {l} attention")
