"""HIP path versus the oracle, element by element, on seeded synthetic inputs.

Every call goes through the C ABI (libmsa.so via the ctypes binding). Sizes
are small enough for the fp64 oracle to finish in seconds while spanning
several tiles and ragged tails; the full-size workloads are covered in
``test_gpu_fullsize.py``.
"""
import numpy as np
import pytest
import torch

import routed_sparse_attention_amd as msa
import synth
from oracle import msa_oracle as O
from tests._util import (assert_attn_close, assert_pooled_close, assert_scores_close,
                         assert_topk_matches, u16)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _pool_gpu(mem, d=None):
    dco_h = msa.plan_chunks(mem.doc_token_offsets, (d or msa.dims()).chunk)
    C = int(dco_h[-1])
    dto = torch.from_numpy(mem.doc_token_offsets).to(DEV)
    dco = torch.from_numpy(dco_h).to(DEV)
    Kb, Vb, Rb = msa.encode_pool(mem.K.to(DEV), mem.V.to(DEV), mem.KR.to(DEV), dto, dco, C, d)
    torch.cuda.synchronize()
    return Kb, Vb, Rb, dco_h, dco


# ---------------------------------------------------------------------------
# pooling (stage 1)
# ---------------------------------------------------------------------------
def test_pool_cfg1():
    _banner("pool cfg1 64x512")
    mem, _, _ = synth.cfg1_tiny("cpu")
    Kb, Vb, Rb, dco_h, _ = _pool_gpu(mem)
    oK, oV, oR, odco = O.pool(u16(mem.K), u16(mem.V), u16(mem.KR), mem.doc_token_offsets)
    assert np.array_equal(dco_h, odco)
    for g, e, n in ((Kb, oK, "K"), (Vb, oV, "V"), (Rb, oR, "KR")):
        assert_pooled_close(u16(g), e, n)


@pytest.mark.parametrize("mode", [O.DOC_ROPE_TOKEN, O.DOC_ROPE_CHUNK])
def test_pool_ragged(mode):
    _banner(f"pool ragged mode={mode}")
    lengths = [1, 2, 63, 64, 65, 127, 128, 129, 300, 1000, 7, 640, 513]
    mem = synth.raw_memory(lengths, 11, "cpu", n_plant=2)
    d = msa.dims(doc_rope_mode=mode, rope_theta=1e4)
    Kb, Vb, Rb, dco_h, _ = _pool_gpu(mem, d)
    oK, oV, oR, odco = O.pool(u16(mem.K), u16(mem.V), u16(mem.KR), mem.doc_token_offsets,
                              theta=1e4, doc_rope_mode=mode)
    assert np.array_equal(dco_h, odco)
    for g, e, n in ((Kb, oK, "K"), (Vb, oV, "V"), (Rb, oR, "KR")):
        assert_pooled_close(u16(g), e, n)
    # planted chunks pool to the planted vector exactly
    for doc, (c, uvec) in mem.planted.items():
        assert np.array_equal(u16(Rb[int(dco_h[doc]) + c]), u16(uvec))


def test_pool_chunk_size_and_long_doc():
    _banner("pool chunk=16 long doc")
    lengths = [5000, 3, 17]
    mem = synth.raw_memory(lengths, 12, "cpu")
    d = msa.dims(chunk=16)
    Kb, Vb, Rb, dco_h, _ = _pool_gpu(mem, d)
    oK, oV, oR, odco = O.pool(u16(mem.K), u16(mem.V), u16(mem.KR), mem.doc_token_offsets, chunk=16)
    for g, e, n in ((Kb, oK, "K"), (Vb, oV, "V"), (Rb, oR, "KR")):
        assert_pooled_close(u16(g), e, n)


def test_pool_deterministic():
    mem = synth.raw_memory([300, 77, 1024], 13, "cpu")
    a = _pool_gpu(mem)
    b = _pool_gpu(mem)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)


# ---------------------------------------------------------------------------
# routing + top-k (stage 2)
# ---------------------------------------------------------------------------
def _store(n_chunks, seed, lo=1, hi=40):
    rng = synth.np_rng(seed, 0)
    counts = synth.counts_until(rng, n_chunks, lo, hi)
    st = synth.pooled_store(counts, seed, "cpu")
    return st


def _check_route(QR, st, d, accumulate=False, prev=None):
    B = QR.shape[0]
    dco = torch.from_numpy(st.doc_chunk_offsets).to(DEV)
    ds_in = None
    if prev is not None:
        ds_in = torch.from_numpy(prev.astype(np.float32)).to(DEV)
    ds, ids, sc, ns = msa.route_topk(QR.to(DEV), st.KRbar.to(DEV), dco, d, doc_scores=ds_in,
                                     accumulate=accumulate)
    torch.cuda.synchronize()
    ds, ids, sc, ns = ds.cpu().numpy(), ids.cpu().numpy(), sc.cpu().numpy(), ns.cpu().numpy()
    R = u16(st.KRbar)
    worst = 0.0
    for b in range(B):
        s = O.doc_scores(O.chunk_scores(u16(QR[b]), R, d.token_reduce), st.doc_chunk_offsets)
        if prev is not None:
            s = np.maximum(prev[b], s)
        worst = max(worst, assert_scores_close(ds[b], s, f"query {b} doc scores"))
        assert_topk_matches(ids[b], ns[b], s, d.top_k)
        n = int(ns[b])
        # reported scores are the GPU's own doc scores of the selected ids
        assert np.array_equal(sc[b][:n], ds[b][ids[b][:n]], equal_nan=True)
    return ds, ids, worst


@pytest.mark.parametrize("B,M", [(1, 1), (3, 1), (2, 3), (1, 8), (5, 13), (1, 64), (9, 1),
                                 (64, 1), (1, 130), (3, 70), (70, 1)])
def test_route_shapes(B, M):
    _banner(f"route B={B} M={M}")
    st = _store(3000, 21 + B * 100 + M)
    g = synth.torch_gen(5, B * 1000 + M)
    QR = synth.randn_bf16((B, M, 8, 128), g)
    _check_route(QR, st, msa.dims())


def test_route_cfg1_planted():
    _banner("route cfg1 planted")
    mem, q, _ = synth.cfg1_tiny("cpu")
    Kb, Vb, Rb, dco_h, dco = _pool_gpu(mem)
    ds, ids, sc, ns = msa.route_topk(q.QR.to(DEV), Rb, dco)
    torch.cuda.synchronize()
    oK, oV, oR, odco = O.pool(u16(mem.K), u16(mem.V), u16(mem.KR), mem.doc_token_offsets)
    s = O.doc_scores(O.chunk_scores(u16(q.QR[0]), oR), odco)
    assert_scores_close(ds.cpu().numpy()[0], s)
    assert_topk_matches(ids.cpu().numpy()[0], ns.cpu().numpy()[0], s, 16)
    assert set(ids.cpu().numpy()[0][:4].tolist()) == set(mem.planted.keys())


@pytest.mark.parametrize("B,M", [(2, 11), (1, 3), (2, 100)])
def test_route_mean_mode(B, M):
    _banner(f"route MEAN B={B} M={M}")
    st = _store(2000, 31)
    QR = synth.randn_bf16((B, M, 8, 128), synth.torch_gen(6, M))
    _check_route(QR, st, msa.dims(token_reduce=O.TOKEN_REDUCE_MEAN))


def test_route_accumulate():
    _banner("route accumulate")
    st = _store(2500, 41)
    QR1 = synth.randn_bf16((1, 4, 8, 128), synth.torch_gen(7, 1))
    QR2 = synth.randn_bf16((1, 4, 8, 128), synth.torch_gen(7, 2))
    d = msa.dims()
    ds1, _, _ = _check_route(QR1, st, d)
    prev = O.doc_scores(O.chunk_scores(u16(QR1[0]), u16(st.KRbar)), st.doc_chunk_offsets)[None]
    _check_route(QR2, st, d, accumulate=True, prev=prev)
    with pytest.raises(msa.MsaError):
        msa.route_topk(QR1.to(DEV), st.KRbar.to(DEV), torch.from_numpy(st.doc_chunk_offsets).to(DEV),
                       msa.dims(token_reduce=O.TOKEN_REDUCE_MEAN),
                       doc_scores=torch.from_numpy(ds1).to(DEV), accumulate=True)


def test_route_ties_small_n_and_nan():
    _banner("route ties / N<k / NaN")
    # 5 docs, docs 1 and 3 byte copies of doc 0 -> exact ties resolve to lowest id
    counts = [3, 3, 2, 3, 4]
    st = synth.pooled_store(counts, 51, "cpu")
    KR = st.KRbar.clone()
    KR[3:6] = KR[0:3]
    KR[8:11] = KR[0:3]
    st.KRbar = KR
    QR = KR[1:2].unsqueeze(0).clone()                    # aligned with chunk 1 of doc 0
    ds, ids, _ = _check_route(QR, st, msa.dims())        # k=16 > N=5
    assert list(ids[0][:3]) == [0, 1, 3] and list(ids[0][5:]) == [-1] * 11
    assert ds[0][0] == ds[0][1] == ds[0][3]
    # a NaN chunk makes its document's score NaN, which ranks last
    KR2 = KR.clone()
    KR2[6, 2, 5] = float("nan")                          # chunk 6 belongs to doc 2
    st.KRbar = KR2
    dco = torch.from_numpy(st.doc_chunk_offsets).to(DEV)
    ds2, ids2, sc2, ns2 = msa.route_topk(QR.to(DEV), KR2.to(DEV), dco)
    torch.cuda.synchronize()
    nan_doc = int(np.searchsorted(st.doc_chunk_offsets, 6, side="right") - 1)
    assert np.isnan(ds2.cpu().numpy()[0][nan_doc])
    assert int(ids2.cpu().numpy()[0][4]) == nan_doc


def test_route_deterministic():
    st = _store(4000, 61)
    QR = synth.randn_bf16((4, 1, 8, 128), synth.torch_gen(8, 1)).to(DEV)
    dco = torch.from_numpy(st.doc_chunk_offsets).to(DEV)
    R = st.KRbar.to(DEV)
    a = msa.route_topk(QR, R, dco)
    b = msa.route_topk(QR, R, dco)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ---------------------------------------------------------------------------
# sparse attention (stage 3)
# ---------------------------------------------------------------------------
def _attend_case(M, M_loc, counts, sel, seed, host_kv=False, pos0=-1, k_rot=False, top_k=16,
                 sel_gpu=None):
    """sel: the selection the oracle attends over; sel_gpu (default sel): the
    ids the GPU is given, which may hold invalid ids that it must skip."""
    st = synth.pooled_store(counts, seed, "cpu", with_kv=True)
    att = synth.attend_inputs(M, M_loc, seed)
    dco_h = st.doc_chunk_offsets
    d = msa.dims(top_k=top_k)
    sel_gpu = sel if sel_gpu is None else sel_gpu
    sel_pad = np.full(top_k, -1, np.int32)
    sel_pad[:len(sel_gpu)] = sel_gpu
    sel_t = torch.from_numpy(sel_pad).to(DEV)
    ns_t = torch.tensor([len(sel_gpu)], dtype=torch.int32, device=DEV)
    if host_kv:
        Kb = st.Kbar.pin_memory()
        Vb = st.Vbar.pin_memory()
    else:
        Kb, Vb = st.Kbar.to(DEV), st.Vbar.to(DEV)
    max_sel = int(sum(int(dco_h[i + 1] - dco_h[i]) for i in sel)) + 3
    out, of = msa.sparse_attend(att.Q.to(DEV), att.K_loc.to(DEV), att.V_loc.to(DEV), Kb, Vb,
                                torch.from_numpy(dco_h).to(DEV), sel_t, ns_t, max_sel, pos0=pos0,
                                k_loc_rotated=k_rot, d=d, want_f32=True)
    torch.cuda.synchronize()
    ref = O.sparse_attend(u16(att.Q), u16(att.K_loc), u16(att.V_loc), u16(st.Kbar), u16(st.Vbar),
                          dco_h, sel, None if pos0 < 0 else pos0, k_rot)
    assert_attn_close(of.cpu().numpy(), ref, "fp32 out")
    assert_attn_close(O.bf16_to_f64(u16(out)), ref, "bf16 out")
    # bf16 output is the rounding of the fp32 output
    assert np.array_equal(u16(out), O.f64_to_bf16(of.cpu().numpy().astype(np.float64)))


def test_attend_prefill():
    _banner("attend prefill M=64")
    rng = synth.np_rng(71, 0)
    counts = rng.integers(1, 20, size=30)
    sel = [int(x) for x in rng.choice(30, size=16, replace=False)]
    _attend_case(64, 64, counts, sel, 71)


def test_attend_decode():
    _banner("attend decode M=1 M_loc=129")
    counts = [64] * 20 + [3, 40, 17]
    _attend_case(1, 129, counts, list(range(3, 19)), 72)


def test_attend_decode_host_kv():
    _banner("attend decode pinned host KV")
    counts = [33, 64, 5, 12, 64, 64, 1, 9, 40, 2, 64, 30, 18, 7, 64, 50, 11]
    _attend_case(1, 129, counts, list(range(16, 0, -1)), 73, host_kv=True)


def test_attend_ragged_prefill_pos0_prerotated():
    _banner("attend M=37 M_loc=100 pos0=5 pre-rotated")
    counts = [13, 2, 70, 9, 31]
    _attend_case(37, 100, counts, [2, 0, 4], 74, pos0=5, k_rot=True, top_k=4)


def test_attend_no_memory_and_one_token():
    _banner("attend empty selection")
    _attend_case(1, 1, [4, 4], [], 75, top_k=2)


def test_attend_long_local():
    _banner("attend M=256 M_loc=700")
    counts = [64] * 10 + [100, 128, 7]
    _attend_case(256, 700, counts, [10, 11, 0, 5, 12, 3], 76)


@pytest.mark.parametrize("M,M_loc,pos0", [(1, 40, 70_000), (3, 35, 1_000_003), (8, 71, 12_345),
                                           (9, 40, 123_456), (1, 33, -1)])
def test_attend_rope_positions(M, M_loc, pos0):
    """Global RoPE of Q and local K at large positions: up to 8 query tokens
    rotate their local keys inside the attention waves, 9 use the separate
    rotation kernel; local tiles straddle the memory/local boundary."""
    _banner(f"attend RoPE M={M} M_loc={M_loc} pos0={pos0}")
    counts = [5, 17, 2, 64, 9, 33, 1, 12, 40, 7, 3, 21]
    sel = [3, 8, 0, 11, 5, 1, 9, 6, 2, 10]
    _attend_case(M, M_loc, counts, sel, 78 + M, pos0=pos0)


def test_attend_k64_with_invalid_ids():
    """top_k = 64 (the chunk list's largest search), with invalid ids mixed
    into the selection: the GPU skips them, so it must equal the oracle over
    the valid ids in the same order (pos0 given, since n_sel counts them)."""
    _banner("attend top_k=64, invalid ids skipped")
    rng = synth.np_rng(79, 0)
    counts = rng.integers(1, 4, size=80)
    valid = [int(x) for x in rng.choice(80, size=60, replace=False)]
    sel_gpu = list(valid)
    for pos, bad in ((0, -1), (17, 80), (33, 10 ** 6), (63, -7)):
        sel_gpu.insert(pos, bad)
    assert len(sel_gpu) == 64
    _attend_case(2, 50, counts, valid, 79, pos0=64, top_k=64, sel_gpu=sel_gpu)


def test_attend_rejects_pageable_host_kv():
    st = synth.pooled_store([4, 4], 77, "cpu", with_kv=True)
    att = synth.attend_inputs(1, 2, 77)
    sel = torch.tensor([0, 1], dtype=torch.int32, device=DEV)
    ns = torch.tensor([2], dtype=torch.int32, device=DEV)
    with pytest.raises((msa.MsaError, ValueError)):
        msa.sparse_attend(att.Q.to(DEV), att.K_loc.to(DEV), att.V_loc.to(DEV), st.Kbar, st.Vbar,
                          torch.from_numpy(st.doc_chunk_offsets).to(DEV), sel, ns, 8,
                          d=msa.dims(top_k=2))


# ---------------------------------------------------------------------------
# Memory Interleave
# ---------------------------------------------------------------------------
def test_interleave_rounds():
    _banner("interleave 3 rounds")
    mem, chains = synth.cfg5_memory("cpu", seed=9, n_tokens=120_000, n_queries=1, hops=3)
    Kb, Vb, Rb, dco_h, dco = _pool_gpu(mem)
    oK, oV, oR, odco = O.pool(u16(mem.K), u16(mem.V), u16(mem.KR), mem.doc_token_offsets)
    d = msa.dims(top_k=4)
    max_sel = int(np.diff(dco_h).max()) * 4
    il = msa.Interleave(len(dco_h) - 1, cap_loc=3 * 96, d=d)
    st = O.InterleaveState(len(dco_h) - 1)
    for r, doc in enumerate(chains[0]):
        QR, Q, Kn, Vn = synth.cfg5_round(mem, doc, 0, r, seed=9, M_new=96, block=64)
        out = il.step(Q.to(DEV), Kn.to(DEV), Vn.to(DEV), QR.to(DEV), Rb, Kb, Vb, dco, max_sel)
        torch.cuda.synchronize()
        ids, sc, mg, ref = O.interleave_step(st, u16(Q), u16(Kn), u16(Vn), u16(QR), oR, oK, oV, odco, k=4)
        assert_scores_close(il.doc_scores.cpu().numpy(), st.doc_scores, f"round {r} doc scores")
        assert_topk_matches(il.topk_ids.cpu().numpy(), il.n_sel.cpu().numpy()[0], st.doc_scores, 4)
        assert doc in set(il.topk_ids.cpu().numpy().tolist())
        assert_attn_close(O.bf16_to_f64(u16(out)), ref, f"round {r} attention")
    assert il.n_loc == 3 * 96


# ---------------------------------------------------------------------------
# boundary behaviour
# ---------------------------------------------------------------------------
def test_workspace_too_small():
    st = _store(500, 81)
    QR = synth.randn_bf16((1, 1, 8, 128), synth.torch_gen(9, 1)).to(DEV)
    dco = torch.from_numpy(st.doc_chunk_offsets).to(DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    d = msa.dims()
    ds = torch.full((1, st.n_docs), 7.0, device=DEV)
    ids = torch.full((1, 16), 5, dtype=torch.int32, device=DEV)
    lib = msa.lib()
    import ctypes
    rc = lib.msa_route_topk(ctypes.byref(d), QR.data_ptr(), 1, 1, st.KRbar.to(DEV).data_ptr(),
                            dco.data_ptr(), st.n_docs, st.n_chunks, ds.data_ptr(), 0, ids.data_ptr(),
                            ds.data_ptr(), ids.data_ptr(), ws.data_ptr(), 16, None)
    torch.cuda.synchronize()
    assert rc == -3 and b"workspace" in lib.msa_last_error()
    assert torch.all(ds == 7.0) and torch.all(ids == 5)   # nothing written on error


# ---------------------------------------------------------------------------
# the two halves of routing as separate calls
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,M", [(1, 1), (2, 40)])
def test_route_scores_call(B, M):
    _banner(f"route_scores B={B} M={M}")
    st = _store(1500, 91 + M)
    QR = synth.randn_bf16((B, M, 8, 128), synth.torch_gen(10, M))
    S = msa.route_scores(QR.to(DEV), st.KRbar.to(DEV))
    torch.cuda.synchronize()
    for b in range(B):
        assert_scores_close(S[b].cpu().numpy(), O.chunk_scores(u16(QR[b]), u16(st.KRbar)),
                            f"chunk scores q{b}")


def test_select_topk_exact_on_given_scores():
    _banner("select_topk on synthetic chunk scores")
    rng = synth.np_rng(92, 0)
    counts = synth.counts_until(rng, 40_000, 1, 64)
    dco_h = synth.offsets_from_lengths(counts)
    C = int(dco_h[-1])
    # fp32 chunk scores with repeated values (ties) drawn by the generator
    S = (rng.integers(-300, 300, size=(3, C)) / 300.0).astype(np.float32)
    d = msa.dims()
    ds, ids, sc, ns = msa.select_topk(torch.from_numpy(S).to(DEV), torch.from_numpy(dco_h).to(DEV), d)
    torch.cuda.synchronize()
    for b in range(3):
        s = O.doc_scores(S[b].astype(np.float64), dco_h)
        assert np.array_equal(ds[b].cpu().numpy().astype(np.float64), s)
        exp_ids, exp_sc, _ = O.topk(s, 16)
        assert list(ids[b].cpu().numpy()) == list(exp_ids)      # bit-exact, ties included
        assert int(ns[b]) == 16


@pytest.mark.parametrize("case", ["all_equal", "k40", "small_n"])
def test_select_topk_fallback_paths(case):
    _banner(f"select_topk fallback {case}")
    rng = synth.np_rng(93, 0)
    n_docs = {"all_equal": 5000, "k40": 3000, "small_n": 7}[case]
    counts = rng.integers(1, 9, size=n_docs)
    dco_h = synth.offsets_from_lengths(counts)
    C = int(dco_h[-1])
    if case == "all_equal":
        S = np.full((2, C), 0.25, np.float32)            # every document ties
    else:
        S = (rng.integers(-50, 50, size=(2, C)) / 50.0).astype(np.float32)
    k = 40 if case == "k40" else 16
    d = msa.dims(top_k=k)
    ds, ids, sc, ns = msa.select_topk(torch.from_numpy(S).to(DEV), torch.from_numpy(dco_h).to(DEV), d)
    torch.cuda.synchronize()
    for b in range(2):
        s = O.doc_scores(S[b].astype(np.float64), dco_h)
        exp_ids, exp_sc, _ = O.topk(s, k)
        n = len(exp_ids)
        assert int(ns[b]) == n
        assert list(ids[b].cpu().numpy()[:n]) == list(exp_ids)
        assert np.array_equal(sc[b].cpu().numpy()[:n].astype(np.float64), exp_sc)
        assert all(x == -1 for x in ids[b].cpu().numpy()[n:])


@pytest.mark.parametrize("n_chunks", [1, 2, 5, 31, 33, 3001])
@pytest.mark.parametrize("B,M", [(1, 1), (9, 1), (2, 13)])
def test_route_ragged_chunk_counts(n_chunks, B, M):
    """Chunk counts that fill no tile, end mid-tile, or are not a multiple of
    four, on both scans (8 rows or fewer: VALU; more: MFMA)."""
    _banner(f"route n_chunks={n_chunks} B={B} M={M}")
    st = _store(n_chunks, 500 + n_chunks, lo=1, hi=7)
    QR = synth.randn_bf16((B, M, 8, 128), synth.torch_gen(9, n_chunks * 100 + B * 10 + M))
    _check_route(QR, st, msa.dims())


def _doc_scores_case(rng, case):
    """fp32 chunk scores for the threshold paths of the top-k select."""
    n_docs, k = {"bs128_nan": (3000, 16), "bs256_ragged": (20_000, 16), "wave_bs32": (2100, 40),
                 "k64_wave": (2500, 64), "k64_bs256": (70_000, 64), "tie_top": (20_000, 16),
                 "blocks_over_2048": (600_000, 16)}[case]
    counts = rng.integers(1, 4, size=n_docs)
    dco_h = synth.offsets_from_lengths(counts)
    C = int(dco_h[-1])
    S = rng.standard_normal((2, C)).astype(np.float32)
    if case == "bs128_nan":
        S[:, rng.choice(C, size=50, replace=False)] = np.nan
    if case == "tie_top":
        # 40 documents spread over many blocks share the best score exactly
        for b in range(2):
            docs = rng.choice(n_docs, size=40, replace=False)
            S[b, dco_h[docs]] = 9.0
    return S, dco_h, k


@pytest.mark.parametrize("case", ["bs128_nan", "bs256_ragged", "wave_bs32", "k64_wave", "k64_bs256",
                                  "tie_top", "blocks_over_2048"])
def test_select_topk_threshold_paths(case):
    """Above 2048 documents the select thresholds on block maxima; the block
    size depends on N and k (down to one wave per 32-document block), and past
    2048 blocks it takes the radix path. Every form is exact."""
    _banner(f"select_topk threshold path {case}")
    rng = synth.np_rng(94, len(case))
    S, dco_h, k = _doc_scores_case(rng, case)
    d = msa.dims(top_k=k)
    ds, ids, sc, ns = msa.select_topk(torch.from_numpy(S).to(DEV), torch.from_numpy(dco_h).to(DEV), d)
    torch.cuda.synchronize()
    for b in range(S.shape[0]):
        s = O.doc_scores(S[b].astype(np.float64), dco_h)
        assert np.array_equal(ds[b].cpu().numpy().astype(np.float64), s, equal_nan=True)
        exp_ids, exp_sc, _ = O.topk(s, k)
        assert int(ns[b]) == k
        assert list(ids[b].cpu().numpy()) == list(exp_ids)
        assert np.array_equal(sc[b].cpu().numpy().astype(np.float64), exp_sc)
