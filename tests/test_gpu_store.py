"""Streaming memory update (msa_store_*), through the C ABI.

Pooling is per document, so a store grown by appending documents in batches
must equal the store of one msa_encode_pool call over all of them, bit for
bit, and its new rows must match the oracle's pooling of those documents.
A saved store must load back bit-exact, and routing over a grown (or loaded)
store must find documents planted in the newest batch.
"""
import numpy as np
import pytest
import torch

import routed_sparse_attention_amd as msa
import synth
from oracle import msa_oracle as O
from tests._util import assert_pooled_close, u16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _lengths(seed, n):
    rng = np.random.default_rng(seed)
    L = rng.integers(1, 300, size=n)
    L[:4] = [1, 64, 128, 65]      # a one-token document, exact multiples of 64, a 1-token tail
    return L


def _batch(mem, a, b):
    """Raw states and 0-based token offsets of documents [a, b)."""
    offs = mem.doc_token_offsets
    t0, t1 = int(offs[a]), int(offs[b])
    return mem.K[t0:t1], mem.V[t0:t1], mem.KR[t0:t1], offs[a:b + 1] - offs[a]


def _encode_all(mem, d):
    dco_h = msa.plan_chunks(mem.doc_token_offsets)
    dto = torch.from_numpy(mem.doc_token_offsets).to(DEV)
    dco = torch.from_numpy(dco_h).to(DEV)
    Kb, Vb, Rb = msa.encode_pool(mem.K, mem.V, mem.KR, dto, dco, int(dco_h[-1]), d)
    return Kb, Vb, Rb, dco_h


def _grow(mem, cuts, d, cap_docs=64, cap_chunks=2048, **kw):
    st = msa.Store(cap_docs, cap_chunks, d=d, **kw)
    for a, b in zip(cuts[:-1], cuts[1:]):
        K, V, KR, offs = _batch(mem, a, b)
        ids = st.append(K, V, KR, offs)
        assert list(ids) == list(range(a, b))
    torch.cuda.synchronize()
    return st


def _same(a, b, what):
    assert a.shape == b.shape, what
    assert torch.equal(a.view(torch.int16).cpu(), b.view(torch.int16).cpu()), f"{what} differs"


@pytest.mark.parametrize("mode", [msa.DOC_ROPE_TOKEN, msa.DOC_ROPE_CHUNK])
def test_append_in_batches_equals_one_encode(mode):
    _banner(f"store append in 3 batches vs one encode, doc_rope_mode={mode}")
    d = msa.dims(doc_rope_mode=mode)
    mem = synth.raw_memory(_lengths(61, 40), seed=61, device=DEV)
    Kb, Vb, Rb, dco_h = _encode_all(mem, d)
    st = _grow(mem, [0, 13, 14, 40], d)
    assert st.n_docs == 40 and st.n_chunks == int(dco_h[-1])
    assert np.array_equal(st.offsets_h, dco_h)
    assert np.array_equal(st.doc_chunk_offsets.cpu().numpy(), dco_h)
    _same(st.Kbar, Kb, "Kbar")
    _same(st.Vbar, Vb, "Vbar")
    _same(st.KRbar, Rb, "KRbar")


def test_appended_rows_match_the_oracle():
    _banner("store append: new rows vs oracle pooling")
    d = msa.dims()
    mem = synth.raw_memory(_lengths(62, 30), seed=62, device=DEV)
    st = _grow(mem, [0, 20, 30], d)
    offs, dco_h = mem.doc_token_offsets, st.offsets_h
    for i in (0, 3, 19, 20, 21, 25, 29):
        t0, t1 = int(offs[i]), int(offs[i + 1])
        oK, oV, oR, _ = O.pool(u16(mem.K[t0:t1]), u16(mem.V[t0:t1]), u16(mem.KR[t0:t1]),
                               np.array([0, t1 - t0]))
        r0, r1 = int(dco_h[i]), int(dco_h[i + 1])
        for g, e, n in ((st.Kbar, oK, "K"), (st.Vbar, oV, "V"), (st.KRbar, oR, "KR")):
            assert_pooled_close(u16(g[r0:r1]), e, f"doc {i} {n}")


def test_route_over_a_grown_store_finds_new_documents():
    _banner("store append: routing finds a document planted in the newest batch")
    d = msa.dims()
    lengths = _lengths(63, 48)
    mem = synth.raw_memory(lengths, seed=63, device=DEV, plant_docs=[45])
    st = _grow(mem, [0, 32, 48], d)
    q = synth.route_query_planted_raw(mem, M=8, seed=63, device=DEV)
    ds, ids, sc, ns = msa.route_topk(q.QR, st.KRbar, st.doc_chunk_offsets, d)
    torch.cuda.synchronize()
    assert 45 in set(ids.cpu().numpy()[0].tolist())


def test_save_and_load_round_trip(tmp_path):
    _banner("store save/load round trip, partial loads, errors")
    d = msa.dims()
    mem = synth.raw_memory(_lengths(64, 24), seed=64, device=DEV)
    st = _grow(mem, [0, 10, 24], d)
    path = str(tmp_path / "mem.msastore")
    st.save(path, staging_bytes=1 << 20)   # forces several staging rounds
    assert msa.store_file_info(path) == (24, st.n_chunks, msa.STORE_KR | msa.STORE_K | msa.STORE_V)

    back = msa.Store(32, 4096, d=d)
    back.load(path)
    torch.cuda.synchronize()
    assert back.n_docs == 24 and back.n_chunks == st.n_chunks
    assert np.array_equal(back.offsets_h, st.offsets_h)
    assert np.array_equal(back.doc_chunk_offsets.cpu().numpy(), st.offsets_h)
    for a, b, n in ((back.Kbar, st.Kbar, "K"), (back.Vbar, st.Vbar, "V"), (back.KRbar, st.KRbar, "KR")):
        _same(a, b, n)

    # a router-only store loads just K̄^R (the K̄/V̄ sections are skipped)
    kr_only = msa.Store(32, 4096, d=d, tensors=("KR",))
    kr_only.load(path)
    torch.cuda.synchronize()
    _same(kr_only.KRbar, st.KRbar, "KR only")

    # too small, or other pooling settings: rejected before anything is written
    small = msa.Store(8, 4096, d=d)
    with pytest.raises(msa.MsaError) as e:
        small.load(path)
    assert e.value.code == -2 and small.n_docs == 0
    with pytest.raises(msa.MsaError) as e:
        msa.Store(32, 4096, d=msa.dims(doc_rope_mode=msa.DOC_ROPE_CHUNK)).load(path)
    assert e.value.code == -2

    # a truncated tensor section: I/O error, and the store is left empty
    raw = open(path, "rb").read()
    cut = str(tmp_path / "cut.msastore")
    open(cut, "wb").write(raw[:-4096])
    victim = msa.Store(32, 4096, d=d)
    victim.append(*_batch(mem, 0, 3))
    with pytest.raises(msa.MsaError) as e:
        victim.load(cut)
    assert e.value.code == -6 and victim.n_docs == 0 and victim.n_chunks == 0


def test_grow_after_load_and_host_tier(tmp_path):
    _banner("store: load, keep appending; pinned-host K̄/V̄ tier; capacity errors")
    d = msa.dims()
    mem = synth.raw_memory(_lengths(65, 36), seed=65, device=DEV)
    Kb, Vb, Rb, dco_h = _encode_all(mem, d)
    first = _grow(mem, [0, 20], d)
    path = str(tmp_path / "part.msastore")
    first.save(path)

    st = msa.Store(40, 2048, d=d, kv_on_host=True)
    assert st._K.device.type == "cpu" and st._K.is_pinned()
    st.load(path)
    st.append(*_batch(mem, 20, 36))
    torch.cuda.synchronize()
    assert np.array_equal(st.offsets_h, dco_h)
    _same(st.Kbar, Kb, "Kbar (host tier)")
    _same(st.Vbar, Vb, "Vbar (host tier)")
    _same(st.KRbar, Rb, "KRbar")

    # the full store does not take one more document; nothing changes
    before = (st.n_docs, st.n_chunks)
    with pytest.raises(msa.MsaError) as e:
        st.append(*_batch(mem, 0, 5))
    assert e.value.code == -2 and (st.n_docs, st.n_chunks) == before
    st.reset()
    assert st.n_docs == 0 and st.n_chunks == 0
