"""Router supervision (msa_route_aux_loss) against the oracle, through the C ABI.

Where a document's maximising chunk or token is not unique within the
kernels' precision, several subgradients are correct: the test checks that
the GPU's (chunk, token) choice of every document is a valid maximiser
(within the scan's score tolerance) and compares loss, document scores and
gradients with the oracle evaluated at those same choices.
"""
import numpy as np
import pytest
import torch

import routed_sparse_attention_amd as msa
import synth
from oracle import msa_oracle as O
from tests._util import u16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _case(B, M, n_docs, seed):
    rng = np.random.default_rng(seed)
    counts = rng.integers(1, 9, size=n_docs)
    store = synth.pooled_store(counts, seed=seed, device=DEV)
    g = synth.torch_gen(seed, 31, DEV)
    QR = synth.randn_bf16((B, M, 8, 128), g, DEV)
    return store, QR


def _close(gpu, ref, what, rel=2e-3):
    gpu = np.asarray(gpu, dtype=np.float64)
    scale = max(np.abs(ref).max(), 1e-30)
    err = np.abs(gpu - ref)
    bad = err > rel * scale + 1e-3 * np.abs(ref)
    assert not bad.any(), f"{what}: max err {err.max():.3e} vs scale {scale:.3e}"


@pytest.mark.parametrize("B,M,n_docs,tau,seed", [
    (1, 1, 40, 0.05, 71),     # decode shape (VALU scan)
    (2, 3, 30, 0.1, 72),      # small batch (MFMA scan, 6 rows)
    (12, 1, 50, 0.05, 73),    # batched single tokens (MFMA scan)
    (3, 17, 25, 0.2, 74),     # queries longer than one 16-row segment (MFMA, parts)
    (1, 40, 20, 0.5, 75),
])
def test_aux_loss_matches_oracle(B, M, n_docs, tau, seed):
    _banner(f"aux loss B={B} M={M} docs={n_docs} tau={tau}")
    store, QR = _case(B, M, n_docs, seed)
    rng = np.random.default_rng(seed + 1)
    positives = [sorted(set(int(x) for x in rng.choice(n_docs, size=1 + b % 3, replace=False)))
                 for b in range(B)]
    dco_h = store.doc_chunk_offsets
    dco = torch.from_numpy(dco_h).to(DEV)
    loss, dQ, dK, ds, bc, bt = msa.route_aux_loss(QR, store.KRbar, dco, positives, tau)
    torch.cuda.synchronize()
    bc, bt = bc.cpu().numpy(), bt.cpu().numpy()
    # the GPU's choices are valid maximisers
    ref_free = O.route_aux_loss(u16(QR), u16(store.KRbar), dco_h, positives, tau)
    q = O.bf16_to_f64(u16(QR))
    k = O.bf16_to_f64(u16(store.KRbar))
    qh = q / np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), O.NORM_EPS)
    kh = k / np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), O.NORM_EPS)
    for b in range(B):
        for i in range(n_docs):
            c, t = int(bc[b, i]), int(bt[b, i])
            assert dco_h[i] <= c < dco_h[i + 1] and 0 <= t < M
            at = np.einsum("hd,hd->h", qh[b, t], kh[c]).mean()
            assert at >= ref_free[3][b, i] - 2e-4, (b, i, at, ref_free[3][b, i])
    # everything else at those choices
    loss_o, dQ_o, dK_o, s_o, *_ = O.route_aux_loss(u16(QR), u16(store.KRbar), dco_h, positives,
                                                    tau, choice=(bc, bt))
    np.testing.assert_allclose(ds.cpu().numpy(), s_o, atol=2e-6, rtol=0)
    np.testing.assert_allclose(loss.cpu().numpy(), loss_o, atol=1e-4, rtol=1e-4)
    _close(dQ.cpu().numpy(), dQ_o, "dQR")
    _close(dK.cpu().numpy(), dK_o, "dKRbar")


def test_aux_loss_positive_lists_and_errors():
    _banner("aux loss: repeated / invalid positives, a query without positives, errors")
    B, M, n_docs, tau = 3, 2, 30, 0.1
    store, QR = _case(B, M, n_docs, 76)
    dco_h = store.doc_chunk_offsets
    dco = torch.from_numpy(dco_h).to(DEV)
    given = [[4, 4, 9, -3, 1000], [], [29]]
    clean = [[4, 9], [], [29]]
    loss, dQ, dK, ds, bc, bt = msa.route_aux_loss(QR, store.KRbar, dco, given, tau)
    torch.cuda.synchronize()
    bc, bt = bc.cpu().numpy(), bt.cpu().numpy()
    # the query without positives: loss 0 and no gradient from it
    assert loss[1].item() == 0.0 and not dQ[1].any()
    lo, dQo, dKo, *_ = O.route_aux_loss(u16(QR[[0, 2]]), u16(store.KRbar), dco_h, [clean[0], clean[2]],
                                        tau, choice=(bc[[0, 2]], bt[[0, 2]]))
    np.testing.assert_allclose(loss.cpu().numpy()[[0, 2]], lo, atol=1e-4, rtol=1e-4)
    _close(dQ.cpu().numpy()[[0, 2]], dQo, "dQR")
    _close(dK.cpu().numpy(), dKo, "dKRbar")
    with pytest.raises(msa.MsaError) as e:
        msa.route_aux_loss(QR, store.KRbar, dco, clean, 0.0)
    assert e.value.code == -1
    with pytest.raises(msa.MsaError) as e:
        msa.route_aux_loss(QR, store.KRbar, dco, clean, 0.1, d=msa.dims(token_reduce=1))
    assert e.value.code == -5


def test_aux_loss_gradient_step_lowers_the_loss():
    """A small step along −gradient lowers the loss (the planted positive's
    score rises relative to the rest); checked with the GPU's own loss."""
    _banner("aux loss: a gradient step lowers the loss")
    B, M, n_docs, tau = 2, 4, 40, 0.1
    store, QR = _case(B, M, n_docs, 77)
    dco = torch.from_numpy(store.doc_chunk_offsets).to(DEV)
    pos = [[3], [17, 30]]
    loss, dQ, dK, *_ = msa.route_aux_loss(QR, store.KRbar, dco, pos, tau)
    step = 0.05 / max(dQ.abs().max().item(), dK.abs().max().item())
    QR2 = (QR.float() - step * dQ).to(torch.bfloat16)
    KR2 = (store.KRbar.float() - step * dK).to(torch.bfloat16)
    loss2 = msa.route_aux_loss(QR2, KR2, dco, pos, tau)[0]
    torch.cuda.synchronize()
    assert (loss2 < loss).all(), (loss.tolist(), loss2.tolist())
