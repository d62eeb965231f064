"""Helpers shared by the tests: tensor conversion and the parity criteria.

Parity criteria (the tolerances stated for the MSA hot path):
  - pooled bf16 tensors: within 1 bf16 ulp of the oracle, compared as
    monotone integer codes (|ord(a) − ord(b)| <= 1);
  - routing scores: within 1e-3 absolute;
  - selected document ids: the selected *set* must equal the oracle's when the
    oracle's gap between rank k and rank k+1 exceeds 1e-3, and the id at rank r
    must equal the oracle's when the gaps on both sides of rank r exceed 1e-3;
    every selected id must in any case be a document whose oracle score is
    within 2e-3 of the oracle's k-th score (a valid choice under 1e-3 error);
    every document whose oracle score exceeds the k-th by more than 2e-3 must
    be selected; and the selected ranks must be non-increasing in oracle
    score up to 2e-3. (With every GPU score within 1e-3 of the oracle's, a
    correct select can violate none of these.)
  - attention output: relative L2 error <= 1e-2 over the whole output, and
    <= 3e-2 for every (token, head) row of 128 values. The row bound is three
    times the global one: one row is 128 values, so its error estimate is
    noisier than the global one, but a row that is wrong by more than a few
    per cent fails it however many correct rows surround it.
"""
import numpy as np
import torch

from oracle import msa_oracle as O

SCORE_TOL = 1e-3
MARGIN = 1e-3
ATTN_REL_L2 = 1e-2
ATTN_ROW_REL_L2 = 3e-2


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def assert_pooled_close(got_bits, exp_bits, what=""):
    d = np.abs(O.bf16_ord(got_bits) - O.bf16_ord(exp_bits))
    assert d.max() <= 1, f"{what}: pooled values differ by up to {d.max()} bf16 ulp " \
                         f"({int((d > 1).sum())} values beyond 1 ulp)"
    return int((d == 1).sum())


def assert_scores_close(got, exp, what=""):
    got = np.asarray(got, dtype=np.float64)
    exp = np.asarray(exp, dtype=np.float64)
    both_nan = np.isnan(got) & np.isnan(exp)
    err = np.where(both_nan, 0.0, np.abs(got - exp))
    assert not np.any(np.isnan(err)), f"{what}: NaN mismatch"
    assert err.max() <= SCORE_TOL, f"{what}: max score error {err.max():.3e}"
    return float(err.max())


def assert_topk_matches(got_ids, got_nsel, exp_scores_all, k):
    """got_ids: GPU ids [k] (-1 padded), exp_scores_all: oracle doc scores [N]."""
    exp_ids, exp_sc, margins = O.topk(exp_scores_all, k)
    n_sel = len(exp_ids)
    assert int(got_nsel) == n_sel, f"n_sel {got_nsel} != {n_sel}"
    got = [int(x) for x in got_ids[:n_sel]]
    assert all(x == -1 for x in got_ids[n_sel:]), "entries past n_sel must be -1"
    # gap before rank r (r=0 has none) and after rank r
    before = np.concatenate([[np.inf], margins[:-1]])
    after = margins
    for r in range(n_sel):
        if before[r] > MARGIN and after[r] > MARGIN:
            assert got[r] == int(exp_ids[r]), f"rank {r}: id {got[r]} != oracle {exp_ids[r]}"
    if margins[-1] > MARGIN:
        assert set(got) == set(int(x) for x in exp_ids), "selected set differs from the oracle"
    kth = exp_sc[-1]
    s = np.asarray(exp_scores_all, dtype=np.float64)
    for x in got:
        assert 0 <= x < len(s), f"id {x} out of range"
        if not np.isnan(kth):
            assert s[x] >= kth - 2 * MARGIN, f"id {x} (score {s[x]}) is not a valid top-{k} choice"
    assert len(set(got)) == len(got), "duplicate ids"
    if not np.isnan(kth):
        # every document clearly above the k-th must be there
        clear = np.flatnonzero(~np.isnan(s) & (s > kth + 2 * MARGIN))
        missing = sorted(set(int(x) for x in clear) - set(got))
        assert not missing, f"documents {missing[:8]} score > s_k + {2 * MARGIN} but are not selected"
        # ranks follow the oracle's scores up to the combined error
        sg = s[np.array(got, dtype=np.int64)] if got else np.zeros(0)
        sg = np.where(np.isnan(sg), -np.inf, sg)     # a NaN score ranks last
        run_min = np.minimum.accumulate(sg) if len(sg) else sg
        for r in range(1, len(sg)):
            assert sg[r] <= run_min[r - 1] + 2 * MARGIN, \
                f"rank {r}: id {got[r]} (oracle {sg[r]:.6f}) ranked below a lower-scoring id"


def attn_row_errors(got, exp):
    """Relative L2 error of every (token, head) row of 128 values."""
    got = np.asarray(got, dtype=np.float64)
    exp = np.asarray(exp, dtype=np.float64)
    num = np.linalg.norm(got - exp, axis=-1)
    den = np.maximum(np.linalg.norm(exp, axis=-1), 1e-30)
    return num / den


def assert_attn_close(got, exp, what=""):
    got = np.asarray(got, dtype=np.float64)
    exp = np.asarray(exp, dtype=np.float64)
    assert got.shape == exp.shape, f"{what}: shape {got.shape} != {exp.shape}"
    rel = np.linalg.norm(got - exp) / max(np.linalg.norm(exp), 1e-30)
    assert rel <= ATTN_REL_L2, f"{what}: attention relative L2 error {rel:.3e}"
    rows = attn_row_errors(got, exp)
    worst = np.unravel_index(int(np.argmax(rows)), rows.shape)
    assert rows.max() <= ATTN_ROW_REL_L2, \
        f"{what}: row {tuple(int(i) for i in worst)} relative L2 error {rows.max():.3e}"
    return float(rel)
