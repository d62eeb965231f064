"""The parity criteria themselves (tests/_util.py), on the CPU: they accept
every result a correct GPU path can give and reject the mistakes they exist
to catch."""
import numpy as np
import pytest

from oracle import msa_oracle as O
from tests._util import assert_attn_close, assert_topk_matches


def _scores():
    # 40 documents; ranks 0..3 well separated, then a dense band where
    # neighbouring scores are within 1e-3 (the margins are waived there)
    s = np.concatenate([[0.9, 0.8, 0.7, 0.6], 0.5 - 5e-4 * np.arange(36)])
    return np.random.default_rng(3).permutation(s)


def test_topk_accepts_the_oracle_and_near_ties():
    s = _scores()
    ids, _, _ = O.topk(s, 16)
    assert_topk_matches(np.array(ids), 16, s, 16)
    # swapping two neighbours inside the dense band is a valid result
    alt = list(ids)
    alt[8], alt[9] = alt[9], alt[8]
    assert_topk_matches(np.array(alt), 16, s, 16)
    # so is the k+1-th document in place of the k-th when they are 5e-4 apart
    order = sorted(range(len(s)), key=lambda i: (-s[i], i))
    alt = list(order[:15]) + [order[16]]
    assert_topk_matches(np.array(alt), 16, s, 16)


def test_topk_rejects_a_dropped_clear_winner():
    s = _scores()
    order = sorted(range(len(s)), key=lambda i: (-s[i], i))
    # rank-5 document (score 0.4995, neighbours within 1e-3, so no rank
    # or set rule applies) replaced by the 17th: > s_k + 2e-3, must be present
    bad = list(order[:5]) + list(order[6:16]) + [order[16]]
    with pytest.raises(AssertionError, match="not selected"):
        assert_topk_matches(np.array(bad), 16, s, 16)


def test_topk_rejects_ranks_out_of_order():
    s = _scores()
    order = sorted(range(len(s)), key=lambda i: (-s[i], i))
    bad = list(order[:16])
    bad[6], bad[14] = bad[14], bad[6]        # 4e-3 apart in the dense band
    with pytest.raises(AssertionError, match="ranked below"):
        assert_topk_matches(np.array(bad), 16, s, 16)


def test_attention_row_bound_catches_one_wrong_row():
    rng = np.random.default_rng(5)
    exp = rng.standard_normal((256, 32, 128))
    got = exp * (1 + 1e-3 * rng.standard_normal(exp.shape))
    assert_attn_close(got, exp)
    bad = got.copy()
    bad[17, 5] *= 1.5                         # one (token, head) row 50% off
    with pytest.raises(AssertionError, match="row \\(17, 5\\)"):
        assert_attn_close(bad, exp)
