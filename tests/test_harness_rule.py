"""The comparison rule of the parity tests (CPU only): which GPU/oracle mismatches are excused.

A mismatch is excused only by the margin of the decision where the two sides part ways, or by
the top-p margin of a row of that same position; a near-boundary row elsewhere excuses nothing.
"""
import numpy as np

import harness as H
from oracle import spec_oracle as O


def _result(num_accepted, tokens, decisions, gamma=3):
    nan = np.full(gamma, np.nan)
    return O.RequestResult(num_accepted=num_accepted, tokens=tokens, status=0, p_y=nan, q_y=nan,
                           one_minus_tv=nan, tv=nan, draft_entropy_bits=nan, draft_max_prob=nan,
                           target_entropy_bits=np.full(gamma + 1, np.nan),
                           target_max_prob=np.full(gamma + 1, np.nan), req_stats=np.full(4, np.nan),
                           decisions=decisions)


D = O.Decision


def test_count_mismatch_uses_the_accept_margin_at_the_first_differing_position():
    # the oracle accepted position 1 and rejected position 2
    ref = _result(1, [5, 9], [D("accept", 1, 0.3), D("accept", 2, 5e-7), D("sample", 2, 0.2)])
    assert H._first_divergence_excused(ref, 2, [5, 6, 1, -1])       # GPU accepted 2: margin 5e-7
    assert H._first_divergence_excused(ref, 3, [5, 6, 7, 2])        # still decided at position 2
    ref = _result(1, [5, 9], [D("accept", 1, 4e-7), D("accept", 2, 0.4), D("sample", 2, 0.2)])
    assert H._first_divergence_excused(ref, 0, [3, -1, -1, -1])     # GPU rejected position 1
    assert not H._first_divergence_excused(ref, 2, [5, 6, 1, -1])   # position 2 was far from a


def test_token_mismatch_uses_the_sample_margin():
    ref = _result(1, [5, 9], [D("accept", 1, 0.3), D("accept", 2, 0.2), D("sample", 2, 3e-7)])
    assert H._first_divergence_excused(ref, 1, [5, 8, -1, -1])
    ref = _result(1, [5, 9], [D("accept", 1, 0.3), D("accept", 2, 2e-7), D("sample", 2, 0.2)])
    assert not H._first_divergence_excused(ref, 1, [5, 8, -1, -1])  # the accept margin is not it


def test_topp_margin_counts_only_for_the_rows_of_that_position():
    dec = [D("accept", 1, 0.3), D("accept", 2, 0.25), D("sample", 2, 0.2),
           D("topp", 1, 0.1, "target"), D("topp", 3, 1e-8, "target"), D("topp", 4, 1e-8, "target")]
    ref = _result(1, [5, 9], dec)
    # the old rule excused any request holding a near-boundary top-p row; rows 3 and 4 decide
    # nothing here
    assert not H._first_divergence_excused(ref, 1, [5, 8, -1, -1])
    assert not H._first_divergence_excused(ref, 2, [5, 6, 1, -1])
    ref = _result(1, [5, 9], dec + [D("topp", 2, 5e-7, "draft")])
    assert H._first_divergence_excused(ref, 1, [5, 8, -1, -1])      # draft row 2 decides position 2
    assert H._first_divergence_excused(ref, 2, [5, 6, 1, -1])


def test_bonus_draw_and_rejections_without_an_accept_decision():
    # every draft accepted: the emitted token is the bonus draw at position gamma + 1
    ref = _result(3, [1, 2, 3, 4], [D("accept", i, 0.2) for i in (1, 2, 3)] + [D("sample", 4, 6e-7)])
    assert H._first_divergence_excused(ref, 3, [1, 2, 3, 7])
    # a zero-q rejection at position 1 records no accept decision: only a top-p row can excuse it
    ref = _result(0, [4], [D("sample", 1, 0.3)])
    assert not H._first_divergence_excused(ref, 1, [4, 2, -1, -1])
    ref = _result(0, [4], [D("sample", 1, 0.3), D("topp", 1, 2e-7, "draft")])
    assert H._first_divergence_excused(ref, 1, [4, 2, -1, -1])


def test_report_bar():
    r = H.Report()
    r.draws, r.excused = 20000, 2
    assert r.ok()
    r.excused = 3
    assert not r.ok()
