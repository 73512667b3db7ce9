"""Host logic of the parity harness (no GPU): the kept-set rule for
low-margin sampled rows."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(__file__))
import harness  # noqa: E402

NI = -np.inf


def _row(vals):
    return np.asarray(vals, np.float32)


def test_kept_sets_equal():
    a = _row([3.0, NI, 1.0, 2.0])
    assert harness.kept_sets_agree(a, a.copy(), 3, 3)


def test_kept_sets_boundary_difference_allowed():
    # order: id 0 (3), id 3 (2), id 2 (1), id 1 (0.5); the oracle keeps 3,
    # the GPU keeps 2: a prefix of the same order, within [2, 3]
    o = _row([3.0, NI, 1.0, 2.0])
    g = _row([3.0, NI, NI, 2.0])
    assert harness.kept_sets_agree(g, o, 2, 3)
    assert not harness.kept_sets_agree(g, o, 3, 3)  # outside the allowed range


def test_kept_sets_not_a_prefix():
    o = _row([3.0, NI, 1.0, 2.0])
    g = _row([3.0, NI, 1.0, NI])  # drops id 3 but keeps the lower id 2
    assert not harness.kept_sets_agree(g, o, 2, 3)


def test_kept_sets_ties_in_id_order():
    # equal scores: the kept prefix takes the lower ids first
    o = _row([1.0, 1.0, 1.0, 1.0])
    assert harness.kept_sets_agree(_row([1.0, 1.0, NI, NI]), o, 2, 4)
    assert not harness.kept_sets_agree(_row([1.0, NI, 1.0, NI]), o, 2, 4)


def test_kept_sets_value_mismatch():
    o = _row([3.0, NI, 1.0, 2.0])
    g = _row([3.0, NI, 1.0000001, 2.0])
    assert not harness.kept_sets_agree(g, o, 3, 3)


def test_logprobs_agree_rule():
    one = np.float32(-1.25)
    assert harness.logprobs_agree(one, one)
    assert harness.logprobs_agree(np.nextafter(one, np.float32(0)), one)
    assert not harness.logprobs_agree(np.float32(-1.2501), one)
    qnan = np.array([0x7FC00000], np.uint32).view(np.float32)[0]
    assert harness.logprobs_agree(qnan, qnan)
    assert not harness.logprobs_agree(np.array([0xFFC00000], np.uint32).view(np.float32)[0], qnan)
    assert not harness.logprobs_agree(np.float32(0.0), qnan)


def test_logprob_of_row():
    row = np.log(np.array([1.0, 2.0, 3.0, 4.0], np.float32)).astype(np.float32)
    assert abs(float(harness.logprob_of(row, 3)) - np.log(0.4)) < 3e-7
    row[0] = -np.inf  # kept set 2:3:4
    assert abs(float(harness.logprob_of(row, 1)) - np.log(2 / 9)) < 3e-7
    assert np.isnan(harness.logprob_of(np.full(3, -np.inf, np.float32), 0))
