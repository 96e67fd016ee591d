"""Host-side logic of the geometry tuner: candidate validation and the choice
rule (no GPU needed)."""
import numpy as np
import pytest

from decode_gemv_byte_amd import tune
from decode_gemv_byte_amd.tune import Candidate


def test_default_candidates_are_valid_and_distinct():
    c = tune.check_candidates(tune.DEFAULT_CANDIDATES)
    assert len(c) == len(set(c)) == len(tune.DEFAULT_CANDIDATES)
    assert (8, 8) in c   # the library default is always among them


@pytest.mark.parametrize("bad", [[(3, 8)], [(128, 8)], [(0, 8)], [(8, 5)], [(8, 13)], []])
def test_invalid_candidates_rejected(bad):
    with pytest.raises(ValueError):
        tune.check_candidates(bad)


def test_duplicates_dropped_in_order():
    assert tune.check_candidates([(16, 8), (8, 8), (16, 8)]) == [(16, 8), (8, 8)]


def test_pick_fastest_and_size_slack():
    a = Candidate(4, 8, 1100, 10.0)
    b = Candidate(8, 8, 1000, 10.05)
    c = Candidate(16, 8, 990, 11.0)
    assert tune.pick([a, b, c]) is a
    # within 1% of the fastest, the smaller blob wins
    assert tune.pick([a, b, c], size_slack=0.01) is b
    # a slack that reaches every candidate picks the smallest overall
    assert tune.pick([a, b, c], size_slack=0.2) is c


def test_tune_rejects_bad_inputs_before_touching_a_gpu():
    w = np.zeros((8, 8), np.uint16)
    with pytest.raises(ValueError):
        tune.tune_geometry(w.astype(np.int32))
    with pytest.raises(ValueError):
        tune.tune_geometry(w, batch=33)
    with pytest.raises(ValueError):
        tune.tune_geometry([w] * 9)
    with pytest.raises(ValueError):
        tune.tune_geometry([])
