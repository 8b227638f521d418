"""CPU checks of the test helpers themselves: the exact prefix check of selected sets."""
import numpy as np
import pytest

from tests import parity as P
from oracle import rtp_oracle as O


def test_check_prefix_accepts_prefixes_and_rejects_others():
    s = np.float32([3, 1, 2, 2, 2, -0.0, 0.0, 5])
    P.check_prefix(np.array([0, 7]), s)
    P.check_prefix(np.array([0, 2, 3, 7]), s)                 # ties at 2: lowest indices first
    P.check_prefix(np.array([0, 1, 2, 3, 4, 5, 7]), s)        # -0 and +0 tie: index 5 first
    for bad in ([0, 3, 4, 7], [0, 1, 2, 3, 4, 6, 7], [0], [1, 7]):
        with pytest.raises(AssertionError):
            P.check_prefix(np.sort(np.array(bad)), s)


def test_oracle_sets_are_prefixes_of_the_score_order():
    rng = np.random.default_rng(5)
    for p in (0.3, 0.9, 0.99):
        s = np.round(rng.standard_normal(3000), 1)             # many exact ties
        sel, _ = O.topp_select(s, p)
        P.check_prefix(np.sort(sel), s.astype(np.float32))
