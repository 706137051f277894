"""Which learners a merge takes, and their weights (Decoupled DiLoCo digest,
"fault tolerance" items 1-3: minimum quorum, a bounded grace wait, token-weighted
merge): the library's host function against the oracle, on hand-worked and
random cases.  No GPU needed."""
import math

import numpy as np
import pytest

import diloco_outer_step_amd as dlc
import oracle

INF = math.inf


HAND_WORKED = [
    # quorum met at the 2nd arrival (t = 2); grace 0.5 -> deadline 2.5: learners 0 and 2
    ([100, 200, 300, 0], [1.0, 3.0, 2.0, INF], 2, 0.5, [100, 0, 300, 0], 2.5),
    # everyone arrived before the deadline: merge at the last arrival
    ([100, 200, 300, 50], [1.0, 3.0, 2.0, 2.2], 2, 5.0, [100, 200, 300, 50], 3.0),
    # quorum of one, no grace: only the earliest (ties: lower index first, both at t = 1)
    ([10, 20, 30], [1.0, 1.0, 4.0], 1, 0.0, [10, 20, 0], 1.0),
    # a learner arriving exactly at the deadline is taken
    ([1, 1, 1], [0.0, 0.5, 1.5], 1, 1.5, [1, 1, 1], 1.5),
    # NaN = not arrived
    ([5, 7], [float("nan"), 3.0], 1, 1.0, [0, 7], 4.0),
]


def oracle_matches_hand_worked_tables():
    for tokens, arrival, quorum, grace, want_w, want_t in HAND_WORKED:
        w, t = oracle.merge_weights(tokens, arrival, quorum, grace)
        assert w == [float(x) for x in want_w] and t == want_t


@pytest.mark.parametrize("tokens, arrival, quorum, grace, want_w, want_t", HAND_WORKED)
def test_hand_worked(tokens, arrival, quorum, grace, want_w, want_t):
    w, t = dlc.dlc_merge_weights(tokens, arrival, quorum, grace)
    assert w == [float(x) for x in want_w] and t == want_t
    ow, ot = oracle.merge_weights(tokens, arrival, quorum, grace)
    assert ow == w and ot == t


@pytest.mark.parametrize("tokens, arrival, quorum", [
    ([1, 1, 1], [0.0, INF, INF], 2),      # too few arrived
    ([0, 0, 5], [0.0, 0.1, 9.0], 2),      # the merged learners processed no tokens
])
def test_no_quorum(tokens, arrival, quorum):
    with pytest.raises(dlc.NoQuorumError):
        dlc.dlc_merge_weights(tokens, arrival, quorum, 1.0)
    with pytest.raises(oracle.NoQuorum):
        oracle.merge_weights(tokens, arrival, quorum, 1.0)


def test_random_against_oracle():
    rng = np.random.default_rng(0)
    checked = 0
    for _ in range(2000):
        k = int(rng.integers(1, 17))
        tokens = [float(x) for x in rng.integers(0, 5, k) * 1000]
        arrival = [float(x) if rng.random() > 0.25 else INF for x in np.round(rng.uniform(0, 10, k), 1)]
        quorum = int(rng.integers(1, k + 1))
        grace = float(np.round(rng.uniform(0, 3), 1))
        try:
            want = oracle.merge_weights(tokens, arrival, quorum, grace)
        except oracle.NoQuorum:
            with pytest.raises(dlc.NoQuorumError):
                dlc.dlc_merge_weights(tokens, arrival, quorum, grace)
            continue
        assert dlc.dlc_merge_weights(tokens, arrival, quorum, grace) == want
        checked += 1
    assert checked > 500


@pytest.mark.parametrize("args", [
    ([1.0], [0.0], 0, 0.0),           # quorum below 1
    ([1.0], [0.0], 2, 0.0),           # quorum above K
    ([1.0], [0.0], 1, -1.0),          # negative grace
    ([1.0], [0.0], 1, INF),           # unbounded grace
    ([-1.0], [0.0], 1, 0.0),          # negative tokens of an arrived learner
    ([1.0], [-2.0], 1, 0.0),          # negative arrival time
])
def test_argument_errors(args):
    with pytest.raises(dlc.DlcError) as e:
        dlc.dlc_merge_weights(*args)
    assert e.value.code == dlc.DLC_ERR_INVALID_ARGUMENT
