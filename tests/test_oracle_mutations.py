"""Planted mistakes in the CPU oracle must each fail at least one pin.

Each case swaps one oracle function (or constant) for a plausible wrong version,
runs the pins that should notice, and expects an AssertionError.  Everything
runs on the CPU; the real oracle is restored after each case.
"""
import numpy as np
import pytest

import oracle
import oracle.core as core
from tests import test_merge_policy as mp
from tests import test_oracle_pins as pins


def _patch(monkeypatch, name, value):
    monkeypatch.setattr(core, name, value)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, value)


def _sample_std(x):
    x64 = np.asarray(x, np.float32).astype(np.float64)
    mu = float(np.mean(x64))
    return mu, float(np.sqrt(np.sum((x64 - mu) ** 2) / (x64.size - 1)))


def _midpoint_codebook(s, n, lo, wd):
    return np.array([np.float32(float(lo) + (c + 0.5) * float(wd)) for c in range(256)], np.float32)


def _wrong_sign(a, b):
    return np.subtract(np.asarray(b, np.float32), np.asarray(a, np.float32), dtype=np.float32)


def _unnormalized(w):
    return [float(v) for v in w]


def _heavy_ball(theta, momentum, g, lr=0.7, beta=0.9):
    th = np.asarray(theta, np.float32).astype(np.float64)
    v = beta * np.asarray(momentum, np.float32).astype(np.float64) + np.asarray(g, np.float64)
    return (th - lr * v).astype(np.float32), v.astype(np.float32)


def _round_not_floor(x, lo, wd):
    t = np.subtract(np.asarray(x, np.float32), np.float32(lo), dtype=np.float32)
    q = np.divide(t, np.float32(wd), dtype=np.float32)
    return np.clip(np.rint(q), 0, 255).astype(np.uint8)


def _lpt_last_tie(numel, n_fragments):
    loads = [0] * n_fragments
    frag = [0] * len(numel)
    for t in sorted(range(len(numel)), key=lambda t: (-numel[t], t)):
        best = max(range(n_fragments), key=lambda p: (-loads[p], p))
        frag[t] = best
        loads[best] += numel[t]
    return frag, loads


def _rda_parts(codes_per_learner, codebook_per_learner, w_hat):
    xs = [(w, oracle.dequantize(c, cb).astype(np.float64))
          for c, cb, w in zip(codes_per_learner, codebook_per_learner, w_hat) if w != 0.0]
    return xs, [float(np.sqrt(np.sum(x * x))) for _, x in xs]


def _rda_no_renormalize(codes_per_learner, codebook_per_learner, w_hat):
    xs, rs = _rda_parts(codes_per_learner, codebook_per_learner, w_hat)
    r = sum(w * ri for (w, _), ri in zip(xs, rs))
    return r * sum(w * (x / ri) for (w, x), ri in zip(xs, rs) if ri > 0)


def _rda_plain_mean(codes_per_learner, codebook_per_learner, w_hat):
    xs, rs = _rda_parts(codes_per_learner, codebook_per_learner, w_hat)
    return sum(w * x for w, x in xs)


def _rda_unweighted_norm(codes_per_learner, codebook_per_learner, w_hat):
    xs, rs = _rda_parts(codes_per_learner, codebook_per_learner, w_hat)
    r = sum(rs) / len(rs)
    d = sum(w * (x / ri) for (w, x), ri in zip(xs, rs) if ri > 0)
    return r * d / np.sqrt(np.sum(d * d))


def _rda_exact_zero_test(codes_per_learner, codebook_per_learner, w_hat):
    xs, rs = _rda_parts(codes_per_learner, codebook_per_learner, w_hat)
    r = sum(w * ri for (w, _), ri in zip(xs, rs))
    d = sum(w * (x / ri) for (w, x), ri in zip(xs, rs) if ri > 0)
    dn = float(np.sqrt(np.sum(d * d)))
    return r * d / dn if dn > 0.0 else np.zeros_like(d)


_OUTER_STEP = core.outer_step


def _step_ignoring_rule(*args, rule="mean", **kwargs):
    return _OUTER_STEP(*args, **kwargs)


def _ring_wrong_direction(rank, hop, k):
    return (rank + hop) % k


def _ring_exact_messages(x):
    q = core.quantize_tensor(x)
    return q, np.asarray(x, np.float32)


def _grace_exclusive(tokens, arrival, quorum, grace):
    k = len(tokens)
    came = [i for i in range(k) if np.isfinite(arrival[i])]
    if len(came) < quorum:
        raise core.NoQuorum("quorum")
    t_q = arrival[sorted(came, key=lambda i: (arrival[i], i))[quorum - 1]]
    w = [float(tokens[i]) if i in came and arrival[i] < t_q + grace else 0.0 for i in range(k)]
    if sum(w) <= 0:
        raise core.NoQuorum("tokens")
    return w, float(t_q + grace)


def _quorum_off_by_one(tokens, arrival, quorum, grace):
    return _orig_merge_weights(tokens, arrival, min(quorum + 1, len(tokens)), grace)


_orig_merge_weights = core.merge_weights


def _broadcast_all_rows(theta_g, theta_L, tensors, rows=None):
    return _orig_broadcast(theta_g, theta_L, tensors, None)


_orig_broadcast = core.broadcast


def _bases_ignored(theta_g, momentum, theta_L, learner_stride, tensors, weights, present=None, lr=0.7, beta=0.9,
                   given_ranges=None, bases=None, rule="mean"):
    return _orig_outer_step(theta_g, momentum, theta_L, learner_stride, tensors, weights, present, lr, beta,
                            given_ranges, None, rule)


_orig_outer_step = core.outer_step


MUTATIONS = {
    "clip_at_5_sigma": (lambda mp: _patch(mp, "CLIP_SIGMAS", 5.0),
                        [pins.test_worked_example_range_from_printed_sigma]),
    "sample_std": (lambda mp: _patch(mp, "tensor_stats", _sample_std),
                   [pins.test_stats_arithmetic_progression]),
    "midpoint_codebook": (lambda mp: _patch(mp, "codebook", _midpoint_codebook),
                          [lambda: pins.test_histogram_and_codebook_bruteforce(0)]),
    "pseudo_gradient_sign": (lambda mp: _patch(mp, "pseudo_gradient", _wrong_sign),
                             [pins.test_fedavg_reduction_pins_the_sign]),
    "weights_not_normalized": (lambda mp: _patch(mp, "normalize_weights", _unnormalized),
                               [pins.test_merge_identical_learners]),
    "heavy_ball_not_nesterov": (lambda mp: _patch(mp, "nesterov", _heavy_ball),
                                [pins.test_nesterov_closed_form_constant_g,
                                 pins.test_nesterov_matches_torch_sgd]),
    "round_not_floor": (lambda mp: _patch(mp, "encode", _round_not_floor),
                        [pins.test_encode_exact_grid_boundaries]),
    "lpt_ties_to_last_fragment": (lambda mp: _patch(mp, "fragment_plan", _lpt_last_tie),
                                  [pins.test_lpt_hand_worked]),
    "rda_direction_not_renormalized": (lambda mp: _patch(mp, "rda_merge", _rda_no_renormalize),
                                       [lambda: pins.test_rda_norm_is_the_weighted_mean_norm(0)]),
    "rda_plain_mean": (lambda mp: _patch(mp, "rda_merge", _rda_plain_mean),
                       [pins.test_rda_two_equal_weights_bisect_the_angle,
                        lambda: pins.test_rda_orthogonal_halves_closed_form(3.0, 1.0)]),
    "rda_null_direction_tested_exactly": (lambda mp: _patch(mp, "rda_merge", _rda_exact_zero_test),
                                          [lambda: pins.test_rda_balanced_constant_learners_give_zero(2)]),
    "cycle_ignores_the_merge_rule": (lambda mp: _patch(mp, "outer_step", _step_ignoring_rule),
                                     [pins.test_rda_cycle_is_not_the_mean_cycle]),
    "rda_unweighted_norm": (lambda mp: _patch(mp, "rda_merge", _rda_unweighted_norm),
                            [lambda: pins.test_rda_norm_is_the_weighted_mean_norm(0)]),
    "ring_chunks_travel_the_wrong_way": (lambda mp: _patch(mp, "ring_sent_chunk", _ring_wrong_direction),
                                         [lambda: pins.test_ring_on_constant_chunks_is_the_ring_order_fp32_mean(3)]),
    "ring_without_requantization": (lambda mp: _patch(mp, "ring_message", _ring_exact_messages),
                                    [pins.test_ring_error_exceeds_the_star_and_grows_with_the_ring]),
    "grace_deadline_exclusive": (lambda mp: _patch(mp, "merge_weights", _grace_exclusive),
                                 [mp.oracle_matches_hand_worked_tables]),
    "quorum_off_by_one": (lambda mp: _patch(mp, "merge_weights", _quorum_off_by_one),
                          [mp.oracle_matches_hand_worked_tables]),
    "broadcast_ignores_rows": (lambda mp: _patch(mp, "broadcast", _broadcast_all_rows),
                               [pins.test_broadcast_copies_exactly_and_only_the_tensors]),
    "stale_bases_ignored": (lambda mp: _patch(mp, "outer_step", _bases_ignored),
                            [pins.test_stale_learner_without_progress_only_dilutes_the_others]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(monkeypatch, name):
    apply, checks = MUTATIONS[name]
    apply(monkeypatch)
    for check in checks:
        with pytest.raises(AssertionError):
            check()


def test_width_over_255_is_caught(monkeypatch):
    orig = core.clip_range

    def width_255(mu, sigma):
        lo, hi, _, m, deg = orig(mu, sigma)
        return lo, hi, np.float32(12 * sigma / 255), m, deg

    _patch(monkeypatch, "clip_range", width_255)
    with pytest.raises(AssertionError):
        pins.test_worked_example_4096x4096()


def test_unclipped_codebook_is_caught(monkeypatch):
    """Averaging raw instead of clipped values moves the edge entries outside the range."""
    orig = core.clip_values
    _patch(monkeypatch, "clip_values", lambda x, lo, hi: np.asarray(x, np.float32))
    with pytest.raises(AssertionError):
        pins.test_histogram_and_codebook_bruteforce(0)
    _patch(monkeypatch, "clip_values", orig)
