"""Pins of the oracle's GRPO token ratio and clipped surrogate ("QeRL: When Quantized Weights Help Reinforcement
Learning, and Where the Evidence Stops", §2.3: rho = exp(log pi_theta - log pi_b), surrogate = the smaller of rho A
and its clipped-ratio version; §2.2: group-relative advantages).

Pinned against: the on-policy case (rho = 1 makes the surrogate the advantage itself), the pages' worked advantages
for rewards [1, 0, 0, 0] (they sum to zero, so the on-policy loss vanishes), the four one-sided clipping cases in
closed form, central finite differences of the loss for the gradient, and the two aggregations agreeing when every
response has the same length.
"""
import math

import numpy as np
import pytest

from conftest import read_golden


def case(orc, seed, n_seq=6, t_max=20, spread=0.3):
    rng = np.random.default_rng(seed)
    logp_old = (-rng.exponential(2.0, (n_seq, t_max))).astype(np.float32)
    logp = (logp_old + rng.normal(0.0, spread, (n_seq, t_max))).astype(np.float32)
    lengths = rng.integers(0, t_max + 1, n_seq).astype(np.int32)
    adv = rng.normal(0.0, 1.0, n_seq).astype(np.float32)
    return logp, logp_old, lengths, adv


def test_on_policy_surrogate_is_the_advantage(orc):
    logp, _, lengths, adv = case(orc, 1)
    sur, grad, st = orc.grpo_surrogate(logp, logp, lengths, adv)
    for i, L in enumerate(lengths):
        assert np.all(sur[i, :L] == np.float64(adv[i]))
        assert np.all(sur[i, L:] == 0.0) and np.all(grad[i, L:] == 0.0)
    n = lengths.sum()
    assert st["tokens"] == n and st["clipped"] == 0
    assert st["ratio_min"] == 1.0 and st["ratio_max"] == 1.0 and st["ratio_mean"] == 1.0
    assert math.isclose(st["loss"], -float((adv.astype(np.float64) * lengths).sum()) / n, rel_tol=1e-14)


def test_worked_advantages_give_zero_on_policy_loss(orc):
    """The pages' example: rewards [1, 0, 0, 0] -> advantages [sqrt3, -1/sqrt3 x 3]. They sum to zero, so with one
    token-mean over responses of equal length the on-policy loss is zero (to rounding) and each token's gradient is
    -A / (number of tokens)."""
    rewards, expr = read_golden("advantage_example.txt")[0].split("|")
    assert rewards.split() == ["1", "0", "0", "0"]
    adv = np.array([eval(e, {"__builtins__": {}, "sqrt": math.sqrt}) for e in expr.split()], dtype=np.float32)
    assert math.isclose(float(adv[0]), math.sqrt(3), rel_tol=1e-7)
    T = 7
    lp = np.full((4, T), -1.25, dtype=np.float32)
    for agg in (0, 1):
        sur, grad, st = orc.grpo_surrogate(lp, lp, np.full(4, T, np.int32), adv, agg=agg)
        assert abs(st["loss"]) < 1e-7
        assert np.allclose(grad, -np.repeat(adv[:, None], T, 1).astype(np.float64) / (4 * T), rtol=1e-15, atol=0)


@pytest.mark.parametrize("A,delta,expect_clipped", [
    (1.5, math.log(1.6), True),     # A > 0, rho above 1 + eps: capped at (1 + eps) A, no gradient
    (-0.7, math.log(0.5), True),    # A < 0, rho below 1 - eps: floored at (1 - eps) A, no gradient
    (1.5, math.log(0.5), False),    # A > 0, rho below 1 - eps: the unclipped rho A is smaller, gradient flows
    (-0.7, math.log(1.6), False),   # A < 0, rho above 1 + eps: the unclipped rho A is smaller, gradient flows
    (0.9, math.log(1.1), False),    # inside the range: both terms equal rho A
])
def test_one_sided_clipping(orc, A, delta, expect_clipped):
    eps = 0.2
    lp_old = np.array([[-2.0]], dtype=np.float32)
    lp = (lp_old + np.float32(delta)).astype(np.float32)
    rho = math.exp(float(lp[0, 0]) - float(lp_old[0, 0]))
    sur, grad, st = orc.grpo_surrogate(lp, lp_old, np.array([1], np.int32), np.array([A], np.float32), eps, eps)
    A = float(np.float32(A))
    if expect_clipped:
        bound = 1 + eps if A > 0 else 1 - eps
        assert math.isclose(sur[0, 0], bound * A, rel_tol=1e-15)
        assert grad[0, 0] == 0.0 and st["clipped"] == 1
    else:
        assert math.isclose(sur[0, 0], rho * A, rel_tol=1e-15)
        assert math.isclose(grad[0, 0], -rho * A, rel_tol=1e-15) and st["clipped"] == 0


@pytest.mark.parametrize("agg", [0, 1])
def test_gradient_is_the_derivative_of_the_loss(orc, agg):
    """d loss / d log pi_theta by central differences in fp64 (logp perturbed one token at a time, away from the
    clip boundaries) equals the oracle's per-token gradient."""
    logp, logp_old, lengths, adv = case(orc, 7, n_seq=4, t_max=9, spread=0.4)
    lengths[0] = 9
    _, grad, st0 = orc.grpo_surrogate(logp, logp_old, lengths, adv, 0.2, 0.28, agg)
    h = 1e-3
    checked = 0
    for i in range(4):
        for t in range(int(lengths[i])):
            rho = math.exp(float(logp[i, t]) - float(logp_old[i, t]))
            if min(abs(rho - 0.8), abs(rho - 1.28)) < 5e-3:
                continue
            # f32 inputs: perturb through a power-of-two step that f32 represents exactly at these magnitudes
            up, dn = logp.copy(), logp.copy()
            up[i, t] += np.float32(h)
            dn[i, t] -= np.float32(h)
            lu = orc.grpo_surrogate(up, logp_old, lengths, adv, 0.2, 0.28, agg)[2]["loss"]
            ld = orc.grpo_surrogate(dn, logp_old, lengths, adv, 0.2, 0.28, agg)[2]["loss"]
            step = float(up[i, t]) - float(dn[i, t])
            fd = (lu - ld) / step
            assert abs(fd - grad[i, t]) <= 1e-6 * max(1.0, abs(grad[i, t])) + 1e-9, (i, t, fd, grad[i, t])
            checked += 1
    assert checked > 10


def test_aggregations_agree_for_equal_lengths(orc):
    logp, logp_old, _, adv = case(orc, 9)
    lengths = np.full(6, 20, np.int32)
    s0, g0, st0 = orc.grpo_surrogate(logp, logp_old, lengths, adv, agg=0)
    s1, g1, st1 = orc.grpo_surrogate(logp, logp_old, lengths, adv, agg=1)
    assert np.array_equal(s0, s1)
    assert math.isclose(st0["loss"], st1["loss"], rel_tol=1e-13)
    assert np.allclose(g0, g1, rtol=1e-13, atol=0)
    # with unequal lengths the per-response mean weights short responses more
    lengths2 = np.array([20, 1, 20, 20, 20, 20], np.int32)
    l0 = orc.grpo_surrogate(logp, logp_old, lengths2, adv, agg=0)[2]["loss"]
    l1 = orc.grpo_surrogate(logp, logp_old, lengths2, adv, agg=1)[2]["loss"]
    assert not math.isclose(l0, l1)


def test_zero_advantage_and_empty_responses(orc):
    logp, logp_old, lengths, _ = case(orc, 11)
    sur, grad, st = orc.grpo_surrogate(logp, logp_old, lengths, np.zeros(6, np.float32))
    assert np.all(sur == 0.0) and np.all(grad == 0.0) and st["loss"] == 0.0
    sur, grad, st = orc.grpo_surrogate(logp, logp_old, np.zeros(6, np.int32), np.ones(6, np.float32))
    assert st["tokens"] == 0 and st["loss"] == 0.0 and np.all(grad == 0.0)
