"""GPU parity of the GRPO token ratio and clipped surrogate (grpo_clipped_surrogate) against the fp64 oracle.

Inputs have the shape of the 8192-token prefill workload: 8 prompts x 8 responses of up to 128 tokens (ragged
lengths), synthetic log-probabilities of the behavior policy (log pi_b = -Exponential(2)) and of the current one
(log pi_b + N(0, s)), and the group-relative advantages of Bernoulli(0.3) rewards (computed by the oracle).
Per token the surrogate and gradient are the fp64 values rounded once to f32; a clip decision may differ only where
rho sits within rounding of a clip bound (then either is accepted and checked for consistency).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import nvfp4_weight_only_amd as qn
    return qn


def batch(seed, n_prompts=8, g=8, t_max=128, spread=0.3, ragged=True):
    s = lambda t: synth.seed_for(5, seed, t)
    n_seq = n_prompts * g
    rng = np.random.default_rng(seed)
    logp_old = (-rng.exponential(2.0, (n_seq, t_max))).astype(np.float32)
    logp = (logp_old + rng.normal(0.0, spread, (n_seq, t_max))).astype(np.float32)
    lengths = (rng.integers(1, t_max + 1, n_seq) if ragged else np.full(n_seq, t_max)).astype(np.int32)
    rewards = synth.bernoulli_f32(s("rewards"), (n_prompts, g), 0.3)
    adv = oracle.group_advantage(rewards, 1e-6).astype(np.float32).reshape(-1)
    return logp, logp_old, lengths, adv


def run(qn, logp, logp_old, lengths, adv, lo, hi, agg):
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(DEV)
    sur, grad, st = qn.grpo_surrogate(t(logp, np.float32), t(logp_old, np.float32), t(lengths, np.int32),
                                      t(adv, np.float32), lo, hi, agg)
    torch.cuda.synchronize()
    return sur.cpu().numpy(), grad.cpu().numpy(), qn.grpo_stats(st)


def check(qn, logp, logp_old, lengths, adv, lo=0.2, hi=0.2, agg=0):
    sur, grad, st = run(qn, logp, logp_old, lengths, adv, lo, hi, agg)
    # the library takes the widths as f32: the oracle sees the same values
    rs, rg, rst = oracle.grpo_surrogate(logp, logp_old, lengths, adv, float(np.float32(lo)), float(np.float32(hi)), agg)
    rho = np.exp(logp.astype(np.float64) - logp_old.astype(np.float64))
    near = (np.abs(rho - (1 - np.float64(np.float32(lo)))) < 1e-12) | (np.abs(rho - (1 + np.float64(np.float32(hi)))) < 1e-12)
    ok_s = np.abs(sur - rs) <= 2.0 ** -23 * np.abs(rs) + 1e-30
    ok_g = np.abs(grad - rg) <= 2.0 ** -23 * np.abs(rg) + 1e-30
    assert np.all(ok_s | near) and np.all(ok_g | near)
    assert st["tokens"] == rst["tokens"]
    assert abs(st["clipped"] - rst["clipped"]) <= int(near.sum())
    assert abs(st["loss"] - rst["loss"]) <= 1e-12 * max(1.0, abs(rst["loss"]))
    assert abs(st["ratio_mean"] - rst["ratio_mean"]) <= 1e-12 * max(1.0, rst["ratio_mean"])
    assert st["ratio_min"] == np.float32(rst["ratio_min"]) and st["ratio_max"] == np.float32(rst["ratio_max"])
    return st, rst


@pytest.mark.parametrize("agg", [0, 1])
@pytest.mark.parametrize("lo,hi", [(0.2, 0.2), (0.2, 0.28), (0.0, 0.0)])
def test_prefill_batch(qn, agg, lo, hi):
    logp, logp_old, lengths, adv = batch(3 + agg)
    st, rst = check(qn, logp, logp_old, lengths, adv, lo, hi, agg)
    assert 0 < rst["clipped"] < rst["tokens"]  # both branches are exercised


def test_on_policy_and_edges(qn):
    logp, _, lengths, adv = batch(7)
    check(qn, logp, logp, lengths, adv)                     # rho = 1: surrogate = advantage
    lengths2 = lengths.copy()
    lengths2[:5] = [0, -3, 500, 128, 1]                     # empty, negative (-> 0), beyond t_max (-> clamped)
    check(qn, logp, logp[::-1].copy(), lengths2, adv, agg=1)
    check(qn, logp, logp, np.zeros_like(lengths), adv)      # no valid token
    check(qn, logp, logp[::-1].copy(), lengths, np.zeros_like(adv))  # zero advantages


def test_empty_batch(qn):
    z = np.zeros((0, 16), np.float32)
    sur, grad, st = run(qn, z, z, np.zeros(0, np.int32), np.zeros(0, np.float32), 0.2, 0.2, 0)
    assert st["tokens"] == 0 and st["loss"] == 0.0


def test_large_batch(qn):
    """2 million tokens (1024 responses of up to 2048) through the one-workgroup kernel."""
    logp, logp_old, lengths, adv = batch(11, n_prompts=128, g=8, t_max=2048, spread=0.2)
    check(qn, logp, logp_old, lengths, adv)
