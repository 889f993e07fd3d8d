"""Pins of the bandit oracle (online draft selection).

The FlashSpec summary (Methodology section 2) frames draft selection as a
K-armed bandit with reward = fraction of draft tokens accepted, solved by UCB1
or Thompson sampling; its Significance section states Theorem 1 (the output
distribution stays the target's whatever the history-only policy does). Its
results section reports a simulation (10,000 rounds, K = 3) with UCB1 regret
100.2 against a bound of about 526 and Thompson regret 18.9; the arm means and
reward noise behind those figures are not given, so they are not reproduced
here (parity unpinned for those two numbers).

What pins the oracle instead:
* UCB1's opening round robin (Auer, Cesa-Bianchi and Fischer 2002, Fig. 1);
* UCB1's finite-time regret bound (same paper, Theorem 1) on simulated
  verification outcomes, and logarithmic (not linear) regret growth;
* the Gamma and Beta samplers behind Thompson sampling against
  ``scipy.stats.gamma`` / ``scipy.stats.beta`` (Kolmogorov-Smirnov);
* Thompson sampling's logarithmic regret growth and convergence;
* the pages' Theorem 1: with the bandit picking one of three draft
  distributions every step, the V = 8 output-marginal gate still passes.
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle
import specgen
from test_oracle_stats import chi2_ok, discrete_ks, scaled_probs

GAMMA = 4
ALPHAS = np.array([0.75, 0.6, 0.45])  # per-token acceptance probability of each arm


def mean_reward(alpha: float, gamma: int = GAMMA) -> float:
    """E[k / gamma] when each draft token is accepted with probability alpha
    until the first rejection: E[k] = sum_{i=1..gamma} alpha^i."""
    return sum(alpha ** i for i in range(1, gamma + 1)) / gamma


def sample_accept_len(rng, alpha: np.ndarray, gamma: int = GAMMA) -> np.ndarray:
    """k = number of leading accepts among gamma independent tokens."""
    acc = rng.random((alpha.size, gamma)) < alpha[:, None]
    k = np.where(acc.all(axis=1), gamma, np.argmin(acc, axis=1))
    return k.astype(np.int32)


def run_bandits(policy, seeds: int, rounds: int, snapshot: int, alphas=ALPHAS):
    """``seeds`` independent bandits run side by side as groups of one sequence."""
    band = oracle.Bandit(policy, groups=seeds, arms=len(alphas), batch=seeds, gamma=GAMMA)
    rng = np.random.default_rng(31337)
    arm, _ = band.step(seed=5, offset=0)
    snap = None
    for t in range(1, rounds + 1):
        k = sample_accept_len(rng, alphas[arm])
        arm, _ = band.step(k, arm, seed=5, offset=t)
        if t == snapshot:
            snap = band.counts.copy()
    return band, snap


def pseudo_regret(counts: np.ndarray, alphas=ALPHAS) -> np.ndarray:
    mu = np.array([mean_reward(a) for a in alphas])
    return (counts * (mu.max() - mu)[None, :]).sum(axis=1)


def auer_bound(n: int, alphas=ALPHAS) -> float:
    """Auer et al. 2002, Theorem 1: E[regret] <= 8 sum ln n / D_i + (1 + pi^2/3) sum D_i."""
    mu = np.array([mean_reward(a) for a in alphas])
    d = mu.max() - mu
    d = d[d > 0]
    return float((8.0 * math.log(n) / d).sum() + (1.0 + math.pi ** 2 / 3.0) * d.sum())


def test_ucb1_opening_plays_every_arm_once_in_index_order():
    band = oracle.Bandit(oracle.UCB1, groups=1, arms=5, batch=2, gamma=GAMMA)
    arm, margin = band.step()
    seen = [int(arm[0])]
    for t in range(4):
        arm, margin = band.step(np.array([GAMMA, GAMMA], np.int32), arm)
        seen.append(int(arm[0]))
        assert margin[0] == np.inf
    # the best possible rewards do not cut the opening short
    assert seen == [0, 1, 2, 3, 4]
    assert band.counts.tolist() == [[1, 1, 1, 1, 0]]


@pytest.fixture(scope="module")
def ucb1_run():
    return run_bandits(oracle.UCB1, seeds=24, rounds=10_000, snapshot=1_000)


@pytest.fixture(scope="module")
def thompson_run():
    return run_bandits(oracle.THOMPSON, seeds=24, rounds=10_000, snapshot=1_000)


def test_ucb1_regret_within_auer_bound(ucb1_run):
    band, _ = ucb1_run
    reg = pseudo_regret(band.counts)
    assert band.counts.sum(axis=1).tolist() == [10_000] * band.G
    assert reg.mean() <= auer_bound(10_000)
    assert reg.max() <= auer_bound(10_000)


def test_ucb1_regret_grows_logarithmically(ucb1_run):
    """Regret(10^4) / Regret(10^3): about ln(10^4)/ln(10^3) = 1.33 for a
    logarithmic-regret policy, 10 for one that has locked onto a worse arm."""
    band, snap = ucb1_run
    ratio = pseudo_regret(band.counts).mean() / pseudo_regret(snap).mean()
    assert 1.0 < ratio < 4.0
    # every bandit ends on the best arm, and still samples the others
    assert (band.counts.argmax(axis=1) == 0).all()
    assert (band.counts[:, 1:] >= 20).all()


def test_gamma_sampler_matches_scipy():
    for shape in (1.0, 2.5, 17.3, 400.0):
        x = np.array([oracle.gamma_sample(shape, seed=11, offset=o)[0] for o in range(4000)])
        assert stats.kstest(x, stats.gamma(shape).cdf).pvalue > 0.001, shape


def test_beta_sampler_matches_scipy():
    for a, b in ((1.0, 1.0), (2.5, 7.25), (40.3, 12.1), (1.0, 300.0)):
        x = np.array([oracle.beta_sample(a, b, seed=3, offset=o, group=2, arm=1)[0]
                      for o in range(4000)])
        assert ((x > 0) & (x < 1)).all()
        assert stats.kstest(x, stats.beta(a, b).cdf).pvalue > 0.001, (a, b)


def test_beta_draws_are_independent_across_arms_and_groups():
    """Different (group, arm) pairs read different Philox blocks."""
    xs = {}
    for g in range(3):
        for j in range(3):
            xs[g, j] = np.array([oracle.beta_sample(2.0, 2.0, 9, o, g, j)[0] for o in range(2000)])
    keys = list(xs)
    for i in range(len(keys)):
        for j in range(i + 1, len(keys)):
            r = np.corrcoef(xs[keys[i]], xs[keys[j]])[0, 1]
            assert abs(r) < 0.1, (keys[i], keys[j], r)


def test_thompson_choice_probabilities_match_the_posterior():
    """From a fixed state, P(arm j is played) = P(theta_j is the largest) with
    theta_i ~ Beta(1 + S_i, 1 + n_i - S_i) independent, which is the integral
    of pdf_j(x) * prod_{i != j} cdf_i(x) over [0, 1] (scipy quad)."""
    from scipy.integrate import quad
    counts = np.array([[12, 30, 7]], np.uint32)
    sums = np.array([[7.25, 15.5, 4.75]])
    post = [stats.beta(1 + sums[0, j], 1 + counts[0, j] - sums[0, j]) for j in range(3)]
    law = []
    for j in range(3):
        f = lambda x, j=j: post[j].pdf(x) * np.prod([post[i].cdf(x) for i in range(3) if i != j])
        law.append(quad(f, 0, 1, limit=200)[0])
    assert abs(sum(law) - 1) < 1e-6
    n = 6000
    picks = np.zeros(3, int)
    for o in range(n):
        band = oracle.Bandit(oracle.THOMPSON, groups=1, arms=3, batch=1, gamma=GAMMA)
        band.counts[:] = counts
        band.sums[:] = sums
        arm, _ = band.step(seed=21, offset=o)
        picks[arm[0]] += 1
    assert stats.chisquare(picks, np.array(law) * n).pvalue > 0.001, (picks, law)


def test_thompson_regret_logarithmic_and_below_ucb1_bound(thompson_run):
    band, snap = thompson_run
    reg = pseudo_regret(band.counts)
    assert reg.mean() <= auer_bound(10_000)
    ratio = reg.mean() / pseudo_regret(snap).mean()
    assert 1.0 < ratio < 4.0
    assert (band.counts.argmax(axis=1) == 0).all()


def test_bandit_skips_invalid_rows_and_bad_arms():
    band = oracle.Bandit(oracle.UCB1, groups=2, arms=3, batch=4, gamma=GAMMA)
    band.step()
    # group 0: one valid row (k = 2) and one sentinel; group 1: both sentinels
    arm, _ = band.step(np.array([2, -1, -1, -1], np.int32), np.array([0, 0], np.int32))
    assert band.counts.tolist() == [[1, 0, 0], [0, 0, 0]]
    assert band.sums[0, 0] == 0.5
    assert arm.tolist() == [1, 0]
    # an out-of-range played arm: no update, no arm
    arm, _ = band.step(np.array([4, 4, 4, 4], np.int32), np.array([3, -2], np.int32))
    assert arm.tolist() == [-1, -1]
    assert band.counts.tolist() == [[1, 0, 0], [0, 0, 0]]
    # accept lengths above gamma are not valid either
    band.step(np.array([5, 5, 1, 3], np.int32), np.array([1, 1], np.int32))
    assert band.counts.tolist() == [[1, 0, 0], [0, 1, 0]]
    assert band.sums[1, 1] == 0.5


def test_theorem1_output_marginal_with_bandit_choosing_the_draft():
    """Three draft distributions of different quality; every decoding step the
    bandit (from past accept lengths only) picks one for the whole batch. The
    verified tokens must still follow the target at every position."""
    rng = np.random.default_rng(77)
    G, V, T = 3, 8, 0.9
    base = rng.normal(0, 1.2, size=(G + 1, V))
    zp = (base + rng.normal(0, 0.8, size=base.shape)).astype(np.float32)
    drafts = [(base[:G] + rng.normal(0, s, size=(G, V))).astype(np.float32)
              for s in (0.2, 1.0, 2.5)]
    steps, per_step = 500, 20
    for policy in (oracle.UCB1, oracle.THOMPSON):
        band = oracle.Bandit(policy, groups=1, arms=3, batch=per_step, gamma=G)
        arm, _ = band.step(seed=1, offset=0)
        toks, lens, plays = [], [], np.zeros(3, int)
        tok_rng = np.random.default_rng(5)
        target = np.ascontiguousarray(np.broadcast_to(zp, (per_step, G + 1, V)))
        temp = np.full(per_step, T, np.float32)
        for t in range(steps):
            zq = drafts[int(arm[0])]
            plays[int(arm[0])] += 1
            draft = np.ascontiguousarray(np.broadcast_to(zq, (per_step, G, V)))
            dt = np.stack([specgen.gumbel_max_tokens(zq, T, tok_rng)
                           for _ in range(per_step)]).astype(np.int32)
            out = oracle.verify(draft, target, dt, temp, seed=2025, offset=t)
            toks.append(out["tokens"])
            lens.append(out["accept_len"])
            arm, _ = band.step(out["accept_len"], arm, seed=1, offset=t + 1)
        tok = np.concatenate(toks)
        k = np.concatenate(lens)
        p = scaled_probs(zp, T)
        assert discrete_ks(tok[:, 0], p[0]) < 1.628 / math.sqrt(len(tok))
        for i in range(G + 1):
            sel = k >= i
            assert chi2_ok(tok[sel, i], p[i]), (policy, i)
        # the bandit did prefer the closest draft
        assert plays[0] > plays[1] and plays[0] > plays[2], plays
