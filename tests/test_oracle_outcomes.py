"""Pins of the verification-outcome oracle (``oracle.outcomes``).

Speculative speculative decoding predicts the outcome of a verification -- the
accepted count k and the extra token -- and keys its speculation cache on it;
Saguaro spends the cache on likely lengths and, per length, on the top-F
tokens of the residual (Speculative Speculative Decoding summary, section 2:
central concept, Saguaro challenges 1 and 2). Given the drafted tokens the
outcome has an exact law, which ``oracle.outcomes`` writes out:
P(k = i | t) and, per length, the extra token's distribution and its top F.

What pins it (none of these re-types its formulas):
* the law of (k, extra token) that the verification oracle actually produces
  over 20,000 Philox draws with the drafts held fixed (chi-square at 0.01
  over every (k, token) cell) -- the verification oracle is itself pinned by
  the closed forms and gates of test_oracle_stats.py;
* the top-F lists against numpy's stable sort of the distribution (largest
  first, lowest index first among equal values), including planted ties;
* the residual mass against the total-variation distance 0.5 * sum |p - q|
  of scipy softmax distributions;
* degenerate cases: p = q (every draft accepted; lists fall back to p),
  disjoint supports (the first draft is always rejected), greedy sequences
  against the verification oracle's deterministic outcome, V < F padding,
  sentinel sequences.
"""
import itertools

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import chisquare

import oracle
import specgen
from test_oracle_stats import scaled_probs


def fixed_draft_case(seed=4, G=3, V=8, T=0.9, n=20_000, target_ratio=(0.6, 1.8, 0.4)):
    rng = np.random.default_rng(seed)
    base = rng.normal(0, 1.2, size=(G + 1, V))
    zp = (base + rng.normal(0, 0.8, size=base.shape)).astype(np.float32)
    zq = base[:G].astype(np.float32)
    # drafts whose ratio p/q is near the given values: below 1 the length law
    # spreads over several k, above 1 the acceptance is capped at 1
    ratio = scaled_probs(zp[:G], T) / scaled_probs(zq, T)
    want = np.asarray(target_ratio, np.float64)[:G, None]
    t = np.argmin(np.abs(np.log(ratio / want)), axis=1).astype(np.int32)
    draft = np.ascontiguousarray(np.broadcast_to(zq, (n, G, V)))
    target = np.ascontiguousarray(np.broadcast_to(zp, (n, G + 1, V)))
    toks = np.ascontiguousarray(np.broadcast_to(t, (n, G)))
    temp = np.full(n, T, np.float32)
    return draft, target, toks, temp


@pytest.mark.parametrize("ratios", [(0.6, 0.6, 0.6), (0.6, 1.8, 0.4)])
def test_outcome_law_matches_the_verification_oracle(ratios):
    draft, target, toks, temp = fixed_draft_case(target_ratio=ratios)
    n, G, V = draft.shape
    ver = oracle.verify(draft, target, toks, temp, seed=31, offset=2)
    k = ver["accept_len"]
    extra = ver["tokens"][np.arange(n), k]
    out = oracle.outcomes(draft[:1], target[:1], toks[:1], temp[:1], F=V, with_dist=True)
    law = out["pk"][0][:, None] * out["dist"][0]          # [G+1, V]
    assert (law >= 0).all() and abs(law.sum() - 1.0) < 1e-12
    counts = np.zeros((G + 1, V))
    np.add.at(counts, (k, extra), 1)
    keep = law.ravel() > 0
    assert counts.ravel()[~keep].sum() == 0, "an outcome the law gives probability 0"
    expected = law.ravel()[keep] * n
    assert chisquare(counts.ravel()[keep], expected).pvalue > 0.01
    # the marginal law of k alone
    pk = out["pk"][0]
    nk = np.bincount(k, minlength=G + 1)
    assert (nk[pk == 0] == 0).all() and (pk > 0).sum() >= 3
    assert chisquare(nk[pk > 0], pk[pk > 0] * n).pvalue > 0.01


def test_top_f_is_the_stable_sort_of_the_distribution():
    rng = np.random.default_rng(12)
    B, G, V, F = 4, 3, 50, 7
    zq = rng.normal(0, 1.5, size=(B, G, V)).astype(np.float32)
    zp = (np.concatenate([zq, zq[:, :1]], axis=1)
          + rng.normal(0, 1.0, size=(B, G + 1, V))).astype(np.float32)
    # planted ties: equal logits in both rows give equal residual entries
    zq[:, :, 30] = zq[:, :, 10]
    zp[:, :G, 30] = zp[:, :G, 10]
    zp[:, G, 31] = zp[:, G, 11]
    toks = rng.integers(0, V, size=(B, G)).astype(np.int32)
    temp = np.array([0.7, 1.0, 1.3, 0.0], np.float32)
    out = oracle.outcomes(zq, zp, toks, temp, F, with_dist=True)
    for b in range(B):
        for i in range(G + 1):
            d = out["dist"][b, i]
            if temp[b] == 0.0:
                order = np.argsort(-zp[b, i].astype(np.float64), kind="stable")[:F]
            else:
                order = np.argsort(-d, kind="stable")[:F]
                np.testing.assert_allclose(out["probs"][b, i], d[order], rtol=0, atol=0)
            assert out["tokens"][b, i].tolist() == order.tolist(), (b, i)


def test_residual_mass_is_total_variation():
    rng = np.random.default_rng(5)
    B, G, V = 3, 4, 40
    zq = rng.normal(0, 2, size=(B, G, V)).astype(np.float32)
    zp = rng.normal(0, 2, size=(B, G + 1, V)).astype(np.float32)
    toks = rng.integers(0, V, size=(B, G)).astype(np.int32)
    temp = np.array([0.5, 1.0, 1.7], np.float32)
    out = oracle.outcomes(zq, zp, toks, temp, 4)
    for b in range(B):
        p = scaled_probs(zp[b], temp[b])
        q = scaled_probs(zq[b], temp[b])
        tv = 0.5 * np.abs(p[:G] - q).sum(axis=1)
        np.testing.assert_allclose(out["mass"][b, :G], tv, rtol=1e-12, atol=1e-15)
        assert out["mass"][b, G] == 1.0
        assert abs(out["pk"][b].sum() - 1.0) < 1e-12


def test_p_equal_q_and_disjoint_supports():
    rng = np.random.default_rng(6)
    G, V, F = 3, 16, 4
    z = rng.normal(0, 1, size=(1, G + 1, V)).astype(np.float32)
    toks = rng.integers(0, V, size=(1, G)).astype(np.int32)
    same = oracle.outcomes(np.ascontiguousarray(z[:, :G]), z, toks, np.float32([0.8]), F)
    assert same["pk"][0].tolist() == [0.0] * G + [1.0]
    assert (same["mass"][0, :G] == 0).all()
    for i in range(G):  # empty residual: the list is that of p_i
        p = softmax(z[0, i].astype(np.float32) * np.float32(1 / np.float32(0.8)))
        assert same["tokens"][0, i].tolist() == np.argsort(-p, kind="stable")[:F].tolist()
    # disjoint supports: the draft puts all its mass where the target has none
    zq = np.full((1, G, V), -np.inf, np.float32)
    zq[..., :4] = 0.0
    zp = np.full((1, G + 1, V), -np.inf, np.float32)
    zp[..., 8:] = rng.normal(0, 1, size=(1, G + 1, V - 8)).astype(np.float32)
    toks = np.zeros((1, G), np.int32)
    dis = oracle.outcomes(zq, zp, toks, np.float32([1.0]), F)
    assert dis["pk"][0].tolist() == [1.0] + [0.0] * G
    np.testing.assert_allclose(dis["mass"][0, :G], 1.0, rtol=0, atol=1e-12)


def test_greedy_outcome_is_the_verification_outcome():
    rng = np.random.default_rng(8)
    B, G, V, F = 16, 4, 30, 3
    zp = np.round(rng.normal(0, 2, size=(B, G + 1, V))).astype(np.float32)  # many ties
    zq = rng.normal(0, 2, size=(B, G, V)).astype(np.float32)
    amax = np.argmax(zp, axis=-1)
    toks = np.where(rng.random((B, G)) < 0.7, amax[:, :G], rng.integers(0, V, (B, G))).astype(np.int32)
    temp = np.zeros(B, np.float32)
    ver = oracle.verify(zq, zp, toks, temp)
    out = oracle.outcomes(zq, zp, toks, temp, F)
    for b in range(B):
        k = ver["accept_len"][b]
        assert out["pk"][b].tolist() == [1.0 if i == k else 0.0 for i in range(G + 1)]
        assert out["tokens"][b, k, 0] == ver["tokens"][b, k]
        assert out["probs"][b, :, 0].tolist() == [1.0] * (G + 1)


def test_padding_and_sentinels():
    rng = np.random.default_rng(9)
    G, V, F = 2, 5, 8
    zq = rng.normal(0, 1, size=(3, G, V)).astype(np.float32)
    zp = rng.normal(0, 1, size=(3, G + 1, V)).astype(np.float32)
    toks = np.array([[1, 2], [0, 7], [3, 3]], np.int32)       # row 1: token out of range
    temp = np.array([1.0, 1.0, np.nan], np.float32)            # row 2: bad temperature
    out = oracle.outcomes(zq, zp, toks, temp, F)
    assert (out["tokens"][0, :, V:] == -1).all() and (out["probs"][0, :, V:] == 0).all()
    assert sorted(out["tokens"][0, 0, :V].tolist()) == list(range(V))
    for b in (1, 2):
        assert (out["tokens"][b] == -1).all() and not out["probs"][b].any()
        assert not out["pk"][b].any() and not out["mass"][b].any()


# ------------------------------------------------------------------ fan-out ---
# Speculation-cache budget per length (Speculative Speculative Decoding summary,
# section 2, Saguaro challenge 1: more of a fixed budget for likely lengths, to
# hit the cache as often as possible). The oracle places entries one at a time
# on the most valuable next list entry; these pins check it against an
# exhaustive search, a closed form and the edge cases.

def _sorted_lists(rng, B, L, F):
    pk = rng.dirichlet(np.ones(L), size=B).astype(np.float32)
    probs = np.sort(rng.dirichlet(np.ones(F + 2), size=(B, L))[..., :F], axis=-1)[..., ::-1]
    return pk, np.ascontiguousarray(probs, dtype=np.float32)


def _value(pk, probs, n):
    """Expected hit rate of a cache holding the first n[i] entries of each list."""
    return sum(float(pk[i]) * float(probs[i][j]) for i in range(len(n)) for j in range(n[i]))


def fanout_is_optimal():
    rng = np.random.default_rng(11)
    for L in (1, 2, 3):
        for F in (1, 2, 3):
            pk, probs = _sorted_lists(rng, 4, L, F)
            for budget in range(0, L * F + 2):
                n, hit = oracle.outcome_fanout(pk, probs, budget)
                placed = min(budget, L * F)
                for b in range(4):
                    assert n[b].sum() == placed and (n[b] >= 0).all() and (n[b] <= F).all()
                    best = max(_value(pk[b], probs[b], c)
                               for c in itertools.product(range(F + 1), repeat=L)
                               if sum(c) == placed)
                    got = _value(pk[b], probs[b], n[b])
                    assert abs(got - best) <= 1e-12 * max(1.0, best), (L, F, budget, n[b], got, best)
                    assert abs(hit[b] - got) <= 1e-12 * max(1.0, got)


def test_fanout_maximises_the_hit_rate():
    """Against every allocation of the same number of entries (L, F <= 3)."""
    fanout_is_optimal()


def fanout_diagonals():
    # v(i, j) = 2^-i * 2^-j: whole anti-diagonals i + j < d fill first, the
    # lower length first within one, so d(d+1)/2 entries give n_i = d - i.
    L, F = 7, 7
    pk = np.array([[2.0 ** -i for i in range(L)]], np.float32)
    probs = np.array([[[2.0 ** -j for j in range(F)]] * L], np.float32)
    for d in range(L + 1):
        n, hit = oracle.outcome_fanout(pk, probs, d * (d + 1) // 2)
        assert n[0].tolist() == [max(0, d - i) for i in range(L)], (d, n[0])
        assert hit[0] == sum((k + 1) * 2.0 ** -k for k in range(d))
    # one entry more goes to length 0 (the next anti-diagonal, lowest length first)
    n, _ = oracle.outcome_fanout(pk, probs, 3 * 4 // 2 + 1)
    assert n[0].tolist() == [4, 2, 1, 0, 0, 0, 0]


def test_fanout_closed_form_on_powers_of_two():
    fanout_diagonals()


def test_fanout_follows_a_geometric_law_of_lengths():
    """With P(k = i) of a fixed acceptance rate alpha (geometric in i below G)
    and the same list at every length, shorter lengths never get fewer
    entries than longer ones below G."""
    rng = np.random.default_rng(5)
    G, F = 8, 16
    for alpha in (0.3, 0.6, 0.85):
        pk = np.array([[alpha ** i * (1 - alpha) for i in range(G)] + [alpha ** G]], np.float32)
        row = np.sort(rng.dirichlet(np.ones(F + 4))[:F])[::-1]
        probs = np.array([[row] * (G + 1)], np.float32)
        for budget in (1, 5, 17, 40, 100, 144):
            n, _ = oracle.outcome_fanout(pk, probs, budget)
            assert all(n[0][i] >= n[0][i + 1] for i in range(G - 1)), (alpha, budget, n[0])


def test_fanout_edges():
    rng = np.random.default_rng(3)
    pk, probs = _sorted_lists(rng, 3, 4, 5)
    n, hit = oracle.outcome_fanout(pk, probs, 0)
    assert (n == 0).all() and (hit == 0).all()
    n, hit = oracle.outcome_fanout(pk, probs, 1000)
    assert (n == 5).all()
    for b in range(3):
        assert abs(hit[b] - _value(pk[b], probs[b], [5] * 4)) <= 1e-12
    # equal worth everywhere: lists fill in length order
    n, hit = oracle.outcome_fanout(np.full((1, 3), 0.5, np.float32), np.full((1, 3, 4), 0.25, np.float32), 6)
    assert n[0].tolist() == [4, 2, 0] and hit[0] == 6 * 0.125
    # NaN and negative values are worth 0: placed after every positive entry
    pk1 = np.array([[0.5, np.nan, -1.0]], np.float32)
    probs1 = np.array([[[0.5, 0.25], [0.9, 0.9], [0.9, 0.9]]], np.float32)
    n, hit = oracle.outcome_fanout(pk1, probs1, 3)
    assert n[0].tolist() == [2, 1, 0] and hit[0] == 0.375
    # a list that is not non-increasing still gets a prefix: the next entry
    # of length 0 (0.1) loses to length 1's first (0.3) even though 0.9 follows
    n, hit = oracle.outcome_fanout(np.array([[1.0, 1.0]], np.float32),
                                   np.array([[[0.5, 0.1, 0.9], [0.3, 0.2, 0.0]]], np.float32), 3)
    assert n[0].tolist() == [1, 2] and abs(hit[0] - 1.0) < 1e-7
