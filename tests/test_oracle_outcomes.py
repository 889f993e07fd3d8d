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
