"""Statistical and degenerate-case pins of the oracle's full verification call.

The CI gate the FlashSpec summary describes (Methodology section 3, correctness
and testing: a Kolmogorov-Smirnov hard gate comparing the speculative sampler's
output with the target distribution over 10,000 samples at significance 0.01)
is run here on V = 8 cases, together with the closed forms of standard
speculative sampling:

* P(accept at position i) = sum_v min(p_i(v), q_i(v)) = 1 - TV(p_i, q_i);
* P(k = i) = prod_{j<i} a_j * (1 - a_i), P(k = gamma) = prod_j a_j;
* tokens[i] given k >= i is distributed as p_i (exactness, Theorem 1 of the
  FlashSpec summary's Significance section);
* degenerate cases: gamma = 0, p = q, disjoint supports, greedy (T = 0).

Each of the 10,000 draws is its own batch row with identical logits, so it gets
its own Philox counter. Draft tokens are sampled from the draft distribution by
the input generator (Gumbel-max), independently of the oracle.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import binomtest, chisquare

import oracle
import specgen

N_DRAWS = 10_000
ALPHA = 0.01
KS_CRIT = 1.628 / math.sqrt(N_DRAWS)  # two-sided KS critical value at 0.01


def scaled_probs(z, T):
    inv_t = np.float32(1.0) / np.float32(T)
    return softmax((np.asarray(z, np.float32) * inv_t).astype(np.float64), axis=-1)


def make_batch(zq, zp, T, n, seed):
    """n copies of one sequence; draft tokens drawn from the draft distribution."""
    G = zq.shape[0]
    rng = np.random.default_rng(seed)
    draft = np.ascontiguousarray(np.broadcast_to(zq, (n,) + zq.shape))
    target = np.ascontiguousarray(np.broadcast_to(zp, (n,) + zp.shape))
    if G:
        toks = np.stack([specgen.gumbel_max_tokens(zq, T, rng) for _ in range(n)])
    else:
        toks = np.zeros((n, 0), np.int32)
    temp = np.full(n, T, np.float32)
    return draft, target, toks.astype(np.int32), temp


def discrete_ks(samples, probs):
    V = len(probs)
    emp = np.cumsum(np.bincount(samples, minlength=V)) / len(samples)
    return float(np.max(np.abs(emp - np.cumsum(probs))))


def chi2_ok(samples, probs):
    V = len(probs)
    counts = np.bincount(samples, minlength=V)
    keep = probs > 0
    assert counts[~keep].sum() == 0, "mass on a zero-probability token"
    exp = probs[keep] / probs[keep].sum() * len(samples)
    return chisquare(counts[keep], exp).pvalue > ALPHA


def build_gate_case():
    rng = np.random.default_rng(1234)
    G, V = 3, 8
    base = rng.normal(0, 1.2, size=(G + 1, V))
    zp = (base + rng.normal(0, 0.8, size=base.shape)).astype(np.float32)
    zq = base[:G].astype(np.float32)
    T = 0.9
    draft, target, toks, temp = make_batch(zq, zp, T, N_DRAWS, seed=99)
    out = oracle.verify(draft, target, toks, temp, seed=2024, offset=7)
    return dict(zq=zq, zp=zp, T=T, toks=toks, out=out, G=G, V=V)


@pytest.fixture(scope="module")
def gate_case():
    return build_gate_case()


def test_gate_acceptance_rate_closed_form(gate_case):
    c = gate_case
    p = scaled_probs(c["zp"], c["T"])
    q = scaled_probs(c["zq"], c["T"])
    a0 = np.minimum(p[0], q[0]).sum()
    k = c["out"]["accept_len"]
    assert binomtest(int((k >= 1).sum()), N_DRAWS, a0).pvalue > ALPHA


def test_gate_accept_length_law(gate_case):
    c = gate_case
    p = scaled_probs(c["zp"], c["T"])
    q = scaled_probs(c["zq"], c["T"])
    a = np.minimum(p[:c["G"]], q).sum(axis=1)
    law = [np.prod(a[:i]) * (1 - a[i]) for i in range(c["G"])] + [np.prod(a)]
    k = c["out"]["accept_len"]
    assert k.min() >= 0 and k.max() <= c["G"]
    counts = np.bincount(k, minlength=c["G"] + 1)
    assert chisquare(counts, np.array(law) * N_DRAWS).pvalue > ALPHA


def test_gate_output_marginal_is_target(gate_case):
    """tokens[i] | k >= i ~ p_i: chi-square and KS at 0.01 over 10,000 draws."""
    c = gate_case
    p = scaled_probs(c["zp"], c["T"])
    k = c["out"]["accept_len"]
    tok = c["out"]["tokens"]
    first = tok[:, 0]
    assert discrete_ks(first, p[0]) < KS_CRIT
    assert chi2_ok(first, p[0])
    for i in range(1, c["G"] + 1):
        sel = k >= i
        assert sel.sum() > 500
        assert chi2_ok(tok[sel, i], p[i]), i
    # emitted tokens agree with the drafts up to k, pads after k + 1
    for b in range(0, N_DRAWS, 97):
        kb = k[b]
        assert list(tok[b, :kb]) == list(c["toks"][b, :kb])
        assert np.all(tok[b, kb + 1:] == -1)


def test_gamma_zero_draws_from_p0():
    rng = np.random.default_rng(3)
    zp = rng.normal(0, 1.5, size=(1, 8)).astype(np.float32)
    zq = np.zeros((0, 8), np.float32)
    draft, target, toks, temp = make_batch(zq, zp, 1.3, N_DRAWS, seed=1)
    out = oracle.verify(draft, target, toks, temp, seed=5)
    assert np.all(out["accept_len"] == 0)
    p = scaled_probs(zp[0], 1.3)
    assert chi2_ok(out["tokens"][:, 0], p)
    assert discrete_ks(out["tokens"][:, 0], p) < KS_CRIT


def test_identical_distributions_accept_everything():
    rng = np.random.default_rng(4)
    G = 5
    base = rng.normal(0, 2.0, size=(G + 1, 8)).astype(np.float32)
    draft, target, toks, temp = make_batch(base[:G], base, 0.8, 2000, seed=2)
    out = oracle.verify(draft, target, toks, temp, seed=6)
    assert np.all(out["accept_len"] == G)
    assert np.array_equal(out["tokens"][:, :G], toks)
    assert chi2_ok(out["tokens"][:, G], scaled_probs(base[G], 0.8))


def test_disjoint_supports_reject_everything():
    G, V = 2, 8
    rng = np.random.default_rng(5)
    zq = np.full((G, V), -np.inf, np.float32)
    zp = np.full((G + 1, V), -np.inf, np.float32)
    zq[:, :4] = rng.normal(0, 1, size=(G, 4))
    zp[:, 4:] = rng.normal(0, 1, size=(G + 1, 4))
    draft, target, toks, temp = make_batch(zq, zp, 1.0, 3000, seed=3)
    assert toks.max() < 4
    out = oracle.verify(draft, target, toks, temp, seed=7)
    assert np.all(out["accept_len"] == 0)
    # the residual equals p on its own support
    assert chi2_ok(out["tokens"][:, 0], scaled_probs(zp[0], 1.0))


def test_greedy_rows_are_argmax():
    rng = np.random.default_rng(6)
    B, G, V = 64, 4, 50
    zp = rng.integers(-4, 5, size=(B, G + 1, V)).astype(np.float32)  # many ties
    zq = rng.normal(0, 1, size=(B, G, V)).astype(np.float32)
    amax = np.argmax(zp, axis=-1)
    toks = amax[:, :G].copy().astype(np.int32)
    flip = rng.random((B, G)) < 0.3
    toks[flip] = (toks[flip] + 1) % V
    temp = np.zeros(B, np.float32)
    out = oracle.verify(zq, zp, toks, temp, seed=8)
    for b in range(B):
        mism = np.nonzero(toks[b] != amax[b, :G])[0]
        k = int(mism[0]) if len(mism) else G
        assert out["accept_len"][b] == k
        assert list(out["tokens"][b, :k]) == list(toks[b, :k])
        assert out["tokens"][b, k] == amax[b, k]
        assert np.all(out["tokens"][b, k + 1:] == -1)


def test_greedy_ignores_seed():
    rng = np.random.default_rng(7)
    zp = rng.normal(0, 1, size=(4, 3, 16)).astype(np.float32)
    zq = rng.normal(0, 1, size=(4, 2, 16)).astype(np.float32)
    toks = np.argmax(zp[:, :2], -1).astype(np.int32)
    t0 = np.zeros(4, np.float32)
    a = oracle.verify(zq, zp, toks, t0, seed=1, offset=2)
    b = oracle.verify(zq, zp, toks, t0, seed=99, offset=5)
    assert np.array_equal(a["tokens"], b["tokens"])
    assert np.all(a["accept_len"] == 2)


def test_sentinel_rows():
    rng = np.random.default_rng(8)
    B, G, V = 6, 3, 40
    zq = rng.normal(0, 1, size=(B, G, V)).astype(np.float32)
    zp = rng.normal(0, 1, size=(B, G + 1, V)).astype(np.float32)
    toks = rng.integers(0, V, size=(B, G)).astype(np.int32)
    temp = np.array([1.0, np.nan, -0.5, np.inf, 1.0, 1.0], np.float32)
    toks[4, 1] = V          # out of range
    zp[5, 2, :] = -np.inf   # a row with no finite logit
    out = oracle.verify(zq, zp, toks, temp)
    assert out["accept_len"][0] >= 0
    for b in range(1, 6):
        assert out["accept_len"][b] == -1, b
        assert np.all(out["tokens"][b] == -1)
    # greedy sequence with an all -inf target row is also a sentinel
    zp2 = zp.copy()
    zp2[0, 1, :] = -np.inf
    out2 = oracle.verify(zq, zp2, toks, np.zeros(B, np.float32))
    assert out2["accept_len"][0] == -1


def test_neg_inf_logits_allowed():
    """Padded vocabulary entries (-inf) take no probability mass."""
    rng = np.random.default_rng(9)
    B, G, V = 400, 2, 16
    zq = rng.normal(0, 1, size=(G, V)).astype(np.float32)
    zp = rng.normal(0, 1, size=(G + 1, V)).astype(np.float32)
    zq[:, 12:] = -np.inf
    zp[:, 10:] = -np.inf
    draft, target, toks, temp = make_batch(zq, zp, 1.0, B, seed=4)
    out = oracle.verify(draft, target, toks, temp)
    assert np.all(out["accept_len"] >= 0)
    for b in range(B):
        k = out["accept_len"][b]
        assert out["tokens"][b, k] < 10


def test_scalar_mode_closed_form():
    """Scalar mode with a fixed pair: P(accept at 0) = min(1, exp(lp - lq))."""
    B, G = N_DRAWS, 2
    lp = np.zeros((B, G, 2), np.float32)
    lq_val, lp_val = np.float32(-1.2), np.float32(-1.9)
    lp[:, :, 0] = lq_val
    lp[:, :, 1] = lp_val
    out = oracle.accept_logprobs(lp, seed=3, offset=1)
    a = min(1.0, math.exp(float(lp_val) - float(lq_val)))
    k = out["accept_len"]
    assert binomtest(int((k >= 1).sum()), B, a).pvalue > ALPHA
    assert chisquare(np.bincount(k, minlength=G + 1),
                     np.array([1 - a, a * (1 - a), a * a]) * B).pvalue > ALPHA


def test_scalar_mode_agrees_with_full_call():
    """Scalar mode on the full call's gathered pairs (rounded to fp32) decides the
    same accept lengths, except where a decision margin is inside the 1e-5 band."""
    rec = specgen.config(2).replace(batch=64, vocab=2000)
    d = specgen.generate(rec)
    full = oracle.verify(d["logits_draft"], d["logits_target"], d["draft_tokens"],
                         d["temperature"], seed=0, offset=3)
    pairs = oracle.gather_logprobs(d["logits_draft"], d["logits_target"],
                                   d["draft_tokens"], d["temperature"])
    sc = oracle.accept_logprobs(pairs.astype(np.float32), seed=0, offset=3)
    diff = np.nonzero(sc["accept_len"] != full["accept_len"])[0]
    for b in diff:
        k = min(sc["accept_len"][b], full["accept_len"][b])
        assert np.nanmin(np.abs(full["acc_margin"][b, :k + 1])) < 1e-5
    assert len(diff) <= 1
