"""Property-based checks of the oracle on random small shapes (the FlashSpec
summary, Methodology section 3, names Hypothesis property tests of edge cases in
batch size and speculation length). Invariants that hold for every input:

* 0 <= k <= gamma for a valid sequence, -1 and all tokens -1 for an invalid one;
* tokens[:k] are the draft tokens, tokens[k] has positive target (greedy,
  bonus) or residual mass, tokens after k are -1;
* a greedy sequence's extra token is the first argmax of its target row k;
* the same call twice gives identical outputs.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st
from scipy.special import softmax

import oracle
import specgen


@st.composite
def cases(draw):
    B = draw(st.integers(1, 6))
    G = draw(st.integers(0, 9))
    V = draw(st.integers(1, 300))
    bf16 = draw(st.booleans())
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    sd = draw(st.sampled_from([0.5, 2.0, 6.0]))
    zq = rng.normal(0, sd, size=(B, G, V)).astype(np.float32)
    zp = (rng.normal(0, sd, size=(B, G + 1, V))).astype(np.float32)
    if draw(st.booleans()) and V > 2:
        zp[:, :, V - 1] = -np.inf  # padded vocabulary entry
    temps = np.array([draw(st.sampled_from([0.0, 0.05, 0.3, 1.0, 2.5])) for _ in range(B)],
                     np.float32)
    toks = np.zeros((B, G), np.int32)
    for b in range(B):
        if G:
            toks[b] = specgen.gumbel_max_tokens(zq[b], float(temps[b]), rng)
    if draw(st.booleans()) and G:
        toks[draw(st.integers(0, B - 1)), draw(st.integers(0, G - 1))] = draw(
            st.sampled_from([-1, V, V + 7]))
    if bf16:
        zq, zp = specgen.f32_to_bf16_bits(zq), specgen.f32_to_bf16_bits(zp)
    return zq, zp, toks, temps, draw(st.integers(0, 2**64 - 1)), draw(st.integers(0, 2**64 - 1))


@settings(max_examples=120, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(cases())
def test_oracle_invariants(case):
    zq, zp, toks, temps, seed, offset = case
    B, G1, V = zp.shape
    G = G1 - 1
    out = oracle.verify(zq, zp, toks, temps, seed=seed, offset=offset)
    again = oracle.verify(zq, zp, toks, temps, seed=seed, offset=offset)
    assert np.array_equal(out["accept_len"], again["accept_len"])
    assert np.array_equal(out["tokens"], again["tokens"])
    zpf = specgen.bf16_bits_to_f32(zp) if zp.dtype == np.uint16 else zp
    zqf = specgen.bf16_bits_to_f32(zq) if zq.dtype == np.uint16 else zq
    for b in range(B):
        k = out["accept_len"][b]
        tk = out["tokens"][b]
        bad_tok = G > 0 and (toks[b].min() < 0 or toks[b].max() >= V)
        if bad_tok:
            assert k == -1 and np.all(tk == -1)
            continue
        assert 0 <= k <= G
        assert np.array_equal(tk[:k], toks[b, :k])
        assert np.all(tk[k + 1:] == -1)
        j = tk[k]
        assert 0 <= j < V
        if temps[b] == 0:
            assert j == int(np.argmax(zpf[b, k]))
            continue
        inv_t = np.float32(1.0) / np.float32(temps[b])
        p = softmax((zpf[b, k] * inv_t).astype(np.float64))
        if k < G:
            q = softmax((zqf[b, k] * inv_t).astype(np.float64))
            assert p[j] - q[j] > -1e-12  # the token carries residual mass
        else:
            assert p[j] > 0
