"""The GPU parity tests' match rules, exercised on the CPU: outputs that the
oracle itself produces under the other side of a low-margin decision pass as
excused; any other deviation, and any malformed output, is a mismatch. The
'GPU' outputs here are built from oracle runs, so no device is needed."""
import numpy as np
import pytest

import oracle
import specgen

gpu_helpers = pytest.importorskip("gpu_helpers")
compare = gpu_helpers.compare


def _case(n=64, seed=3, V=64, G=4, T=1.0):
    rec = specgen.config(2).replace(batch=n, vocab=V, gamma=G, temperature=T, seed=seed)
    d = specgen.generate(rec)
    ref = oracle.verify(d["logits_draft"], d["logits_target"], d["draft_tokens"],
                        d["temperature"], seed=0, offset=0, seq_ids=d["seq_ids"])
    return d, ref


def _copy(ref):
    return dict(accept_len=ref["accept_len"].copy(), tokens=ref["tokens"].copy())


def test_identical_outputs_are_exact():
    d, ref = _case()
    rep = compare(_copy(ref), ref, d["temperature"], data=d)
    assert rep["exact"] == len(ref["accept_len"]) and not rep["fails"]


def test_a_changed_token_without_a_small_margin_fails():
    d, ref = _case()
    g = _copy(ref)
    j = int(np.argmax(ref["res_margin"]))
    k = g["accept_len"][j]
    g["tokens"][j, k] = (g["tokens"][j, k] + 1) % 64
    rep = compare(g, ref, d["temperature"], data=d)
    assert [f[0] for f in rep["fails"]] == [j]


def test_a_low_margin_draw_excuses_only_the_neighbour_token():
    d, ref = _case()
    j = 5
    k = int(ref["accept_len"][j])
    tok = int(ref["tokens"][j, k])
    fake = dict(ref, res_margin=ref["res_margin"].copy(), res_alt=ref["res_alt"].copy())
    fake["res_margin"][j] = 1e-7
    # find a neighbour with positive residual mass: any token other than tok
    alt = (tok + 3) % 64
    fake["res_alt"][j] = alt
    g = _copy(ref)
    g["tokens"][j, k] = alt
    rep = compare(g, fake, d["temperature"], data=d)
    assert rep["excused_resample"] == 1 and not rep["fails"]
    g["tokens"][j, k] = (alt + 1) % 64 if (alt + 1) % 64 != tok else (alt + 2) % 64
    rep = compare(g, fake, d["temperature"], data=d)
    assert [f[0] for f in rep["fails"]] == [j]


def test_malformed_outputs_fail_even_when_the_oracle_agrees():
    d, ref = _case()
    g = _copy(ref)
    j = int(np.nonzero(ref["accept_len"] < 4)[0][0])
    k = int(g["accept_len"][j])
    g["tokens"][j, k + 1] = 7                # a pad that is not -1
    fake = dict(ref, tokens=g["tokens"])     # even if the oracle said the same
    rep = compare(g, fake, d["temperature"], data=d)
    assert rep["fails"] and rep["fails"][0][1] == "malformed"


def test_a_parted_length_needs_a_small_margin_and_the_oracles_own_outcome():
    """A sequence whose first rejection the GPU placed one position later
    passes only if the oracle's margin there is small and the GPU's extra
    token is what the oracle draws when it takes the same side."""
    d, ref = _case(n=128, V=32, G=4, T=1.0)
    js = np.nonzero(ref["accept_len"] < 4)[0]
    j = int(js[0])
    k = int(ref["accept_len"][j])
    sid = int(d["seq_ids"][j])
    words = [oracle.philox_words(0, 0, sid, i) for i in range(5)]
    ua = np.array([oracle.uniform24(int(w[0])) for w in words])
    ur = np.array([oracle.uniform24(int(w[1])) for w in words])
    ua[k] = 0.0
    other = oracle.verify_sequence(d["logits_draft"][j], d["logits_target"][j],
                                   d["draft_tokens"][j], float(d["temperature"][j]), ua, ur)
    kg = other["accept_len"]
    assert kg > k
    g = _copy(ref)
    g["accept_len"][j] = kg
    g["tokens"][j] = other["tokens"]
    # with the oracle's real margin (not small) it is a mismatch
    rep = compare(g, ref, d["temperature"], data=d)
    assert [f[0] for f in rep["fails"]] == [j]
    # with a small margin at the parting position it is excused
    fake = dict(ref, acc_margin=ref["acc_margin"].copy())
    fake["acc_margin"][j, k] = 3e-6
    rep = compare(g, fake, d["temperature"], data=d)
    assert rep["excused_accept"] == 1 and not rep["fails"]
    # but not with another extra token
    g["tokens"][j, kg] = (g["tokens"][j, kg] + 1) % 32
    rep = compare(g, fake, d["temperature"], data=d)
    assert [f[0] for f in rep["fails"]] == [j]
    # nor with the small margin at an earlier position than the parting one
    if k > 0:
        g["tokens"][j] = other["tokens"]
        fake2 = dict(ref, acc_margin=ref["acc_margin"].copy())
        fake2["acc_margin"][j, k - 1] = 3e-6
        rep = compare(g, fake2, d["temperature"], data=d)
        assert [f[0] for f in rep["fails"]] == [j]


def test_greedy_sequences_must_match_exactly():
    rec = specgen.config(4).replace(batch=30, vocab=500)
    d = specgen.generate(rec)
    ref = oracle.verify(d["logits_draft"], d["logits_target"], d["draft_tokens"],
                        d["temperature"], seq_ids=d["seq_ids"])
    j = int(np.nonzero(d["temperature"] == 0)[0][0])
    g = _copy(ref)
    k = int(g["accept_len"][j])
    g["tokens"][j, k] = (g["tokens"][j, k] + 1) % 500
    fake = dict(ref, res_margin=np.zeros_like(ref["res_margin"]))
    rep = compare(g, fake, d["temperature"], data=d)
    assert [f[0] for f in rep["fails"]] == [j]
