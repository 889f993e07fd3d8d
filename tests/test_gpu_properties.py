"""Property-based GPU parity (Hypothesis): random batch sizes, speculation
lengths, vocabularies (ragged, tiny, not a multiple of the 16-byte group),
dtypes, temperatures (including greedy), padded -inf entries and invalid
tokens, each checked against the oracle under the match rules."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import specgen
from gpu_helpers import assert_parity, compare, record, run_gpu, to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


@st.composite
def cases(draw):
    B = draw(st.integers(1, 64))
    G = draw(st.integers(0, 70))
    cap = max(1, 8_000_000 // (B * (G + 1)))  # keep the oracle's work to about a second
    V = draw(st.one_of(st.integers(1, min(40, cap)), st.integers(1, min(5000, cap)),
                       st.integers(1, min(70000, cap))))
    bf16 = draw(st.booleans())
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    sd = draw(st.sampled_from([0.5, 2.0, 5.0]))
    base = rng.normal(0, sd, size=(B, G + 1, V))
    zp = (base + rng.normal(0, draw(st.sampled_from([0.2, 1.0])), size=base.shape)).astype(np.float32)
    zq = base[:, :G].astype(np.float32)
    if draw(st.booleans()) and V > 2:
        zp[:, :, V - 1] = -np.inf
        zq[:, :, V - 1] = -np.inf
    temps = np.array([draw(st.sampled_from([0.0, 0.05, 0.3, 0.7, 1.0, 1.5, 3.0])) for _ in range(B)],
                     np.float32)
    toks = np.zeros((B, G), np.int32)
    for b in range(B):
        if G:
            toks[b] = specgen.gumbel_max_tokens(zq[b], float(temps[b]), rng)
    if draw(st.booleans()) and G:
        toks[draw(st.integers(0, B - 1)), draw(st.integers(0, G - 1))] = V
    if bf16:
        zq, zp = specgen.f32_to_bf16_bits(zq), specgen.f32_to_bf16_bits(zp)
    return dict(logits_draft=np.ascontiguousarray(zq), logits_target=np.ascontiguousarray(zp),
                draft_tokens=toks, temperature=temps, seq_ids=np.arange(B)), \
        draw(st.integers(0, 2**64 - 1)), draw(st.integers(0, 2**64 - 1))


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(cases())
def test_random_shapes_match_oracle(case):
    d, seed, offset = case
    gpu = run_gpu(to_device(d), seed=seed, offset=offset)
    ref = oracle.verify(d["logits_draft"], d["logits_target"], d["draft_tokens"],
                        d["temperature"], seed=seed, offset=offset)
    rep = compare(gpu, ref, d["temperature"], data=d, seed=seed, offset=offset)
    assert_parity(rep, f"B={d['logits_target'].shape[0]} shape={d['logits_target'].shape}")
    _TOTALS.append(rep)


_TOTALS = []


def test_zz_record_random_shape_totals():
    """Counts summed over the random cases above (run after them)."""
    if not _TOTALS:
        pytest.skip("no random cases ran")
    tot = dict(n=0, exact=0, excused_accept=0, excused_resample=0, fails=[],
               low_margin_accept=0, low_margin_resample=0, lse_max_abs=0.0, lse_max_rel=0.0)
    for r in _TOTALS:
        for k in ("n", "exact", "excused_accept", "excused_resample", "low_margin_accept",
                  "low_margin_resample"):
            tot[k] += r[k]
        tot["fails"] += r["fails"]
        tot["lse_max_abs"] = max(tot["lse_max_abs"], r["lse_max_abs"])
        tot["lse_max_rel"] = max(tot["lse_max_rel"], r["lse_max_rel"])
    record(f"random shapes ({len(_TOTALS)} Hypothesis cases)", tot, cases=len(_TOTALS))
