"""The oracle against its own stored outputs on small seeded cases.

The fixture is written by tests/golden/make_golden.py, which calls only the
oracle; it guards the oracle against unintended edits. It is not a pin of the
method -- the pins are in test_oracle_pins.py and test_oracle_stats.py."""
import json
import os

import numpy as np

import oracle
import specgen

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_stored_outputs():
    with open(os.path.join(HERE, "golden", "oracle_small.json")) as f:
        cases = json.load(f)
    for c in cases:
        rec = specgen.config(c["config"]).replace(batch=c["batch"], vocab=c["vocab"])
        d = specgen.generate(rec)
        r = oracle.verify(d["logits_draft"], d["logits_target"], d["draft_tokens"],
                          d["temperature"], seed=c["seed"], offset=c["offset"])
        assert r["accept_len"].tolist() == c["accept_len"]
        assert r["tokens"].tolist() == c["tokens"]
        want = np.array([[float.fromhex(x) for x in row] for row in c["lse"]])
        got = r["lse"]
        both_nan = np.isnan(want) & np.isnan(got)
        assert np.all(both_nan | (np.abs(got - want) <= 1e-12 * np.maximum(1, np.abs(want))))
