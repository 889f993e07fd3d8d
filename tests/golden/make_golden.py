"""Writes oracle_small.json: the oracle's outputs on small seeded cases.

It calls only the oracle and the seeded input generator. The stored values pin
the oracle against its own later edits (any change to its arithmetic must come
with a regenerated file and a stated reason); they are not a pin of the method.
Run from the repository root: python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import specgen  # noqa: E402

CASES = [
    # (config whose recipe is reused, batch, vocab, seed, offset)
    (1, 1, 1000, 0, 0),
    (2, 4, 777, 0, 1),
    (3, 3, 1024, 5, 0),
    (4, 10, 999, 0, 2),
    (5, 4, 4001, 9, 3),
]


def build_cases():
    out = []
    for cfg, B, V, seed, offset in CASES:
        rec = specgen.config(cfg).replace(batch=B, vocab=V)
        d = specgen.generate(rec)
        r = oracle.verify(d["logits_draft"], d["logits_target"], d["draft_tokens"],
                          d["temperature"], seed=seed, offset=offset)
        out.append(dict(config=cfg, batch=B, vocab=V, seed=seed, offset=offset,
                        accept_len=r["accept_len"].tolist(),
                        tokens=r["tokens"].tolist(),
                        lse=[[float.hex(float(x)) for x in row] for row in r["lse"]]))
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(build_cases(), f, indent=1)
