"""The benchmark's algorithmic byte counts (the numerator of its roofline
figure) against the sizes the verification's definition fixes: every logit a
step must read, once. Reference values are the products written out, for the
B = 256, gamma = 8, V = 152064 and B = 512, gamma = 4, V = 201088 bf16
workloads."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import specgen  # noqa: E402


def test_row_kernel_reads_every_row_once():
    rec = specgen.config(4)
    B, G, V = rec.batch, rec.gamma, rec.vocab
    t = np.full(B, 1.0, np.float32)
    k = bench.algorithmic_bytes(rec, t, np.zeros(B, np.int32))
    assert k["row_norm"] == 256 * 17 * 152064 * 2 == 1_323_565_056
    rec5 = specgen.config(5)
    k5 = bench.algorithmic_bytes(rec5, np.full(512, 0.8, np.float32), np.zeros(512, np.int32))
    assert k5["row_norm"] == 512 * 9 * 201088 * 2 == 1_853_227_008


def test_greedy_sequences_read_target_rows_only():
    rec = specgen.config(4)
    t = specgen.generate(rec)["temperature"]
    assert int((t == 0).sum()) == 26
    k = bench.algorithmic_bytes(rec, t, np.zeros(rec.batch, np.int32))
    assert k["row_norm"] == (230 * 17 + 26 * 9) * 152064 * 2 == 1_260_306_432


def test_residual_bytes_follow_the_outcome():
    rec = specgen.config(4).replace(batch=5)
    G, V = rec.gamma, rec.vocab
    t = np.array([1.0, 1.0, 0.0, 1.0, 0.5], np.float32)
    k_len = np.array([0, G, 3, -1, G - 1], np.int32)  # reject, bonus, greedy, sentinel, reject
    k = bench.algorithmic_bytes(rec, t, k_len)
    assert k["residual"] == (2 + 1 + 0 + 0 + 2) * V * 2
    every = bench.algorithmic_bytes(specgen.config(4), np.ones(256, np.float32),
                                    np.zeros(256, np.int32))
    assert every["residual"] == 256 * 2 * 152064 * 2 == 155_713_536
