"""Pins of the sampled draft-tree verification oracle (multi-step speculative
sampling, one draft distribution per node): on chains it is the verification
oracle, at T = 0 the greedy tree oracle, and its outputs follow the target
model, the property the rule is published for (SpecInfer, ASPLOS 2024), here
checked by chi-square at V = 8."""
import numpy as np
import pytest
from scipy import stats

import oracle
import specgen


def chain_inputs(d):
    """The verification workload as chain trees: node i + 1 holds draft token i,
    draft row i is the distribution token i was drawn from, target row i the
    distribution after position i."""
    zq, zt = d["logits_draft"], d["logits_target"]
    B, G1, V = zt.shape
    G = G1 - 1
    par = np.tile(np.arange(-1, G, dtype=np.int32), (B, 1))
    tok = np.zeros((B, G1), np.int32)
    tok[:, 1:] = d["draft_tokens"]
    q = np.zeros((B, G1, V), zq.dtype)
    q[:, :G] = zq
    return par, tok, np.full(B, G1, np.int32), q, zt


@pytest.mark.parametrize("cfg,over", [
    (1, dict()), (2, dict()), (3, dict(batch=6, vocab=4096)),
    (4, dict(batch=40, vocab=3000)), (5, dict(batch=20, vocab=2048)),
    (2, dict(batch=6, vocab=500, gamma=12)),
])
def test_chain_is_the_verifier(cfg, over):
    rec = specgen.config(cfg).replace(**over)
    d = specgen.generate(rec)
    par, tok, n, q, zt = chain_inputs(d)
    for offset in (0, 7):
        o = oracle.tree_verify_sample(par, tok, n, q, zt, d["temperature"], seed=5, offset=offset,
                                      seq_ids=d["seq_ids"])
        r = oracle.verify(d["logits_draft"], d["logits_target"], d["draft_tokens"],
                          d["temperature"], seed=5, offset=offset, seq_ids=d["seq_ids"])
        assert np.array_equal(o["length"], r["accept_len"])
        for b in range(rec.batch):
            k = r["accept_len"][b]
            if k < 0:
                assert o["extra"][b] == -1 and (o["path"][b] == -1).all()
                continue
            assert o["path"][b, :k].tolist() == list(range(1, k + 1))
            assert (o["path"][b, k:] == -1).all()
            assert o["extra"][b] == r["tokens"][b, k]


def test_sentinels_and_greedy():
    rec = specgen.config(4).replace(batch=24, vocab=2000)
    d = specgen.generate(rec)
    par, tok, n, q, zt = chain_inputs(d)
    temp = d["temperature"].copy()
    temp[1], temp[2] = np.nan, -1.0
    tok[3, 2] = rec.vocab
    par[4, 3] = 4
    n[5] = 0
    o = oracle.tree_verify_sample(par, tok, n, q, zt, temp, seed=1)
    assert o["length"][1:6].tolist() == [-1] * 5 and (o["extra"][1:6] == -1).all()
    g = temp == 0
    assert g.any()
    og = oracle.tree_verify_greedy(par[g], tok[g], n[g], zt[g])
    for key in ("length", "path", "extra"):
        assert np.array_equal(o[key][g], og[key]), key


def draw_tree(rng, logq_root, logq_child, k1, k2):
    """Root, k1 children drawn i.i.d. from q_root, each with k2 children drawn
    i.i.d. from q(. | child token). Returns parent, token, and each node's path
    of tokens."""
    V = logq_root.size
    par, tok, paths = [-1], [0], [()]
    p_root = np.exp(logq_root)
    for _ in range(k1):
        x = int(rng.choice(V, p=p_root))
        par.append(0)
        tok.append(x)
        paths.append((x,))
    n1 = len(par)
    for c in range(1, n1):
        x1 = tok[c]
        pq = np.exp(logq_child[x1])
        for _ in range(k2):
            x2 = int(rng.choice(V, p=pq))
            par.append(c)
            tok.append(x2)
            paths.append((x1, x2))
    return np.array(par, np.int32), np.array(tok, np.int32), paths


def log_softmax(z):
    z = z - z.max(axis=-1, keepdims=True)
    return z - np.log(np.exp(z).sum(axis=-1, keepdims=True))


def test_outputs_follow_the_target(n_trials=10000, k1=3, k2=2, alpha=0.01):
    """Children drawn from the draft model: the first emitted token follows
    p(. | root) and, where there is one, the second follows p(. | first)."""
    V = 8
    rng = np.random.default_rng(11)
    zp0, zp1, zp2 = rng.normal(0, 1.5, V), rng.normal(0, 1.5, (V, V)), rng.normal(0, 1.5, (V, V, V))
    zq0 = zp0 + rng.normal(0, 1.0, V)
    zq1 = zp1 + rng.normal(0, 1.0, (V, V))
    lq0, lq1 = log_softmax(zq0.astype(np.float32).astype(np.float64)), \
        log_softmax(zq1.astype(np.float32).astype(np.float64))
    M = 1 + k1 + k1 * k2
    batch = 1000
    first = np.zeros(V, np.int64)
    second = np.zeros((V, V), np.int64)
    for start in range(0, n_trials, batch):
        par = np.zeros((batch, M), np.int32)
        tok = np.zeros((batch, M), np.int32)
        zt = np.zeros((batch, M, V), np.float32)
        zq = np.zeros((batch, M, V), np.float32)
        for b in range(batch):
            pb, tb, paths = draw_tree(rng, lq0, lq1, k1, k2)
            par[b], tok[b] = pb, tb
            for u, pth in enumerate(paths):
                if len(pth) == 0:
                    zt[b, u], zq[b, u] = zp0, zq0
                elif len(pth) == 1:
                    zt[b, u], zq[b, u] = zp1[pth[0]], zq1[pth[0]]
                else:
                    zt[b, u] = zp2[pth[0], pth[1]]
        o = oracle.tree_verify_sample(par, tok, np.full(batch, M, np.int32), zq, zt,
                                      np.ones(batch, np.float32), seed=3,
                                      seq_ids=np.arange(start, start + batch))
        for b in range(batch):
            L = o["length"][b]
            emitted = [tok[b, s] for s in o["path"][b, :L]] + [o["extra"][b]]
            first[emitted[0]] += 1
            if len(emitted) > 1:
                second[emitted[0], emitted[1]] += 1
    p0 = np.exp(log_softmax(zp0.astype(np.float32).astype(np.float64)))
    assert stats.chisquare(first, n_trials * p0).pvalue > alpha
    p1 = np.exp(log_softmax(zp1.astype(np.float32).astype(np.float64)))
    chi, df = 0.0, 0
    for x in range(V):
        m = second[x].sum()
        if m >= 50:
            e = m * p1[x]
            chi += ((second[x] - e) ** 2 / e).sum()
            df += V - 1
    assert df >= 4 * (V - 1)
    assert stats.chi2.sf(chi, df) > alpha
