"""GPU parity of spec_verify_outcomes (the law of the verification outcome)
against oracle.outcomes.

Match rule, per (sequence, length i):
* greedy and sentinel sequences: everything exact (integers, and 1/0);
* P(k = i | drafts): |gpu - oracle| <= 1e-6 * (i + 1) + 1e-5 * oracle. Each
  factor beta_j = min(1, exp(d_j)) moves by at most |delta d_j|, the error of
  two row log-normalisers (measured below 1.4e-7 each), and P(k = i) has
  i + 1 factors; the error is absolute because 1 - beta_i can be tiny;
* residual mass: |gpu - oracle| <= 2e-5;
* top-F lists: the GPU ranks values computed in binary32, so two tokens whose
  probabilities differ by less than their rounding may trade places. With
  tol = 2e-5 * (p + q) / S of the tokens involved (the scale of the two terms
  behind an entry) + 1e-9:
  - each listed token is distinct and valid, and its oracle probability is
    within tol of the oracle's probability at the same rank;
  - the GPU probability is within tol of the oracle's for the same token;
  - a rank whose oracle value is more than 2 tol from its neighbours
    (including rank F+1) must hold exactly the oracle's token.
  Ranks that differ only inside a tie are counted and reported.
"""
import numpy as np
import pytest
import torch

import device_draft_verification_amd as sv
import oracle
import specgen
from gpu_helpers import run_gpu, to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


def run_outcomes(t, F, seed=0, offset=0, ctx=None):
    zp = t["logits_target"]
    B, G1, V = zp.shape
    G = G1 - 1
    if ctx is None:
        ctx = sv.spec_verify_init(B, G, V, zp.dtype)
    run_gpu(t, seed=seed, offset=offset, ctx=ctx, with_lse=False)
    dev = zp.device
    tok = torch.full((B, G + 1, F), -7, dtype=torch.int32, device=dev)
    prob = torch.full((B, G + 1, F), -7.0, dtype=torch.float32, device=dev)
    pk = torch.full((B, G + 1), -7.0, dtype=torch.float32, device=dev)
    mass = torch.full((B, G + 1), -7.0, dtype=torch.float32, device=dev)
    sv.spec_verify_outcomes(ctx, t["logits_draft"] if G else None, zp,
                            t["draft_tokens"] if G else None, F, tok, prob, pk, mass)
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), probs=prob.cpu().numpy(), pk=pk.cpu().numpy(),
                mass=mass.cpu().numpy())


def oracle_rows(d, rows, F):
    rows = np.asarray(rows)
    G = d["logits_target"].shape[1] - 1
    return oracle.outcomes(np.ascontiguousarray(d["logits_draft"][rows]) if G else None,
                           np.ascontiguousarray(d["logits_target"][rows]),
                           np.ascontiguousarray(d["draft_tokens"][rows]) if G else None,
                           d["temperature"][rows], F, with_dist=True)


def compare(gpu, ref, temp, rows, F):
    """Apply the match rule to the sequences `rows` (gpu indexed by row id,
    ref by position in `rows`). Returns the count of tie-swapped ranks."""
    ties = 0
    for n, b in enumerate(rows):
        G1 = ref["pk"].shape[1]
        for i in range(G1):
            g_tok, o_tok = gpu["tokens"][b, i], ref["tokens"][n, i]
            where = f"seq {b} length {i}"
            if temp[n] == 0 or not np.isfinite(temp[n]) or ref["pk"][n].sum() == 0:
                assert np.array_equal(g_tok, o_tok), (where, g_tok, o_tok)
                assert np.array_equal(gpu["probs"][b, i], ref["probs"][n, i].astype(np.float32)), where
                assert gpu["pk"][b, i] == np.float32(ref["pk"][n, i]), where
                assert gpu["mass"][b, i] == np.float32(ref["mass"][n, i]), where
                continue
            o_pk = ref["pk"][n, i]
            assert abs(gpu["pk"][b, i] - o_pk) <= 1e-6 * (i + 1) + 1e-5 * o_pk, (where, gpu["pk"][b, i], o_pk)
            assert abs(gpu["mass"][b, i] - ref["mass"][n, i]) <= 2e-5, (where, gpu["mass"][b, i], ref["mass"][n, i])
            dist, scale = ref["dist"][n, i], ref["scale"][n, i]
            V = dist.size
            nf = min(F, V)
            assert (g_tok[nf:] == -1).all() and (o_tok[nf:] == -1).all()
            g_tok, o_tok = g_tok[:nf], o_tok[:nf]
            assert len(set(g_tok.tolist())) == nf and ((g_tok >= 0) & (g_tok < V)).all(), where
            order = np.argsort(-dist, kind="stable")[:nf + 1]
            assert np.array_equal(order[:nf], o_tok), where
            o_val = dist[o_tok]
            g_val = dist[g_tok]
            tol = 2e-5 * np.maximum(scale[o_tok], scale[g_tok]) + 1e-9
            assert (np.abs(g_val - o_val) <= tol).all(), (where, g_tok, o_tok, g_val - o_val, tol)
            assert (np.abs(gpu["probs"][b, i, :nf] - g_val) <= tol).all(), (where, gpu["probs"][b, i, :nf], g_val)
            nxt = dist[order[nf]] if order.size > nf else -np.inf
            vals = np.concatenate([[np.inf], o_val, [nxt]])
            for j in range(nf):
                unique = vals[j] - vals[j + 1] > 2 * tol[j] and vals[j + 1] - vals[j + 2] > 2 * tol[j]
                if unique:
                    assert g_tok[j] == o_tok[j], (where, j, g_tok, o_tok)
                elif g_tok[j] != o_tok[j]:
                    ties += 1
    return ties


@pytest.mark.parametrize("cfg,over,F", [
    (1, dict(), 8),                                  # fp32, full workload
    (2, dict(), 16),                                 # bf16, full workload
    (4, dict(batch=12, vocab=20008), 64),            # several splits, ragged tail, F = 64
    (4, dict(batch=12, vocab=20011), 5),             # element path
    (1, dict(batch=6, vocab=10003), 1),              # fp32 element path, F = 1
    (2, dict(batch=3, vocab=700, gamma=70), 4),      # more lengths than one wavefront
    (2, dict(batch=5, vocab=4096, gamma=0), 8),      # bonus only
    (3, dict(batch=4, vocab=33000), 12),             # Zipf rows
    (5, dict(batch=9, vocab=257), 64),               # tiny vocabulary
    (2, dict(batch=2, vocab=5), 8),                  # V < F
])
def test_outcomes_parity(cfg, over, F):
    rec = specgen.config(cfg).replace(**over)
    d = specgen.generate(rec)
    print(f"\n[outcomes {rec.name} {over} F={F}]", flush=True)
    gpu = run_outcomes(to_device(d), F)
    rows = np.arange(rec.batch)
    ref = oracle_rows(d, rows, F)
    ties = compare(gpu, ref, d["temperature"], rows, F)
    print(f"  ties={ties}", flush=True)


@pytest.fixture(scope="module", params=[4, 5])
def big(request):
    rec = specgen.config(request.param)
    d = specgen.generate(rec)
    t = to_device(d)
    yield rec, d, t
    del t
    torch.cuda.empty_cache()


def test_outcomes_full_size_sampled(big):
    rec, d, t = big
    F = 16
    print(f"\n[outcomes {rec.name} F={F}]", flush=True)
    gpu = run_outcomes(t, F)
    rng = np.random.default_rng(77 + rec.seed)
    rows = set(rng.choice(rec.batch, size=10, replace=False).tolist())
    rows.update(np.nonzero(d["temperature"] == 0)[0][:2].tolist())
    rows.update([0, rec.batch - 1])
    rows = np.array(sorted(rows))
    ties = 0
    for r in rows:
        ref = oracle_rows(d, [r], F)
        ties += compare(gpu, ref, d["temperature"][[r]], [r], F)
    print(f"  rows={len(rows)} ties={ties}", flush=True)
    # properties over every sequence
    pk = gpu["pk"].astype(np.float64)
    np.testing.assert_allclose(pk.sum(axis=1), 1.0, atol=1e-5)
    probs = gpu["probs"]
    assert (np.diff(probs, axis=2) <= 0).all()
    sampled = d["temperature"] > 0
    assert (probs[sampled].sum(axis=2) <= 1.0 + 1e-5).all()
    again = run_outcomes(t, F)
    for key in ("tokens", "probs", "pk", "mass"):
        assert np.array_equal(again[key], gpu[key]), key


def test_outcomes_degenerate_rows():
    """p = q (every draft accepted, lists fall back to p), disjoint supports
    (the first draft always rejected), greedy ties, sentinels."""
    rng = np.random.default_rng(3)
    B, G, V, F = 6, 3, 96, 6
    zq = rng.normal(0, 1, size=(B, G, V)).astype(np.float32)
    zp = rng.normal(0, 1, size=(B, G + 1, V)).astype(np.float32)
    zp[0, :G] = zq[0]                                   # p = q
    zq[1] = -np.inf; zq[1, :, :8] = 0.0                 # disjoint supports
    zp[1] = -np.inf; zp[1, :, 16:] = rng.normal(0, 1, size=(G + 1, V - 16))
    zp[2] = np.round(zp[2])                             # greedy with ties
    temp = np.array([0.8, 1.0, 0.0, 1.2, np.nan, 0.9], np.float32)
    toks = rng.integers(0, V, size=(B, G)).astype(np.int32)
    toks[1] = 3
    toks[5, 1] = V + 4                                   # sentinel: token out of range
    d = dict(logits_draft=zq, logits_target=zp, draft_tokens=toks, temperature=temp)
    gpu = run_outcomes(to_device(d), F)
    ref = oracle.outcomes(zq, zp, toks, temp, F, with_dist=True)
    compare(gpu, ref, temp, np.arange(B), F)
    assert gpu["pk"][0].tolist() == [0.0] * G + [1.0]
    assert gpu["pk"][1, 0] == 1.0
    assert (gpu["tokens"][4] == -1).all() and (gpu["tokens"][5] == -1).all()


def test_outcomes_ties_at_the_threshold():
    """Rows whose F-th value is shared by thousands of tokens: residuals that
    are exactly 0 outside five tokens (the target equals the draft elsewhere
    and has more mass there), and greedy rows of coarse logits. The lists are
    those of a stable descending sort, lowest index first among equal values,
    so here they equal the oracle's token for token."""
    rng = np.random.default_rng(11)
    B, G, V, F = 4, 2, 65536, 16
    zq = rng.normal(0, 1, size=(B, G, V)).astype(np.float32)
    zp = np.empty((B, G + 1, V), np.float32)
    zp[:, :G] = zq
    zp[:, G] = rng.normal(0, 1, size=(B, V))
    for b in range(B):
        for i in range(G):
            zp[b, i, rng.choice(V, 5, replace=False)] += 3.0
    zp[2] = np.round(zp[2] * 2) / 2                      # greedy, coarse tied logits
    temp = np.array([1.0, 0.7, 0.0, 1.3], np.float32)
    toks = rng.integers(0, V, size=(B, G)).astype(np.int32)
    d = dict(logits_draft=zq, logits_target=zp, draft_tokens=toks, temperature=temp)
    gpu = run_outcomes(to_device(d), F)
    ref = oracle.outcomes(zq, zp, toks, temp, F, with_dist=True)
    compare(gpu, ref, temp, np.arange(B), F)
    for b in (0, 1, 3):
        for i in range(G):
            assert (ref["dist"][b, i] > 0).sum() == 5, (b, i)
            assert np.array_equal(gpu["tokens"][b, i], ref["tokens"][b, i]), (b, i)
    assert np.array_equal(gpu["tokens"][2], ref["tokens"][2])


def test_outcomes_needs_a_verification_first():
    ctx = sv.spec_verify_init(2, 2, 64, torch.float32)
    z = torch.zeros(2, 3, 64, device="cuda")
    q = torch.zeros(2, 2, 64, device="cuda")
    tk = torch.zeros(2, 2, dtype=torch.int32, device="cuda")
    tok = torch.zeros(2, 3, 4, dtype=torch.int32, device="cuda")
    pr = torch.zeros(2, 3, 4, device="cuda")
    pk = torch.zeros(2, 3, device="cuda")
    with pytest.raises(sv.SpecVerifyError) as e:
        sv.spec_verify_outcomes(ctx, q, z, tk, 4, tok, pr, pk)
    assert e.value.code == sv.binding.SPEC_ESTATE
    with pytest.raises(sv.SpecVerifyError):
        sv.spec_verify_outcomes(ctx, q, z, tk, 65, torch.zeros(2, 3, 65, dtype=torch.int32,
                                                                device="cuda"),
                                torch.zeros(2, 3, 65, device="cuda"), pk)


# ------------------------------------------------------------------ fan-out ---
# spec_outcome_fanout against oracle.outcome_fanout on the same float32
# inputs: entry counts exact. The expected hit rate adds the same exact
# binary64 products, the oracle in placement order and the kernel in an order
# of its own; each of the two sums of n <= 16384 non-negative terms is within
# n 2^-53 < 2e-12 of the exact sum, relative to it, so they may differ by
# 4e-12 of it.

def run_fanout(pk, probs, budget):
    pk_d = torch.from_numpy(np.ascontiguousarray(pk, dtype=np.float32)).cuda()
    pr_d = torch.from_numpy(np.ascontiguousarray(probs, dtype=np.float32)).cuda()
    B, L = pk.shape
    n = torch.full((B, L), -7, dtype=torch.int32, device="cuda")
    hit = torch.full((B,), -7.0, dtype=torch.float64, device="cuda")
    sv.spec_outcome_fanout(pk_d, pr_d, budget, n, hit)
    torch.cuda.synchronize()
    return n.cpu().numpy(), hit.cpu().numpy()


def check_fanout(pk, probs, budget, label):
    n, hit = run_fanout(pk, probs, budget)
    n_ref, hit_ref = oracle.outcome_fanout(pk, probs, budget)
    assert np.array_equal(n, n_ref), (label, budget, np.argwhere(n != n_ref)[:4])
    assert (np.abs(hit - hit_ref) <= 4e-12 * hit_ref).all(), (label, budget, np.abs(hit - hit_ref).max())
    return n


def sorted_lists(rng, B, L, F, levels=None):
    pk = rng.dirichlet(np.ones(L), size=B)
    probs = np.sort(rng.dirichlet(np.ones(F + 3), size=(B, L))[..., :F], axis=-1)[..., ::-1]
    if levels:  # coarse values, so that equal worths (ties) occur
        pk = np.round(pk * levels) / levels
        probs = np.round(probs * levels) / levels
    return pk.astype(np.float32), np.ascontiguousarray(probs, dtype=np.float32)


@pytest.mark.parametrize("B,L,F,levels", [
    (64, 9, 16, None),      # the bench workload's shape of lists
    (32, 9, 16, 8),         # many equal worths
    (8, 1, 1, None),        # one length, one entry
    (8, 64, 3, None),       # one length per lane
    (8, 65, 5, 4),          # a second length on lane 0
    (4, 131, 16, None),     # gamma = 130
    (2, 256, 64, 16),       # the largest shape: four lengths per lane, 64 KiB of lists
])
def test_fanout_parity(B, L, F, levels):
    rng = np.random.default_rng(B * 1000 + L * 10 + F)
    pk, probs = sorted_lists(rng, B, L, F, levels)
    print(f"\n[fanout B={B} L={L} F={F} levels={levels}]", flush=True)
    for budget in sorted({0, 1, 2, F, L, 37, L * F // 3, L * F - 1, L * F, L * F + 5}):
        if budget >= 0:
            n = check_fanout(pk, probs, budget, (B, L, F))
            assert (n.sum(axis=1) == min(budget, L * F)).all()


def test_fanout_odd_values():
    """Zero, negative and NaN worths, lists that are not sorted, and length
    probabilities of a greedy sequence (0 or 1)."""
    rng = np.random.default_rng(9)
    B, L, F = 6, 7, 6
    pk, probs = sorted_lists(rng, B, L, F)
    pk[0] = 0.0
    pk[1, 2] = np.nan
    pk[2, 3] = -0.5
    probs[3] = rng.random((L, F)).astype(np.float32)    # unsorted lists
    probs[4, 1, 2] = np.nan
    pk[5] = 0.0
    pk[5, 4] = 1.0                                       # greedy: one certain length
    probs[5] = 0.0
    probs[5, :, 0] = 1.0
    for budget in (1, 3, 10, L * F):
        check_fanout(pk, probs, budget, "odd")
    n, hit = run_fanout(pk, probs, 3)
    assert n[5, 4] == 1 and hit[5] == 1.0


def test_fanout_on_the_outcome_law():
    """End to end: the law of a workload's verification feeds the budget."""
    rec = specgen.config(2)
    d = specgen.generate(rec)
    F = 16
    gpu = run_outcomes(to_device(d), F)
    for budget in (4, 32, (rec.gamma + 1) * F):
        n = check_fanout(gpu["pk"], gpu["probs"], budget, rec.name)
        # the lists are non-increasing, so the placed entries are the most
        # valuable ones: none left out is worth more than one placed
        w = gpu["pk"].astype(np.float64)[:, :, None] * gpu["probs"].astype(np.float64)
        placed = np.arange(F)[None, None, :] < n[:, :, None]
        for b in range(rec.batch):
            if placed[b].any() and (~placed[b]).any():
                assert w[b][placed[b]].min() >= w[b][~placed[b]].max(), (b, budget)
