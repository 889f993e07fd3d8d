"""GPU parity of draft-tree pruning and greedy tree verification against the
oracle. Everything here is exact: path scores are the same double additions
in the same order (compared bit for bit), the kept sets and renumbering are
integer results, and greedy verification takes raw-logit argmaxes (lowest
index on ties) in the logits' own precision."""
import numpy as np
import pytest
import torch

import device_draft_verification_amd as sv
import oracle
import specgen

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_prune(parent, logq, tau, budget):
    B, M = parent.shape
    cum = torch.empty((B, M), dtype=torch.float64, device="cuda")
    ni = torch.empty((B, M), dtype=torch.int32, device="cuda")
    npar = torch.empty((B, M), dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, dtype=torch.int32, device="cuda")
    sv.spec_tree_prune(dev(parent), dev(logq), tau, budget, cum, ni, npar, cnt)
    torch.cuda.synchronize()
    return dict(cum=cum.cpu().numpy(), new_index=ni.cpu().numpy(), new_parent=npar.cpu().numpy(),
                count=cnt.cpu().numpy())


def check_prune(g, o):
    assert np.array_equal(g["count"], o["count"])
    assert np.array_equal(g["new_index"], o["new_index"])
    assert np.array_equal(g["new_parent"], o["new_parent"])
    assert np.array_equal(g["cum"].view(np.uint64), o["cum"].view(np.uint64))


@pytest.mark.parametrize("B,M", [(7, 1), (16, 24), (256, 64), (40, 256)])
def test_prune_parity(B, M):
    trees = specgen.draft_trees(B, M, 1000, seed=M)
    for tau, K in ((np.log(1e-3), max(1, M // 2)), (-np.inf, M), (np.log(0.3), 3), (0.0, 1)):
        g = gpu_prune(trees["parent"], trees["logq"], tau, K)
        o = oracle.tree_prune(trees["parent"], trees["logq"], tau, K)
        check_prune(g, o)


def test_prune_ties_and_sentinels():
    trees = specgen.draft_trees(4, 9, 100, seed=2)
    par, lq = trees["parent"].copy(), trees["logq"].copy()
    par[0, 5] = 7                                   # not topological
    lq[1, 2] = 0.25                                 # positive
    lq[2, 3] = np.nan
    par[3] = [-1, 0, 0, 0, 0, 1, 1, 2, 2]           # equal scores among siblings
    lq[3] = [0] + [np.log(0.25)] * 4 + [np.log(0.5)] * 4
    for K in (1, 3, 6, 9):
        check_prune(gpu_prune(par, lq, -np.inf, K), oracle.tree_prune(par, lq, -np.inf, K))


def gpu_verify(trees, n_nodes, target, dtype):
    B, M = trees["parent"].shape
    V = target.shape[-1]
    ctx = sv.spec_tree_verify_init(B, M, V, dtype)
    if dtype == torch.bfloat16:
        t = torch.from_numpy(target.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        t = dev(target)
    L = torch.empty(B, dtype=torch.int32, device="cuda")
    path = torch.empty((B, M), dtype=torch.int32, device="cuda")
    extra = torch.empty(B, dtype=torch.int32, device="cuda")
    sv.spec_tree_verify_greedy(ctx, dev(trees["parent"]), dev(trees["token"]), dev(n_nodes), t,
                               L, path, extra)
    torch.cuda.synchronize()
    return dict(length=L.cpu().numpy(), path=path.cpu().numpy(), extra=extra.cpu().numpy())


@pytest.mark.parametrize("B,M,V,dt", [(8, 12, 1000, "f32"), (32, 20, 4099, "bf16"),
                                      (16, 64, 32000, "bf16"), (4, 256, 777, "f32")])
def test_greedy_tree_parity(B, M, V, dt):
    trees = specgen.draft_trees(B, M, V, seed=V, max_children=3)
    target = specgen.tree_target_logits(trees, V, seed=1, dtype=dt)
    n = np.full(B, M, np.int32)
    n[::3] = np.maximum(1, M // 2)                    # some trees use fewer nodes
    g = gpu_verify(trees, n, target, torch.bfloat16 if dt == "bf16" else torch.float32)
    o = oracle.tree_verify_greedy(trees["parent"], trees["token"], n, target)
    for key in ("length", "path", "extra"):
        assert np.array_equal(g[key], o[key]), key
    assert (o["length"] >= 2).sum() >= 1


def test_greedy_tree_full_workload():
    """B = 256 trees of 16 nodes over the V = 152064 bf16 vocabulary (the
    B=256 workload's batch and vocabulary); oracle on every tree."""
    B, M, V = 256, 16, 152064
    trees = specgen.draft_trees(B, M, V, seed=21)
    target = specgen.tree_target_logits(trees, V, seed=3)
    n = np.full(B, M, np.int32)
    g = gpu_verify(trees, n, target, torch.bfloat16)
    o = oracle.tree_verify_greedy(trees["parent"], trees["token"], n, target)
    for key in ("length", "path", "extra"):
        assert np.array_equal(g[key], o[key]), key


def test_greedy_tree_sentinels_and_no_finite_row():
    B, M, V = 5, 6, 64
    trees = specgen.draft_trees(B, M, V, seed=8)
    target = specgen.tree_target_logits(trees, V, seed=2, dtype="f32")
    tok = trees["token"].copy()
    tok[1, 3] = V
    par = trees["parent"].copy()
    par[2, 4] = 5
    target[3, 0, :] = -np.inf                      # the root row of tree 3 has no finite logit
    n = np.array([M, M, M, M, 0], np.int32)
    t2 = dict(parent=par, token=tok)
    g = gpu_verify(t2, n, target, torch.float32)
    o = oracle.tree_verify_greedy(par, tok, n, target)
    for key in ("length", "path", "extra"):
        assert np.array_equal(g[key], o[key]), key
    assert o["length"].tolist()[1:] == [-1, -1, -1, -1]
