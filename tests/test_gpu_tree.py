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


@pytest.mark.parametrize("B,M", [(7, 1), (16, 24), (256, 64), (9, 65), (40, 256)])
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


# ------------------------------------------------- sampled verification ---
#
# Match rule: lengths, paths and extra tokens exact, except a tree whose
# oracle takes an accept decision or the draw with a log-margin below 1e-5
# (the verifier's rule), which is counted as flagged. Sentinels and T = 0
# trees are exact.

MARGIN = 1e-5


def to_dev_logits(x, dtype):
    if dtype == torch.bfloat16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return dev(x)


def gpu_sample(parent, token, n_nodes, draft, target, temperature, dtype, seed=0, offset=0,
               ctx=None):
    B, M = parent.shape
    V = target.shape[-1]
    own = ctx is None
    if own:
        ctx = sv.spec_tree_verify_init(B, M, V, dtype)
    L = torch.empty(B, dtype=torch.int32, device="cuda")
    path = torch.empty((B, M), dtype=torch.int32, device="cuda")
    extra = torch.empty(B, dtype=torch.int32, device="cuda")
    sv.spec_tree_verify_sample(ctx, dev(parent), dev(token), dev(n_nodes),
                               to_dev_logits(draft, dtype), to_dev_logits(target, dtype),
                               dev(np.asarray(temperature, np.float32)), seed, offset, L, path, extra)
    torch.cuda.synchronize()
    if own:
        sv.spec_tree_verify_destroy(ctx)
    return dict(length=L.cpu().numpy(), path=path.cpu().numpy(), extra=extra.cpu().numpy())


def check_sample(g, o, temperature, rows=None):
    rows = np.arange(len(o["length"])) if rows is None else np.asarray(rows)
    flagged = 0
    for n, b in enumerate(rows):
        near = o["length"][n] >= 0 and temperature[n] > 0 and (
            o["acc_margin"][n] < MARGIN or o["res_margin"][n] < MARGIN)
        same = (g["length"][b] == o["length"][n] and g["extra"][b] == o["extra"][n]
                and np.array_equal(g["path"][b], o["path"][n]))
        if near:
            flagged += 1
            continue
        assert same, (b, g["length"][b], o["length"][n], g["extra"][b], o["extra"][n],
                      g["path"][b][:6], o["path"][n][:6])
    return flagged


@pytest.mark.parametrize("cfg,over", [(1, dict()), (2, dict()), (3, dict(batch=6, vocab=4096)),
                                      (4, dict(batch=40, vocab=3000)), (5, dict(batch=20, vocab=2048))])
def test_sample_chains(cfg, over):
    """Chain trees built from the verification workloads (node i + 1 holds draft
    token i), including greedy and sentinel sequences."""
    rec = specgen.config(cfg).replace(**over)
    d = specgen.generate(rec)
    zq, zt = d["logits_draft"], d["logits_target"]
    B, G1, V = zt.shape
    par = np.tile(np.arange(-1, G1 - 1, dtype=np.int32), (B, 1))
    tok = np.zeros((B, G1), np.int32)
    tok[:, 1:] = d["draft_tokens"]
    q = np.zeros((B, G1, V), zq.dtype)
    q[:, :G1 - 1] = zq
    n = np.full(B, G1, np.int32)
    dt = torch.bfloat16 if rec.dtype == "bf16" else torch.float32
    print(f"\n[tree sample chains {rec.name} {over}]", flush=True)
    for offset in (0, 5):
        g = gpu_sample(par, tok, n, q, zt, d["temperature"], dt, seed=3, offset=offset)
        o = oracle.tree_verify_sample(par, tok, n, q, zt, d["temperature"], seed=3, offset=offset)
        f = check_sample(g, o, d["temperature"])
        print(f"  offset {offset}: flagged {f}/{B}, mean length {g['length'].mean():.2f}", flush=True)


@pytest.mark.parametrize("B,M,V,dt", [(16, 12, 1000, "f32"), (32, 20, 4099, "bf16"),
                                      (8, 64, 32000, "bf16"), (4, 256, 777, "f32"),
                                      (600, 8, 300, "bf16"),   # more trees than resident at once
                                      (3, 5, 5, "f32")])       # one tile: three parts own nothing
def test_sample_random_trees(B, M, V, dt):
    trees = specgen.draft_trees(B, M, V, seed=M + V)
    zt = specgen.tree_target_logits(trees, V, seed=1, dtype=dt)
    zq = specgen.tree_target_logits(trees, V, seed=2, dtype=dt)
    rng = np.random.default_rng(B + M)
    temp = rng.uniform(0.3, 1.5, B).astype(np.float32)
    temp[::5] = 0.0                                   # some greedy trees
    n = np.full(B, M, np.int32)
    n[1::4] = np.maximum(1, M // 2)
    par, tok = trees["parent"].copy(), trees["token"].copy()
    if B >= 8:
        temp[2] = -1.0                                # sentinel temperature
        tok[3, M - 1] = V                             # token out of range
    torch_dt = torch.bfloat16 if dt == "bf16" else torch.float32
    print(f"\n[tree sample B={B} M={M} V={V} {dt}]", flush=True)
    g = gpu_sample(par, tok, n, zq, zt, temp, torch_dt, seed=9, offset=1)
    o = oracle.tree_verify_sample(par, tok, n, zq, zt, temp, seed=9, offset=1)
    f = check_sample(g, o, temp)
    if B >= 8:
        assert g["length"][2] == -1 and g["length"][3] == -1
    print(f"  flagged {f}/{B}, lengths {g['length'].tolist()[:12]}", flush=True)
    assert (o["length"] >= 1).any()


def test_sample_repeated_calls():
    """Several calls on one context (the parts' exchange slots keep the previous
    call's words), with different inputs, offsets and batch contents."""
    B, M, V = 300, 10, 2048
    ctx = sv.spec_tree_verify_init(B, M, V, torch.bfloat16)
    print(f"\n[tree sample repeated B={B} M={M} V={V}]", flush=True)
    for call in range(3):
        trees = specgen.draft_trees(B, M, V, seed=50 + call)
        zt = specgen.tree_target_logits(trees, V, seed=60 + call, dtype="bf16")
        zq = specgen.tree_target_logits(trees, V, seed=70 + call, dtype="bf16")
        rng = np.random.default_rng(call)
        temp = rng.uniform(0.3, 1.5, B).astype(np.float32)
        temp[rng.random(B) < 0.2] = 0.0
        n = rng.integers(1, M + 1, B).astype(np.int32)
        g = gpu_sample(trees["parent"], trees["token"], n, zq, zt, temp, torch.bfloat16,
                       seed=11, offset=call, ctx=ctx)
        o = oracle.tree_verify_sample(trees["parent"], trees["token"], n, zq, zt, temp, seed=11,
                                      offset=call)
        f = check_sample(g, o, temp)
        print(f"  call {call}: flagged {f}/{B}, mean length {g['length'].mean():.2f}", flush=True)
    sv.spec_tree_verify_destroy(ctx)


def test_sample_full_workload_sampled():
    """B = 256 trees of 16 nodes over V = 152064 bf16, temperatures drawn as in
    the B=256 workload (U[0.3, 1.5], 10 % greedy); the oracle on 12 trees
    (Philox indices kept)."""
    B, M, V = 256, 16, 152064
    trees = specgen.draft_trees(B, M, V, seed=31)
    zt = specgen.tree_target_logits(trees, V, seed=5)
    zq = specgen.tree_target_logits(trees, V, seed=6)
    rng = np.random.default_rng(7)
    temp = rng.uniform(0.3, 1.5, B).astype(np.float32)   # the workload's temperature recipe
    temp[rng.random(B) < 0.1] = 0.0
    n = np.full(B, M, np.int32)
    print(f"\n[tree sample B={B} M={M} V={V}]", flush=True)
    g = gpu_sample(trees["parent"], trees["token"], n, zq, zt, temp, torch.bfloat16, seed=2, offset=4)
    rows = np.array([0, 1, 17, 64, 100, 128, 150, 199, 200, 230, 254, 255])
    o = oracle.tree_verify_sample(trees["parent"][rows], trees["token"][rows], n[rows], zq[rows],
                                  zt[rows], temp[rows], seed=2, offset=4, seq_ids=rows)
    f = check_sample(g, o, temp[rows], rows=rows)
    print(f"  flagged {f}/{rows.size}; GPU mean length {g['length'].mean():.2f}", flush=True)
    assert (g["length"] >= 0).all()


def _sample_inputs(B, M, V, seed):
    trees = specgen.draft_trees(B, M, V, seed=seed)
    zt = specgen.tree_target_logits(trees, V, seed=seed + 1, dtype="bf16")
    zq = specgen.tree_target_logits(trees, V, seed=seed + 2, dtype="bf16")
    rng = np.random.default_rng(seed)
    temp = rng.uniform(0.3, 1.5, B).astype(np.float32)
    temp[rng.random(B) < 0.15] = 0.0
    n = np.full(B, M, np.int32)
    return trees, zq, zt, temp, n


def test_sample_give_up_is_reported_and_counted():
    """A spin limit of zero polls, set from the host, makes parts give up
    waiting for partners that are merely late; every kernel still exits. Part 0
    reports such trees with length -2 and counts them; every other tree is
    still the oracle's outcome. With the default limit restored the next call
    on the same context completes every tree."""
    B, M, V = 64, 8, 2048
    trees, zq, zt, temp, n = _sample_inputs(B, M, V, 90)
    ctx = sv.spec_tree_verify_init(B, M, V, torch.bfloat16)
    before = sv.spec_tree_verify_gave_up(ctx)
    sv.spec_tree_verify_set_spin_limit(ctx, 0)
    g = gpu_sample(trees["parent"], trees["token"], n, zq, zt, temp, torch.bfloat16, seed=4,
                   offset=2, ctx=ctx)
    gave = sv.spec_tree_verify_gave_up(ctx) - before
    lost = np.nonzero(g["length"] == -2)[0]
    print(f"\n[tree give-up] spin limit 0: {lost.size}/{B} trees given up, counted {gave}", flush=True)
    assert gave == lost.size
    assert np.all(g["extra"][lost] == -1) and np.all(g["path"][lost] == -1)
    o = oracle.tree_verify_sample(trees["parent"], trees["token"], n, zq, zt, temp, seed=4, offset=2)
    kept = np.nonzero(g["length"] != -2)[0]
    check_sample(g, {k: v[kept] for k, v in o.items()}, temp[kept], rows=kept)
    sv.spec_tree_verify_set_spin_limit(ctx, 1 << 20)
    g = gpu_sample(trees["parent"], trees["token"], n, zq, zt, temp, torch.bfloat16, seed=4,
                   offset=2, ctx=ctx)
    assert (g["length"] >= 0).all()
    assert sv.spec_tree_verify_gave_up(ctx) - before == gave
    check_sample(g, o, temp)
    sv.spec_tree_verify_destroy(ctx)


def test_sample_graph_replays_match_eager():
    """The sampled call captured into a HIP graph: replays on two input sets
    copied into the captured buffers, with eager work in between, equal eager
    calls bit for bit (each launch tags its exchanges with a number the kernel
    advances itself, so replays never read a previous replay's shares)."""
    B, M, V = 48, 10, 4096
    sets = []
    for sd in (70, 71):
        trees, zq, zt, temp, n = _sample_inputs(B, M, V, sd)
        sets.append(dict(parent=dev(trees["parent"]), token=dev(trees["token"]), n=dev(n),
                         zq=to_dev_logits(zq, torch.bfloat16), zt=to_dev_logits(zt, torch.bfloat16),
                         temp=dev(temp)))
    static = {k: v.clone() for k, v in sets[0].items()}
    s = torch.cuda.Stream()
    ctx = sv.spec_tree_verify_init(B, M, V, torch.bfloat16, stream=s)
    L = torch.empty(B, dtype=torch.int32, device="cuda")
    path = torch.empty((B, M), dtype=torch.int32, device="cuda")
    extra = torch.empty(B, dtype=torch.int32, device="cuda")

    def call():
        sv.spec_tree_verify_sample(ctx, static["parent"], static["token"], static["n"], static["zq"],
                                   static["zt"], static["temp"], 6, 3, L, path, extra)

    eager = []
    for st_ in sets:
        for k in static:
            static[k].copy_(st_[k])
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            call()
        s.synchronize()
        eager.append((L.clone(), path.clone(), extra.clone()))
    assert not torch.equal(eager[0][2], eager[1][2])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for r, j in enumerate([1, 0, 1, 0]):
        for k in static:
            static[k].copy_(sets[j][k])
        L.fill_(-7)
        extra.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(L, eager[j][0]), f"replay {r}"
        assert torch.equal(path, eager[j][1]), f"replay {r}"
        assert torch.equal(extra, eager[j][2]), f"replay {r}"
        _ = (sets[j]["zt"].float().sum()).item()  # eager work between replays
    del g
    assert sv.spec_tree_verify_gave_up(ctx) == 0
    sv.spec_tree_verify_destroy(ctx)
