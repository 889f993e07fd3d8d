"""Pins of the draft-tree oracle (pruning and greedy tree verification).

The SpecLA summary (Methodology section 3) prunes low-probability paths of a
draft tree by their cumulative log-probability before verification; tree
drafts are verified along the path the target agrees with (for T = 0, the
exact-match rule of token-tree speculative decoding; it reduces to the
verifier's greedy rule on a chain). Pins:
* path scores against brute force (each node's root path collected and summed
  root first, independently of the oracle's recursion);
* the kept set against a brute-force sort of the scores, and its closure
  under ancestors; the remapped parents;
* greedy tree verification on chains against the verification oracle's greedy
  outcome on the same logits; on trees, the properties that define the walk
  (every accepted token is the target's argmax after its predecessor, the walk
  takes the lowest-index matching child, the extra token is the argmax after
  the last node and no child of it matches);
* sentinels for malformed trees.
"""
import numpy as np

import oracle
import specgen


def path_of(parent, i):
    path = []
    while i > 0:
        path.append(i)
        i = parent[i]
    return path[::-1]


def test_path_scores_and_kept_set_by_brute_force():
    trees = specgen.draft_trees(6, 24, 1000, seed=3)
    for tau, K in ((np.log(1e-3), 10), (-np.inf, 24), (np.log(0.2), 5), (0.0, 3)):
        out = oracle.tree_prune(trees["parent"], trees["logq"], tau, K)
        for b in range(6):
            par, lq = trees["parent"][b], trees["logq"][b]
            score = np.zeros(24)
            for i in range(1, 24):
                s = 0.0
                for j in path_of(par, i):
                    s += float(lq[j])
                score[i] = s
            assert np.array_equal(out["cum"][b], score)
            order = sorted(range(24), key=lambda i: (-score[i], i))
            keep = sorted(i for i in order[:K] if score[i] >= tau)
            assert out["count"][b] == len(keep)
            assert [i for i in range(24) if out["new_index"][b, i] >= 0] == keep
            assert 0 in keep
            for new, old in enumerate(keep):
                assert out["new_index"][b, old] == new
                if old:
                    assert par[old] in keep                       # closed under ancestors
                    assert out["new_parent"][b, new] == keep.index(par[old])
            assert (out["new_parent"][b, len(keep):] == -1).all()


def test_prune_sentinels():
    trees = specgen.draft_trees(3, 8, 100, seed=1)
    par, lq = trees["parent"].copy(), trees["logq"].copy()
    par[0, 5] = 6               # not topological
    lq[1, 3] = 0.5              # not a log-probability
    lq[2, 4] = np.nan
    out = oracle.tree_prune(par, lq, -np.inf, 8)
    assert out["count"].tolist() == [-1, -1, -1]
    assert (out["new_index"] == -1).all() and np.isnan(out["cum"]).all()


def test_greedy_tree_on_chains_matches_the_verifier():
    """A chain of gamma drafts is the tree parent = i - 1; with T = 0 its
    greedy verification must give the verification oracle's outcome."""
    rng = np.random.default_rng(5)
    B, G, V = 12, 5, 64
    zp = np.round(rng.normal(0, 2, size=(B, G + 1, V))).astype(np.float32)  # ties too
    amax = np.argmax(zp, axis=-1)
    drafts = np.where(rng.random((B, G)) < 0.75, amax[:, :G], rng.integers(0, V, (B, G))).astype(np.int32)
    ver = oracle.verify(np.zeros((B, G, V), np.float32), zp, drafts, np.zeros(B, np.float32))
    parent = np.tile(np.arange(-1, G, dtype=np.int32), (B, 1))
    token = np.concatenate([np.zeros((B, 1), np.int32), drafts], axis=1)
    out = oracle.tree_verify_greedy(parent, token, np.full(B, G + 1), zp)
    assert np.array_equal(out["length"], ver["accept_len"])
    for b in range(B):
        k = ver["accept_len"][b]
        assert out["path"][b, :k].tolist() == list(range(1, k + 1))
        assert out["extra"][b] == ver["tokens"][b, k]


def test_greedy_tree_walk_properties():
    trees = specgen.draft_trees(16, 20, 50, seed=9, max_children=4)
    target = specgen.tree_target_logits(trees, 50, seed=2, dtype="f32")
    n = np.full(16, 20, np.int32)
    n[3] = 7                                  # a tree using only its first 7 nodes
    out = oracle.tree_verify_greedy(trees["parent"], trees["token"], n, target)
    deep = 0
    for b in range(16):
        par, tok = trees["parent"][b], trees["token"][b]
        L = out["length"][b]
        assert L >= 0
        x = 0
        for step in range(L):
            a = int(np.argmax(target[b, x]))
            kids = [j for j in range(1, n[b]) if par[j] == x and tok[j] == a]
            assert out["path"][b, step] == min(kids)
            x = out["path"][b, step]
        a = int(np.argmax(target[b, x]))
        assert out["extra"][b] == a
        assert not any(par[j] == x and tok[j] == a for j in range(1, n[b]))
        assert (out["path"][b, L:] == -1).all()
        deep += L >= 2
    assert deep >= 4                          # the inputs do exercise the walk


def test_greedy_tree_sentinels():
    trees = specgen.draft_trees(4, 6, 30, seed=4)
    target = specgen.tree_target_logits(trees, 30, seed=1, dtype="f32")
    tok = trees["token"].copy()
    tok[1, 2] = 30                            # token outside the vocabulary
    par = trees["parent"].copy()
    par[2, 4] = 4                             # own parent
    n = np.array([6, 6, 6, 0], np.int32)      # tree 3 has no nodes
    out = oracle.tree_verify_greedy(par, tok, n, target)
    assert out["length"].tolist()[1:] == [-1, -1, -1]
    assert out["extra"].tolist()[1:] == [-1, -1, -1]
    assert out["length"][0] >= 0


def test_prune_ties_go_to_the_lower_index():
    # root with four children of equal probability 0.2; budget 3 keeps the root
    # and the two lowest-index children
    parent = np.array([[-1, 0, 0, 0, 0]], np.int32)
    logq = np.array([[0, np.log(0.2), np.log(0.2), np.log(0.2), np.log(0.2)]], np.float32)
    out = oracle.tree_prune(parent, logq, -np.inf, 3)
    assert out["new_index"][0].tolist() == [0, 1, 2, -1, -1]


def test_greedy_tree_duplicate_siblings_take_the_lower_index():
    # two children of the root carry the same token; only the second has a
    # matching grandchild: the walk still takes the first and stops there
    V = 8
    parent = np.array([[-1, 0, 0, 2]], np.int32)
    token = np.array([[0, 5, 5, 3]], np.int32)
    target = np.zeros((1, 4, V), np.float32)
    target[0, 0, 5] = 1.0          # after the root: 5
    target[0, 1, 6] = 1.0          # after node 1: 6 (no child)
    target[0, 2, 3] = 1.0          # after node 2: 3 (node 3 would match)
    out = oracle.tree_verify_greedy(parent, token, np.array([4]), target)
    assert out["length"][0] == 1 and out["path"][0, 0] == 1 and out["extra"][0] == 6
