"""Seeded synthetic inputs for speculative-sampling verification.

This module is shared by the tests, the benchmark and the smoke check. It holds
none of the verification arithmetic: it draws logits, rounds them to the storage
dtype, draws per-sequence temperatures and samples the draft tokens the way a
draft model's sampler would (Gumbel-max on the draft logits divided by T, or the
draft argmax when T == 0). No log-sum-exp, accept test or residual appears here.

Every array is a pure function of (recipe, shape, seed): each sequence b draws
from its own generator ``default_rng([seed, b])``, so any subset of sequences of
a large batch can be regenerated alone and matches the full batch bit for bit.

The five workloads (sizes and distributions as the verification pages' target
workloads are stated for this library):

==  ====  ==  =======  =====  ===========================================  ==========
#   B     g   V        dtype  logits                                       T
==  ====  ==  =======  =====  ===========================================  ==========
1   1     4   32000    fp32   draft N(0,2^2); target = draft + N(0,0.5^2)  1.0
2   8     4   32000    bf16   draft N(0,3^2); target = draft + N(0,1^2)    0.7
3   64    5   128256   bf16   Zipf (below); target = draft + N(0,0.7^2)    1.0
4   256   8   152064   bf16   draft N(0,2.5^2); target rho=0.8 correlated  U[0.3,1.5], 10% = 0
5   512   4   201088   bf16   Zipf; target = draft + N(0,1^2)              0.8
==  ====  ==  =======  =====  ===========================================  ==========

Zipf rows: logit[pi(j)] = -1.1 * ln(j + 1) + N(0, 0.3^2), pi a fresh seeded
permutation of the vocabulary for every (sequence, position) base row.
rho = 0.8 correlation: target = 0.8 * draft + 0.6 * N(0, 2.5^2), which keeps the
marginal variance. Base rows are drawn for positions 0..gamma in float64; the
draft uses positions 0..gamma-1, the target all gamma+1 (position gamma is the
bonus row). Values are rounded float64 -> float32 -> bf16 (round to nearest
even); the target is built from the float64 draft before rounding.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

__all__ = ["Recipe", "CONFIGS", "config", "generate", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "gumbel_max_tokens", "lowrank_head_inputs", "draft_trees",
           "tree_target_logits"]


@dataclasses.dataclass(frozen=True)
class Recipe:
    """How one workload's inputs are drawn."""
    name: str
    batch: int
    gamma: int
    vocab: int
    dtype: str                 # "f32" or "bf16"
    kind: str                  # "gauss" | "corr" | "zipf"
    draft_sigma: float         # std of draft logits (gauss / corr); unused for zipf
    noise_sigma: float         # std of the target's added noise (corr: of the fresh part)
    temperature: float | None  # fixed T, or None for the U[0.3, 1.5] + 10 % greedy mix
    seed: int                  # data seed

    def replace(self, **kw) -> "Recipe":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    1: Recipe("B1_g4_V32000_f32_gauss", 1, 4, 32000, "f32", "gauss", 2.0, 0.5, 1.0, 1),
    2: Recipe("B8_g4_V32000_bf16_gauss", 8, 4, 32000, "bf16", "gauss", 3.0, 1.0, 0.7, 2),
    3: Recipe("B64_g5_V128256_bf16_zipf", 64, 5, 128256, "bf16", "zipf", 0.0, 0.7, 1.0, 3),
    4: Recipe("B256_g8_V152064_bf16_corr", 256, 8, 152064, "bf16", "corr", 2.5, 2.5, None, 4),
    5: Recipe("B512_g4_V201088_bf16_zipf", 512, 4, 201088, "bf16", "zipf", 0.0, 1.0, 0.8, 5),
}


def config(n: int) -> Recipe:
    return CONFIGS[n]


# ------------------------------------------------------------------ rounding --

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16, nearest-even, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return x32 if dtype == "f32" else f32_to_bf16_bits(x32)


def _as_f64(stored: np.ndarray) -> np.ndarray:
    if stored.dtype == np.uint16:
        return bf16_bits_to_f32(stored).astype(np.float64)
    return stored.astype(np.float64)


# ----------------------------------------------------------------- sampling --

def gumbel_max_tokens(z_rows: np.ndarray, temperature: float,
                      rng: np.random.Generator) -> np.ndarray:
    """A draft model's sampler: one token per row of stored draft logits.

    T > 0: argmax_v (z_v / T + g_v) with g_v i.i.d. standard Gumbel, which draws
    exactly from softmax(z / T). T == 0: argmax_v z_v (first index on ties)."""
    z = _as_f64(z_rows)
    if temperature == 0.0:
        return np.argmax(z, axis=-1).astype(np.int32)
    g = rng.gumbel(size=z.shape)
    return np.argmax(z / float(temperature) + g, axis=-1).astype(np.int32)


def _base_rows(recipe: Recipe, rng: np.random.Generator, n_rows: int) -> np.ndarray:
    V = recipe.vocab
    if recipe.kind == "zipf":
        ranks = -1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))
        out = np.empty((n_rows, V), dtype=np.float64)
        for r in range(n_rows):
            perm = rng.permutation(V)
            out[r, perm] = ranks + rng.normal(0.0, 0.3, size=V)
        return out
    return rng.normal(0.0, recipe.draft_sigma, size=(n_rows, V))


def _target_rows(recipe: Recipe, base: np.ndarray, rng: np.random.Generator) -> np.ndarray:
    noise = rng.normal(0.0, recipe.noise_sigma, size=base.shape)
    if recipe.kind == "corr":
        return 0.8 * base + 0.6 * noise
    return base + noise


def temperatures(recipe: Recipe) -> np.ndarray:
    """Per-sequence temperature [B] float32."""
    B = recipe.batch
    if recipe.temperature is not None:
        return np.full(B, recipe.temperature, dtype=np.float32)
    rng = np.random.default_rng([recipe.seed, 1 << 30])
    t = rng.uniform(0.3, 1.5, size=B).astype(np.float32)
    n_greedy = int(round(0.1 * B))
    t[rng.choice(B, size=n_greedy, replace=False)] = 0.0
    return t


def _one_sequence(recipe: Recipe, b: int, temp: float):
    rng = np.random.default_rng([recipe.seed, b])
    G = recipe.gamma
    base = _base_rows(recipe, rng, G + 1)
    target = _store(_target_rows(recipe, base, rng), recipe.dtype)
    draft = _store(base[:G], recipe.dtype)
    tokens = gumbel_max_tokens(draft, temp, rng) if G > 0 else np.zeros(0, np.int32)
    return draft, target, tokens


def generate(recipe: Recipe, seq_ids=None, threads: int | None = None) -> dict:
    """Inputs of a workload: logits_draft [n, G, V], logits_target [n, G+1, V]
    (float32, or bf16 bit patterns as uint16), draft_tokens [n, G] int32,
    temperature [n] float32, for the sequences ``seq_ids`` (default: all B)."""
    B, G, V = recipe.batch, recipe.gamma, recipe.vocab
    ids = np.arange(B) if seq_ids is None else np.asarray(seq_ids, dtype=np.int64)
    temps_all = temperatures(recipe)
    n = len(ids)
    st = np.float32 if recipe.dtype == "f32" else np.uint16
    draft = np.empty((n, G, V), dtype=st)
    target = np.empty((n, G + 1, V), dtype=st)
    tokens = np.empty((n, G), dtype=np.int32)

    def work(k):
        d, t, tok = _one_sequence(recipe, int(ids[k]), float(temps_all[ids[k]]))
        draft[k] = d
        target[k] = t
        tokens[k] = tok

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if n == 1 or threads <= 1:
        for k in range(n):
            work(k)
    else:
        with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, range(n)))
    return dict(logits_draft=draft, logits_target=target, draft_tokens=tokens,
                temperature=temps_all[ids].copy(), seq_ids=ids.astype(np.int64),
                recipe=recipe)


def lowrank_head_inputs(rows: int, hidden: int, rank: int, vocab: int, seed: int = 0,
                        logit_std: float = 2.5, greedy_fraction: float = 0.1):
    """Synthetic inputs of a low-rank draft LM head z = W_up (W_down h), as
    bfloat16 bit patterns: h [rows, hidden] ~ N(0, 1), W_down [rank, hidden]
    ~ N(0, 1/hidden) (so W_down h ~ N(0, 1)), W_up [vocab, rank] ~ N(0,
    logit_std^2 / rank) (so the logits have standard deviation about
    logit_std, that of the B=256 workload's draft rows); temperatures
    U[0.3, 1.5] per row with round(greedy_fraction * rows) rows at 0. Random
    weights stand in for a trained head; no dataset is involved."""
    rng = np.random.default_rng([seed, 7919])
    h = rng.standard_normal((rows, hidden), dtype=np.float32)
    w_down = rng.standard_normal((rank, hidden), dtype=np.float32) * np.float32(1.0 / np.sqrt(hidden))
    w_up = np.empty((vocab, rank), dtype=np.uint16)
    scale = np.float32(logit_std / np.sqrt(rank))
    step = 16384
    for v0 in range(0, vocab, step):   # in slices, to bound the float32 temporaries
        v1 = min(vocab, v0 + step)
        w_up[v0:v1] = f32_to_bf16_bits(rng.standard_normal((v1 - v0, rank), dtype=np.float32) * scale)
    temp = rng.uniform(0.3, 1.5, size=rows).astype(np.float32)
    n_greedy = int(round(greedy_fraction * rows))
    if n_greedy:
        temp[rng.choice(rows, size=n_greedy, replace=False)] = 0.0
    return dict(h=f32_to_bf16_bits(h), w_down=f32_to_bf16_bits(w_down), w_up=w_up,
                temperature=temp)


def draft_trees(batch: int, nodes: int, vocab: int, seed: int = 0, max_children: int = 3,
                chain_bias: float = 0.6):
    """Seeded draft trees in topological order, as a tree-drafting proposer
    would emit them: node 0 is the root; node i >= 1 hangs under node i - 1
    with probability chain_bias (when it has room), else under a uniformly
    chosen earlier node with fewer than max_children children. Each node's
    children split a Dirichlet(1, ..., 1) draft mass with one extra "other"
    share, so logq (the draft log-probability of a node's token) is <= 0 and
    the children's probabilities sum to less than one. Tokens are uniform in
    [0, vocab). Returns parent [B, M] int32 (parent[:, 0] = -1), token [B, M]
    int32 (token[:, 0] = 0), logq [B, M] float32 (logq[:, 0] = 0)."""
    parent = np.full((batch, nodes), -1, np.int32)
    token = np.zeros((batch, nodes), np.int32)
    logq = np.zeros((batch, nodes), np.float32)
    for b in range(batch):
        rng = np.random.default_rng([seed, b, 104729])
        kids = [[] for _ in range(nodes)]
        for i in range(1, nodes):
            if len(kids[i - 1]) < max_children and rng.random() < chain_bias:
                p = i - 1
            else:
                free = [j for j in range(i) if len(kids[j]) < max_children]
                p = int(free[rng.integers(len(free))])
            parent[b, i] = p
            kids[p].append(i)
            token[b, i] = rng.integers(vocab)
        for j in range(nodes):
            if kids[j]:
                w = rng.dirichlet(np.ones(len(kids[j]) + 1))
                for k, c in enumerate(kids[j]):
                    logq[b, c] = np.float32(np.log(w[k]))
    return dict(parent=parent, token=token, logq=logq)


def tree_target_logits(trees: dict, vocab: int, seed: int = 0, follow: float = 0.7,
                       std: float = 2.5, dtype: str = "bf16") -> np.ndarray:
    """Target logits [B, M, V] for draft trees: N(0, std^2) per entry; for each
    node with children, with probability `follow` the token of its first
    child gets +4 std added, so that greedy paths often continue into the
    tree (the input construction adds a bump; it computes no argmax)."""
    parent, token = trees["parent"], trees["token"]
    B, M = parent.shape
    out = np.empty((B, M, vocab), np.uint16 if dtype == "bf16" else np.float32)
    for b in range(B):
        rng = np.random.default_rng([seed, b, 15485863])
        z = rng.standard_normal((M, vocab), dtype=np.float32) * np.float32(std)
        first = {}
        for i in range(1, M):
            first.setdefault(int(parent[b, i]), i)
        for x, c in first.items():
            if rng.random() < follow:
                z[x, token[b, c]] += np.float32(4 * std)
        out[b] = f32_to_bf16_bits(z) if dtype == "bf16" else z
    return out
