"""CPU oracle for batched speculative-sampling verification -- TEST INFRASTRUCTURE ONLY.

This package wraps ``spec_oracle.c`` (plain single-threaded C in IEEE double)
with ctypes. Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import it; the HIP library and its Python binding never do.

What the oracle computes, and the readings it takes where the pages are silent,
is stated at the top of ``spec_oracle.c``. Parity status of each function:

* ``philox4x32_10`` / ``philox_words`` / ``uniform24`` -- pinned against the
  header-only Philox4x32-10 engine that ships with PyTorch's C++ headers
  (an independent library implementation of the SC'11 definition).
* ``row_lse`` -- pinned against ``scipy.special.logsumexp`` and closed forms.
* ``row_argmax`` -- pinned against ``numpy.argmax`` (first index on ties).
* ``inverse_cdf`` -- pinned by exhaustive sweeps of the uniform grid.
* ``verify`` / ``verify_sequence`` -- pinned by the closed-form acceptance
  probability sum_v min(p_v, q_v), the output-marginal gate (chi-square and KS
  at 0.01 over 10,000 draws) and the degenerate cases (gamma = 0, p = q,
  disjoint support, greedy).
* ``accept_logprobs`` -- pinned by agreement with ``verify`` on the gathered
  pairs and by the closed-form acceptance probability min(1, p/q).
* ``gamma_sample`` / ``beta_sample`` (``bandit_oracle.c``) -- pinned by
  Kolmogorov-Smirnov tests against ``scipy.stats.gamma`` / ``scipy.stats.beta``.
* ``lowrank_head`` -- pinned against numpy's float64 matrix products, the
  bfloat16 rounding against PyTorch's float32 -> bfloat16 conversion and
  hand-made ties, the normaliser against ``scipy.special.logsumexp``, and the
  rank-one closed form.
* ``tree_prune`` / ``tree_verify_greedy`` -- pinned by brute force over the
  paths of small trees (path scores summed root to leaf, selection by sorting)
  and, for chains, by the verification oracle's greedy outcome.
* ``bandit_step`` -- UCB1 pinned by its opening round robin and by the regret
  bound of Auer, Cesa-Bianchi and Fischer (2002, Theorem 1); Thompson sampling by
  logarithmic regret growth; both by the output-marginal gate with the bandit
  choosing the draft distribution every step (the pages' Theorem 1).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "spec_oracle.c"), os.path.join(_HERE, "bandit_oracle.c")]
# ORACLE_LIB selects another build of the same sources (the sanitizer test's).
LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1


def build(out: str | None = None, extra_flags=()) -> str:
    """Compile the oracle with gcc: -O2, no fast-math, no FP contraction
    (extra_flags: e.g. the sanitizers of the sanitizer test)."""
    out = out or LIB_PATH
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", *extra_flags, "-o", tmp, *_SRCS, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32, u64, f32, f64 = ctypes.c_int, ctypes.c_uint64, ctypes.c_float, ctypes.c_double
    lib.oracle_philox4x32_10.argtypes = [P, P, P]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_philox_words.argtypes = [u64, u64, ctypes.c_int64, i32, P]
    lib.oracle_philox_words.restype = None
    lib.oracle_uniform24.argtypes = [ctypes.c_uint32]
    lib.oracle_uniform24.restype = f64
    lib.oracle_row_lse.argtypes = [P, i32, ctypes.c_size_t, i32, f32]
    lib.oracle_row_lse.restype = f64
    lib.oracle_row_argmax.argtypes = [P, i32, ctypes.c_size_t, i32]
    lib.oracle_row_argmax.restype = i32
    lib.oracle_inverse_cdf.argtypes = [P, i32, f64, P]
    lib.oracle_inverse_cdf.restype = i32
    lib.oracle_inverse_cdf_alt.argtypes = [P, i32, f64, P, P]
    lib.oracle_inverse_cdf_alt.restype = i32
    lib.oracle_draw_at.argtypes = [i32, i32, P, ctypes.c_size_t, P, ctypes.c_size_t, i32, f32,
                                   f64, P, P, P]
    lib.oracle_draw_at.restype = None
    lib.oracle_verify_sequence.argtypes = [i32, i32, i32, P, ctypes.c_size_t, P,
                                           ctypes.c_size_t, P, f32, P, P, P, P, P, P, P, P]
    lib.oracle_verify_sequence.restype = None
    lib.oracle_verify.argtypes = [i32, i32, i32, i32, P, P, P, P, u64, u64, P,
                                  P, P, P, P, P, P]
    lib.oracle_verify.restype = None
    lib.oracle_accept_logprobs.argtypes = [i32, i32, P, u64, u64, P, P, P]
    lib.oracle_accept_logprobs.restype = None
    lib.oracle_gather_logprobs.argtypes = [i32, i32, i32, i32, P, P, P, P, P]
    lib.oracle_gather_logprobs.restype = None
    lib.oracle_outcomes.argtypes = [i32, i32, i32, i32, P, P, P, P, i32, P, P, P, P, P, P]
    lib.oracle_outcomes.restype = None
    lib.oracle_outcome_fanout.argtypes = [i32, i32, i32, P, P, i32, P, P]
    lib.oracle_outcome_fanout.restype = None
    lib.oracle_lowrank_head.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.oracle_lowrank_head.restype = None
    lib.oracle_tree_prune.argtypes = [i32, i32, P, P, f64, i32, P, P, P, P]
    lib.oracle_tree_prune.restype = None
    lib.oracle_tree_verify_greedy.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P]
    lib.oracle_tree_verify_greedy.restype = None
    lib.oracle_tree_verify_sample.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, u64, u64,
                                              P, P, P, P, P, P]
    lib.oracle_tree_verify_sample.restype = None
    lib.oracle_gamma_mt.argtypes = [f64, u64, u64, i32, i32, i32, P]
    lib.oracle_gamma_mt.restype = f64
    lib.oracle_beta_sample.argtypes = [f64, f64, u64, u64, i32, i32, P]
    lib.oracle_beta_sample.restype = f64
    lib.oracle_ucb1_select.argtypes = [i32, P, P, P]
    lib.oracle_ucb1_select.restype = i32
    lib.oracle_thompson_select.argtypes = [i32, P, P, u64, u64, i32, P]
    lib.oracle_thompson_select.restype = i32
    lib.oracle_bandit_step.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, u64, u64, P, P]
    lib.oracle_bandit_step.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _logits(a: np.ndarray) -> tuple[np.ndarray, int]:
    """Accept float32 logits, or bf16 logits given as their uint16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {a.dtype}")


def philox4x32_10(counter, key) -> np.ndarray:
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    _load().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def philox_words(seed: int, offset: int, b: int, i: int) -> np.ndarray:
    out = np.zeros(4, dtype=np.uint32)
    _load().oracle_philox_words(seed, offset, b, i, _ptr(out))
    return out


def uniform24(word: int) -> float:
    return _load().oracle_uniform24(word)


def row_lse(z: np.ndarray, temperature: float) -> float:
    """LSE of fl32(z * fl32(1/T)) over one row, T > 0."""
    z, dt = _logits(z.reshape(-1))
    inv_t = np.float32(1.0) / np.float32(temperature)
    return _load().oracle_row_lse(_ptr(z), dt, 0, z.size, float(inv_t))


def row_argmax(z: np.ndarray) -> int:
    z, dt = _logits(z.reshape(-1))
    return _load().oracle_row_argmax(_ptr(z), dt, 0, z.size)


def inverse_cdf(r: np.ndarray, u: float) -> tuple[int, float]:
    r = np.ascontiguousarray(r, dtype=np.float64)
    m = ctypes.c_double(0.0)
    j = _load().oracle_inverse_cdf(_ptr(r), r.size, float(u), ctypes.byref(m))
    return j, m.value


def inverse_cdf_alt(r: np.ndarray, u: float) -> tuple[int, float, int]:
    """As ``inverse_cdf``, plus the token across the nearer edge of the chosen
    bin (the nearest positive-weight index on that side, -1 if none)."""
    r = np.ascontiguousarray(r, dtype=np.float64)
    m = ctypes.c_double(0.0)
    a = ctypes.c_int32(-1)
    j = _load().oracle_inverse_cdf_alt(_ptr(r), r.size, float(u), ctypes.byref(m),
                                       ctypes.byref(a))
    return j, m.value, a.value


def draw_at(draft_row, target_row, temperature: float, u: float) -> tuple[int, float, int]:
    """The extra token a sequence emits when its first rejection is at the
    position of these rows (``draft_row`` None: the bonus draw from
    ``target_row``), at uniform u: (token, log-margin, token across the nearer
    bin edge)."""
    zp, dt = _logits(np.ascontiguousarray(target_row).reshape(-1))
    if draft_row is None:
        zq, bonus = zp, 1
    else:
        zq, dq = _logits(np.ascontiguousarray(draft_row).reshape(-1))
        assert dq == dt and zq.size == zp.size
        bonus = 0
    tok = ctypes.c_int32(-1)
    m = ctypes.c_double(0.0)
    a = ctypes.c_int32(-1)
    _load().oracle_draw_at(zp.size, dt, _ptr(zq), 0, _ptr(zp), 0, bonus,
                           float(np.float32(temperature)), float(u), ctypes.byref(tok),
                           ctypes.byref(m), ctypes.byref(a))
    return tok.value, m.value, a.value


def uniform_res(seed: int, offset: int, b: int, i: int) -> float:
    """The resample uniform of position i of sequence b (Philox word 1)."""
    return uniform24(int(philox_words(seed, offset, b, i)[1]))


def verify_sequence(logits_draft, logits_target, draft_tokens, temperature, u_acc, u_res):
    """One sequence with explicit uniforms. logits_draft [G, V], logits_target [G+1, V]."""
    zp, dt = _logits(logits_target)
    G = zp.shape[0] - 1
    V = zp.shape[1]
    if G > 0:
        zq, dq = _logits(logits_draft)
        assert dq == dt and zq.shape == (G, V)
    else:
        zq = np.zeros((1, V), dtype=zp.dtype)
    tok = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(max(G, 1))
    ua = np.ascontiguousarray(u_acc, dtype=np.float64).reshape(-1)
    ur = np.ascontiguousarray(u_res, dtype=np.float64).reshape(-1)
    assert ua.size >= G and ur.size >= G + 1
    alen = ctypes.c_int32(0)
    tokens = np.zeros(G + 1, dtype=np.int32)
    lse = np.zeros(2 * G + 1, dtype=np.float64)
    am = np.zeros(max(G, 1), dtype=np.float64)
    rm = ctypes.c_double(0.0)
    ra = ctypes.c_int32(-1)
    _load().oracle_verify_sequence(G, V, dt, _ptr(zq), 0, _ptr(zp), 0, _ptr(tok),
                                   float(np.float32(temperature)), _ptr(ua), _ptr(ur),
                                   ctypes.byref(alen), _ptr(tokens), _ptr(lse), _ptr(am),
                                   ctypes.byref(rm), ctypes.byref(ra))
    return dict(accept_len=alen.value, tokens=tokens, lse=lse, acc_margin=am[:G],
                res_margin=rm.value, res_alt=ra.value)


def verify(logits_draft, logits_target, draft_tokens, temperature, seed=0, offset=0,
           seq_ids=None):
    """The batched call. logits_draft [B, G, V], logits_target [B, G+1, V] (float32 or
    bf16 bits as uint16), draft_tokens [B, G] int32, temperature [B] float32.
    ``seq_ids`` gives the global sequence index of each row (for sampled checks)."""
    zp, dt = _logits(logits_target)
    B, G1, V = zp.shape
    G = G1 - 1
    if G > 0:
        zq, dq = _logits(logits_draft)
        assert dq == dt and zq.shape == (B, G, V)
        tok = np.ascontiguousarray(draft_tokens, dtype=np.int32)
        assert tok.shape == (B, G)
    else:
        zq = np.zeros((1,), dtype=zp.dtype)
        tok = np.zeros((1,), dtype=np.int32)
    temp = np.ascontiguousarray(temperature, dtype=np.float32).reshape(B)
    ids = None if seq_ids is None else np.ascontiguousarray(seq_ids, dtype=np.int64)
    if ids is not None:
        assert ids.shape == (B,)
    alen = np.zeros(B, dtype=np.int32)
    tokens = np.zeros((B, G + 1), dtype=np.int32)
    lse = np.zeros((B, 2 * G + 1), dtype=np.float64)
    am = np.zeros((B, max(G, 1)), dtype=np.float64)
    rm = np.zeros(B, dtype=np.float64)
    ra = np.zeros(B, dtype=np.int32)
    _load().oracle_verify(B, G, V, dt, _ptr(zq), _ptr(zp), _ptr(tok), _ptr(temp),
                          seed, offset, _ptr(ids), _ptr(alen), _ptr(tokens), _ptr(lse),
                          _ptr(am), _ptr(rm), _ptr(ra))
    return dict(accept_len=alen, tokens=tokens, lse=lse, acc_margin=am[:, :G],
                res_margin=rm, res_alt=ra)


def accept_logprobs(logprobs, seed=0, offset=0, seq_ids=None):
    """Scalar-only mode: logprobs [B, G, 2] float32 ([...,0] = log q, [...,1] = log p)."""
    lp = np.ascontiguousarray(logprobs, dtype=np.float32)
    B, G, two = lp.shape
    assert two == 2
    ids = None if seq_ids is None else np.ascontiguousarray(seq_ids, dtype=np.int64)
    alen = np.zeros(B, dtype=np.int32)
    am = np.zeros((B, max(G, 1)), dtype=np.float64)
    _load().oracle_accept_logprobs(B, G, _ptr(lp), seed, offset, _ptr(ids), _ptr(alen),
                                   _ptr(am))
    return dict(accept_len=alen, acc_margin=am[:, :G])


def gather_logprobs(logits_draft, logits_target, draft_tokens, temperature):
    """[B, G, 2] float64 pairs (log q, log p) of the draft tokens; NaN where undefined."""
    zp, dt = _logits(logits_target)
    B, G1, V = zp.shape
    G = G1 - 1
    zq, dq = _logits(logits_draft)
    assert dq == dt and zq.shape == (B, G, V)
    tok = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    temp = np.ascontiguousarray(temperature, dtype=np.float32).reshape(B)
    out = np.zeros((B, G, 2), dtype=np.float64)
    _load().oracle_gather_logprobs(B, G, V, dt, _ptr(zq), _ptr(zp), _ptr(tok), _ptr(temp),
                                   _ptr(out))
    return out


def outcomes(logits_draft, logits_target, draft_tokens, temperature, F: int,
             with_dist: bool = False):
    """Distribution of each sequence's verification outcome given its drafts:
    per length i in [0, G] the F most likely extra tokens and their
    probabilities, P(k = i | drafts) and the residual mass S_i. With
    ``with_dist`` also the whole distribution and the (p + q) / S magnitudes
    ([B, G+1, V] float64 each)."""
    zp, dt = _logits(logits_target)
    B, G1, V = zp.shape
    G = G1 - 1
    if G > 0:
        zq, dq = _logits(logits_draft)
        assert dq == dt and zq.shape == (B, G, V)
        tok = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    else:
        zq = np.zeros((1,), dtype=zp.dtype)
        tok = np.zeros((1,), dtype=np.int32)
    temp = np.ascontiguousarray(temperature, dtype=np.float32).reshape(B)
    out_tok = np.zeros((B, G + 1, F), np.int32)
    out_prob = np.zeros((B, G + 1, F), np.float64)
    pk = np.zeros((B, G + 1), np.float64)
    mass = np.zeros((B, G + 1), np.float64)
    dist = np.zeros((B, G + 1, V), np.float64) if with_dist else None
    scale = np.zeros((B, G + 1, V), np.float64) if with_dist else None
    _load().oracle_outcomes(B, G, V, dt, _ptr(zq), _ptr(zp), _ptr(tok), _ptr(temp), F,
                            _ptr(out_tok), _ptr(out_prob), _ptr(pk), _ptr(mass), _ptr(dist),
                            _ptr(scale))
    out = dict(tokens=out_tok, probs=out_prob, pk=pk, mass=mass)
    if with_dist:
        out.update(dist=dist, scale=scale)
    return out


def outcome_fanout(pk, probs, budget: int):
    """Speculation-cache entries per length for a budget of `budget` entries
    per sequence (Saguaro's fan-out over likely lengths): pk [B, L] and probs
    [B, L, F] as float32 values. Returns (n [B, L] int32, hit [B] float64)."""
    pk = np.ascontiguousarray(pk, dtype=np.float32)
    probs = np.ascontiguousarray(probs, dtype=np.float32)
    B, L = pk.shape
    F = probs.shape[2]
    assert probs.shape == (B, L, F)
    n = np.zeros((B, L), np.int32)
    hit = np.zeros((B,), np.float64)
    _load().oracle_outcome_fanout(B, L, F, _ptr(pk), _ptr(probs), int(budget), _ptr(n), _ptr(hit))
    return n, hit


def lowrank_head(h, w_down, w_up, temperature, rows=None):
    """z = W_up (W_down h) with bfloat16 inputs (uint16 bit patterns), the
    rank-r activation and the logits rounded to bfloat16, and the logits' row
    log-normaliser at the row's temperature. h [N, d], w_down [r, d],
    w_up [V, r], temperature [N]; ``rows`` restricts the work to some rows."""
    h = np.ascontiguousarray(h, np.uint16)
    w_down = np.ascontiguousarray(w_down, np.uint16)
    w_up = np.ascontiguousarray(w_up, np.uint16)
    N, d = h.shape
    r, d2 = w_down.shape
    V, r2 = w_up.shape
    assert d2 == d and r2 == r
    temp = np.ascontiguousarray(temperature, np.float32).reshape(N)
    idx = None if rows is None else np.ascontiguousarray(rows, np.int32)
    assert idx is None or (idx.size and idx.min() >= 0 and idx.max() < N), "rows outside [0, N)"
    n = N if idx is None else idx.size
    out = dict(u_exact=np.zeros((n, r)), u=np.zeros((n, r), np.uint16), u_abs=np.zeros((n, r)),
               z_exact=np.zeros((n, V)), z=np.zeros((n, V), np.uint16), z_abs=np.zeros((n, V)),
               lse=np.zeros(n))
    _load().oracle_lowrank_head(n, d, r, V, _ptr(h), _ptr(w_down), _ptr(w_up), _ptr(temp),
                                _ptr(idx), _ptr(out["u_exact"]), _ptr(out["u"]), _ptr(out["u_abs"]),
                                _ptr(out["z_exact"]), _ptr(out["z"]), _ptr(out["z_abs"]),
                                _ptr(out["lse"]))
    return out


def tree_prune(parent, logq, tau: float, budget: int):
    """Cumulative path log-probabilities of draft trees and their pruning by a
    threshold and a node budget. parent [B, M] int32 (parent[:, 0] = -1),
    logq [B, M] float32 (logq[:, 0] ignored)."""
    par = np.ascontiguousarray(parent, np.int32)
    lq = np.ascontiguousarray(logq, np.float32)
    B, M = par.shape
    out = dict(cum=np.zeros((B, M)), new_index=np.zeros((B, M), np.int32),
               new_parent=np.zeros((B, M), np.int32), count=np.zeros(B, np.int32))
    _load().oracle_tree_prune(B, M, _ptr(par), _ptr(lq), float(tau), int(budget),
                              _ptr(out["cum"]), _ptr(out["new_index"]), _ptr(out["new_parent"]),
                              _ptr(out["count"]))
    return out


def tree_verify_greedy(parent, token, n_nodes, target):
    """Greedy verification of draft trees: parent, token [B, M] int32,
    n_nodes [B], target logits [B, M, V] (float32 or bf16 bits)."""
    zt, dt = _logits(target)
    B, M, V = zt.shape
    par = np.ascontiguousarray(parent, np.int32)
    tok = np.ascontiguousarray(token, np.int32)
    nn = np.ascontiguousarray(n_nodes, np.int32).reshape(B)
    out = dict(length=np.zeros(B, np.int32), path=np.zeros((B, M), np.int32),
               extra=np.zeros(B, np.int32))
    _load().oracle_tree_verify_greedy(B, M, V, dt, _ptr(par), _ptr(tok), _ptr(nn), _ptr(zt),
                                      _ptr(out["length"]), _ptr(out["path"]), _ptr(out["extra"]))
    return out


def tree_verify_sample(parent, token, n_nodes, draft, target, temperature, seed=0, offset=0,
                       seq_ids=None):
    """Sampled verification of draft trees (multi-step speculative sampling
    with one draft distribution per node): parent, token [B, M] int32,
    n_nodes [B], draft and target logits [B, M, V] (float32 or bf16 bits; draft
    row u is the distribution u's children were drawn from), temperature [B];
    seq_ids [B] are the b of the Philox counter (default 0..B-1)."""
    zt, dt = _logits(target)
    zq, dq = _logits(draft)
    assert dq == dt and zq.shape == zt.shape
    B, M, V = zt.shape
    par = np.ascontiguousarray(parent, np.int32)
    tok = np.ascontiguousarray(token, np.int32)
    nn = np.ascontiguousarray(n_nodes, np.int32).reshape(B)
    temp = np.ascontiguousarray(temperature, np.float32).reshape(B)
    sid = None if seq_ids is None else np.ascontiguousarray(seq_ids, np.int64).reshape(B)
    out = dict(length=np.zeros(B, np.int32), path=np.zeros((B, M), np.int32),
               extra=np.zeros(B, np.int32), acc_margin=np.zeros(B), res_margin=np.zeros(B))
    _load().oracle_tree_verify_sample(B, M, V, dt, _ptr(par), _ptr(tok), _ptr(nn), _ptr(zq),
                                      _ptr(zt), _ptr(temp), seed, offset, _ptr(sid),
                                      _ptr(out["length"]), _ptr(out["path"]), _ptr(out["extra"]),
                                      _ptr(out["acc_margin"]), _ptr(out["res_margin"]))
    return out


UCB1 = 0
THOMPSON = 1


def gamma_sample(shape: float, seed: int, offset: int, group: int = 0, arm: int = 0,
                 which: int = 0) -> tuple[float, float]:
    """One Gamma(shape, 1) variate (shape >= 1) and the smallest decision margin."""
    m = ctypes.c_double(np.inf)
    x = _load().oracle_gamma_mt(float(shape), seed, offset, group, arm, which, ctypes.byref(m))
    return x, m.value


def beta_sample(a: float, b: float, seed: int, offset: int, group: int = 0,
                arm: int = 0) -> tuple[float, float]:
    m = ctypes.c_double(np.inf)
    x = _load().oracle_beta_sample(float(a), float(b), seed, offset, group, arm, ctypes.byref(m))
    return x, m.value


class Bandit:
    """G independent K-armed bandits over groups of B/G consecutive sequences.
    ``counts`` [G, K] uint32 and ``sums`` [G, K] float64 are the whole state."""

    def __init__(self, policy: int, groups: int, arms: int, batch: int, gamma: int):
        assert policy in (UCB1, THOMPSON) and 1 <= arms <= 64 and gamma >= 1
        assert groups >= 1 and batch % groups == 0
        self.policy, self.G, self.K, self.B, self.gamma = policy, groups, arms, batch, gamma
        self.counts = np.zeros((groups, arms), dtype=np.uint32)
        self.sums = np.zeros((groups, arms), dtype=np.float64)

    def step(self, accept_len=None, arm_played=None, seed: int = 0, offset: int = 0):
        """Fold in ``accept_len`` [B] for ``arm_played`` [G] (if given), then choose.
        Returns (next arm [G] int32, decision margin [G] float64)."""
        al = ap = None
        if accept_len is not None:
            al = np.ascontiguousarray(accept_len, dtype=np.int32).reshape(self.B)
            ap = np.ascontiguousarray(arm_played, dtype=np.int32).reshape(self.G)
        out = np.zeros(self.G, dtype=np.int32)
        mg = np.zeros(self.G, dtype=np.float64)
        _load().oracle_bandit_step(self.policy, self.G, self.K, self.B, self.gamma,
                                   _ptr(self.counts), _ptr(self.sums), _ptr(al), _ptr(ap),
                                   seed, offset, _ptr(out), _ptr(mg))
        return out, mg
