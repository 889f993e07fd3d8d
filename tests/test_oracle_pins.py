"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test pins one part of the oracle to a library routine, a closed form, an
exhaustive sweep or a statistical law that the verification method must obey:

* Philox4x32-10 -- bitwise against the header-only engine shipped with
  PyTorch's C++ headers (an independent implementation of the SC'11 definition).
* row log-sum-exp -- scipy.special.logsumexp and three closed forms; the
  temperature-before-log-softmax order (FlashSpec technical summary,
  Methodology section 1, numerical-stability bullet) by an exact power-of-two
  identity.
* argmax -- numpy.argmax (first index on ties).
* inverse CDF -- exact bin counts over the whole uniform grid and worked
  margins.
* the accept test -- exact sweep of u: P(accept) = min(1, p_t / q_t).
* the residual -- exact sweep of u: P(token = v | reject) = max(0, p - q)_v / S.
"""
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
import specgen

TORCH_INCLUDE = None
try:  # torch is only used here for the location of its C++ headers
    import torch.utils.cpp_extension as _ce
    for p in _ce.include_paths():
        if os.path.exists(os.path.join(p, "ATen", "core", "PhiloxRNGEngine.h")):
            TORCH_INCLUDE = p
            break
except Exception:  # pragma: no cover
    TORCH_INCLUDE = None


def scaled_f32(z, temperature):
    """fl32(z * fl32(1/T)) computed with numpy binary32 arithmetic."""
    inv_t = np.float32(1.0) / np.float32(temperature)
    return (np.asarray(z, dtype=np.float32) * inv_t).astype(np.float32)


# --------------------------------------------------------------------- Philox

_PHILOX_PROG = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdlib>
#include <cstdint>
int main(int argc, char** argv) {
  // each stdin line: seed offset b i  -> four words of block (i, b, lo(offset), hi(offset))
  unsigned long long seed, offset, b, i;
  while (std::scanf("%llu %llu %llu %llu", &seed, &offset, &b, &i) == 4) {
    // the engine's counter is (lo(n), hi(n), lo(subsequence), hi(subsequence))
    at::philox_engine e(seed, offset, (b << 32) | i);
    unsigned w0 = e(), w1 = e(), w2 = e(), w3 = e();
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
"""


def build_torch_philox_exe(d):
    """Compile the library-engine Philox program into directory d; its path."""
    if TORCH_INCLUDE is None or shutil.which("g++") is None:
        pytest.skip("PyTorch C++ headers or g++ not available")
    src = os.path.join(d, "p.cpp")
    exe = os.path.join(d, "p")
    with open(src, "w") as f:
        f.write(_PHILOX_PROG)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", TORCH_INCLUDE, src, "-o", exe],
                   check=True, capture_output=True)
    return exe


@pytest.fixture(scope="module")
def torch_philox_exe():
    d = tempfile.mkdtemp(prefix="philox_pin_")
    yield build_torch_philox_exe(d)
    shutil.rmtree(d, ignore_errors=True)


def test_philox_matches_library_engine(torch_philox_exe):
    rng = np.random.default_rng(11)
    cases = [(0, 0, 0, 0), (0, 0, 1, 0), (0, 0, 0, 1), (2**64 - 1, 2**64 - 1, 2**32 - 1, 2**31 - 1),
             (0x0123456789ABCDEF, 7, 255, 8), (1, 2**32, 3, 4)]
    for _ in range(200):
        cases.append((int(rng.integers(0, 2**63)), int(rng.integers(0, 2**63)),
                      int(rng.integers(0, 2**31)), int(rng.integers(0, 71))))
    inp = "".join(f"{s} {o} {b} {i}\n" for s, o, b, i in cases)
    out = subprocess.run([torch_philox_exe], input=inp, capture_output=True, text=True,
                         check=True).stdout.split("\n")
    for (s, o, b, i), line in zip(cases, out):
        ref = np.array([int(w) for w in line.split()], dtype=np.uint32)
        got = oracle.philox_words(s, o, b, i)
        assert np.array_equal(ref, got), (s, o, b, i, ref, got)


def test_philox_raw_interface_matches_words():
    w = oracle.philox_words(0xDEADBEEF12345678, 0x1111222233334444, 77, 5)
    raw = oracle.philox4x32_10([5, 77, 0x33334444, 0x11112222], [0x12345678, 0xDEADBEEF])
    assert np.array_equal(w, raw)


def test_uniform24_range_and_grid():
    assert oracle.uniform24(0) == 0.0
    assert oracle.uniform24(0xFFFFFFFF) == 1.0 - 2.0 ** -24
    assert oracle.uniform24(0x000000FF) == 0.0  # low 8 bits are dropped
    assert oracle.uniform24(0x00000100) == 2.0 ** -24
    assert oracle.uniform24(0x80000000) == 0.5


def test_philox_uniforms_look_uniform_and_independent():
    from scipy.stats import kstest
    n = 20000
    u0 = np.array([oracle.uniform24(oracle.philox_words(3, 9, b, 0)[0]) for b in range(n)])
    u1 = np.array([oracle.uniform24(oracle.philox_words(3, 9, b, 1)[0]) for b in range(n)])
    assert kstest(u0, "uniform").pvalue > 0.01
    assert kstest(u1, "uniform").pvalue > 0.01
    assert abs(np.corrcoef(u0, u1)[0, 1]) < 4.0 / math.sqrt(n)


# ------------------------------------------------------------------------ LSE

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1.0, 0.7, 0.3, 1.5, 2.0])
def test_row_lse_matches_scipy(dtype, T):
    rng = np.random.default_rng(5)
    z = rng.normal(0, 3.0, size=20011).astype(np.float32)
    if dtype == "bf16":
        bits = specgen.f32_to_bf16_bits(z)
        zf = specgen.bf16_bits_to_f32(bits)
        got = oracle.row_lse(bits, T)
    else:
        zf = z
        got = oracle.row_lse(z, T)
    x = scaled_f32(zf, T).astype(np.float64)
    ref = logsumexp(x)
    assert abs(got - ref) <= 1e-12 * max(1.0, abs(ref))


def test_row_lse_closed_forms():
    V = 1000
    c = np.float32(3.25)
    assert abs(oracle.row_lse(np.full(V, c, np.float32), 1.0) - (3.25 + math.log(V))) < 1e-12
    z = np.full(V, -np.inf, np.float32)
    z[417] = np.float32(-2.5)
    assert oracle.row_lse(z, 1.0) == -2.5
    d = np.float32(1.75)
    z = np.full(V, c, np.float32)
    z[3] = c + d
    ref = 3.25 + math.log(V - 1 + math.exp(1.75))
    assert abs(oracle.row_lse(z, 1.0) - ref) < 1e-12
    assert oracle.row_lse(np.full(V, -np.inf, np.float32), 1.0) == -math.inf


def test_temperature_applies_before_log_softmax():
    """T = 2 on z equals T = 1 on z / 2 bit for bit (both are exact scalings).
    Scaling after the log-softmax would give lse(z) / 2 instead."""
    rng = np.random.default_rng(6)
    z = rng.normal(0, 4.0, size=5003).astype(np.float32)
    a = oracle.row_lse(z, 2.0)
    b = oracle.row_lse((z / np.float32(2.0)).astype(np.float32), 1.0)
    assert a == b
    assert abs(a - oracle.row_lse(z, 1.0) / 2.0) > 1e-3


# --------------------------------------------------------------------- argmax

def test_row_argmax_first_index_on_ties():
    rng = np.random.default_rng(7)
    for _ in range(50):
        z = rng.integers(-3, 4, size=257).astype(np.float32)  # many exact ties
        assert oracle.row_argmax(z) == int(np.argmax(z))
    bits = specgen.f32_to_bf16_bits(rng.normal(0, 1, 4099).astype(np.float32))
    bits[100] = bits[3000] = specgen.f32_to_bf16_bits(np.float32([9.0]))[0]
    assert oracle.row_argmax(bits) == 100
    assert oracle.row_argmax(np.full(9, -np.inf, np.float32)) == -1


# ---------------------------------------------------------------- inverse CDF

def test_inverse_cdf_worked_margins():
    r = np.array([1.0, 1.0, 2.0])
    assert oracle.inverse_cdf(r, 0.1) == (0, pytest.approx(math.log(1.0 / 0.4)))
    j, m = oracle.inverse_cdf(r, 0.25)    # tau = 1.0 sits on the edge C_0
    assert j == 1 and m == 0.0
    j, m = oracle.inverse_cdf(r, 0.5)     # tau = 2.0 sits on the edge C_1
    assert j == 2 and m == 0.0
    j, m = oracle.inverse_cdf(r, 0.6)     # tau = 2.4 in [2, 4)
    assert j == 2 and m == pytest.approx(min(math.log(2.4 / 2.0), math.log(4.0 / 2.4)))
    j, m = oracle.inverse_cdf(np.array([0.0, 0.0, 3.0]), 0.0)
    assert j == 2 and m == 0.0
    assert oracle.inverse_cdf(np.zeros(4), 0.5)[0] == -1


def test_inverse_cdf_exact_bin_counts():
    """Over the grid u = k / N the number of draws landing on v is N * r_v / S,
    up to one grid point per bin edge."""
    rng = np.random.default_rng(8)
    N = 4096
    for _ in range(5):
        r = rng.exponential(size=8)
        r[rng.integers(0, 8)] = 0.0
        counts = np.zeros(8, np.int64)
        for k in range(N):
            counts[oracle.inverse_cdf(r, k / N)[0]] += 1
        assert np.all(np.abs(counts - N * r / r.sum()) <= 1.0 + 1e-9)
        assert counts[r == 0].sum() == 0


def test_inverse_cdf_alt_worked_neighbours():
    """The token across the nearer edge of the chosen bin, skipping zero weights."""
    r = np.array([0.0, 1.0, 0.0, 2.0, 3.0, 0.0])            # S = 6, edges 1, 3, 6
    j, m, a = oracle.inverse_cdf_alt(r, 1.0000001 / 6.0)     # just above the edge C_1 = 1
    assert (j, a) == (3, 1) and m == pytest.approx(math.log(1.0000001), rel=1e-6)
    j, m, a = oracle.inverse_cdf_alt(r, 2.9999999 / 6.0)     # just below C_3 = 3
    assert (j, a) == (3, 4) and m == pytest.approx(math.log(3.0 / 2.9999999), rel=1e-6)
    assert oracle.inverse_cdf_alt(r, 5.99 / 6.0)[::2] == (4, -1)   # no mass above
    assert oracle.inverse_cdf_alt(r, 0.5 / 6.0)[::2] == (1, 3)     # lower edge is 0: upper side
    assert oracle.inverse_cdf_alt(r, 0.0) == (1, 0.0, 3)
    assert oracle.inverse_cdf_alt(np.zeros(3), 0.5)[::2] == (-1, -1)


def test_inverse_cdf_alt_is_the_draw_just_across_the_edge():
    """Brute force: moving tau across the nearer bin edge by a hair (a tiny
    change of u, as another summation order would make) lands on the alt
    token, and the margin is the log distance to that edge."""
    rng = np.random.default_rng(31)
    for _ in range(20):
        r = rng.exponential(size=16)
        r[rng.choice(16, size=4, replace=False)] = 0.0
        for u in rng.random(40):
            j, m, a = oracle.inverse_cdf_alt(r, u)
            assert j == oracle.inverse_cdf(r, u)[0] and r[j] > 0
            ud, uu = u * math.exp(-m) * (1 - 1e-9), u * math.exp(m) * (1 + 1e-9)
            down = oracle.inverse_cdf(r, ud)[0]
            up = oracle.inverse_cdf(r, uu)[0] if uu < 1 else -1
            if a >= 0:
                assert a != j and r[a] > 0 and a in (down, up)
            else:
                assert j == np.nonzero(r)[0].max() and down == j


# -------------------------------------------------- accept test and residual

def _tiny_case(seed, V=8, G=1, sd=1.5, noise=1.0):
    rng = np.random.default_rng(seed)
    base = rng.normal(0, sd, size=(G + 1, V))
    zp = (base + rng.normal(0, noise, size=base.shape)).astype(np.float32)
    zq = base[:G].astype(np.float32)
    return zq, zp


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_accept_probability_exact_sweep(T):
    """With the draft token fixed at t, the fraction of the 24-bit-style grid of
    u_acc that accepts equals min(1, p_t / q_t) (standard speculative sampling)."""
    zq, zp = _tiny_case(21)
    q = softmax(scaled_f32(zq[0], T).astype(np.float64))
    p = softmax(scaled_f32(zp[0], T).astype(np.float64))
    N = 2048
    for t in range(8):
        acc = 0
        for k in range(N):
            u = (k + 0.5) / N
            r = oracle.verify_sequence(zq, zp, [t], T, [u], [0.5, 0.5])
            acc += r["accept_len"] == 1
        assert abs(acc / N - min(1.0, p[t] / q[t])) <= 1.0 / N + 1e-12, t


@pytest.mark.parametrize("T", [1.0, 0.8])
def test_residual_distribution_exact_sweep(T):
    """After a rejection at position 0 the token follows max(0, p - q) / S."""
    zq, zp = _tiny_case(22)
    q = softmax(scaled_f32(zq[0], T).astype(np.float64))
    p = softmax(scaled_f32(zp[0], T).astype(np.float64))
    r = np.maximum(0.0, p - q)
    t = int(np.argmax(q / p))           # a token with p_t < q_t: rejectable
    u_acc = 1.0 - 2.0 ** -24             # log u above log(p_t / q_t): reject
    N = 4096
    counts = np.zeros(8, np.int64)
    for k in range(N):
        out = oracle.verify_sequence(zq, zp, [t], T, [u_acc], [k / N, 0.0])
        assert out["accept_len"] == 0
        counts[out["tokens"][0]] += 1
    assert np.all(np.abs(counts - N * r / r.sum()) <= 1.0 + 1e-9)


def test_bonus_distribution_exact_sweep():
    """All drafts accepted (u_acc = 0): the bonus token follows p at position gamma."""
    zq, zp = _tiny_case(23, G=2)
    p2 = softmax(zp[2].astype(np.float64))
    N = 4096
    counts = np.zeros(8, np.int64)
    toks = [int(np.argmax(zq[0])), int(np.argmax(zq[1]))]
    for k in range(N):
        out = oracle.verify_sequence(zq, zp, toks, 1.0, [0.0, 0.0], [0.3, 0.3, k / N])
        assert out["accept_len"] == 2
        assert list(out["tokens"][:2]) == toks
        counts[out["tokens"][2]] += 1
    assert np.all(np.abs(counts - N * p2 / p2.sum()) <= 1.0 + 1e-9)


def test_gathered_logprobs_normalise():
    """sum_v exp(x_v - lse) == 1 for every row the oracle normalises."""
    rec = specgen.config(2).replace(batch=2, vocab=3001)
    d = specgen.generate(rec)
    out = oracle.verify(d["logits_draft"], d["logits_target"], d["draft_tokens"],
                        d["temperature"])
    zf = specgen.bf16_bits_to_f32(d["logits_target"])
    for b in range(2):
        for i in range(rec.gamma + 1):
            x = scaled_f32(zf[b, i], d["temperature"][b]).astype(np.float64)
            s = np.exp(x - out["lse"][b, rec.gamma + i]).sum()
            assert abs(s - 1.0) < 1e-12


def test_draw_at_matches_the_verification_and_its_distribution():
    """The draw at a given position equals the verification's own extra token
    whenever the first rejection (or the bonus) is at that position, and over
    a grid of uniforms it follows max(0, p - q) / S exactly."""
    T = 0.9
    zq, zp = _tiny_case(24, G=2)
    q0 = softmax(scaled_f32(zq[0], T).astype(np.float64))
    p0 = softmax(scaled_f32(zp[0], T).astype(np.float64))
    r = np.maximum(0.0, p0 - q0)
    t = int(np.argmax(q0 / p0))
    N = 2048
    counts = np.zeros(8, np.int64)
    for k in range(N):
        u = k / N
        tok, m, a = oracle.draw_at(zq[0], zp[0], T, u)
        out = oracle.verify_sequence(zq, zp, [t, 0], T, [1.0 - 2.0 ** -24, 0.0], [u, 0.0, 0.0])
        assert out["accept_len"] == 0 and out["tokens"][0] == tok
        assert out["res_margin"] == m and out["res_alt"] == a
        counts[tok] += 1
    assert np.all(np.abs(counts - N * r / r.sum()) <= 1.0 + 1e-9)
    toks = [int(np.argmax(zq[0])), int(np.argmax(zq[1]))]
    for u in (0.0, 0.123, 0.5, 0.999):
        out = oracle.verify_sequence(zq, zp, toks, T, [0.0, 0.0], [0.3, 0.3, u])
        assert out["accept_len"] == 2
        assert oracle.draw_at(None, zp[2], T, u)[0] == out["tokens"][2]
