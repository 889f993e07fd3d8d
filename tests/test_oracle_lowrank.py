"""Pins of the low-rank draft head oracle (``oracle.lowrank_head``).

The SlimSpec summary (Methodology, architecture) factors the draft LM head as
z = W_up W_down h with W_down in R^{r x d}, W_up in R^{V x r}, computed with
dense matrix products; the head's logits are what the verifier's draft rows
read, so the oracle also gives their log-normaliser at the row's temperature.

Pins (independent of the oracle's loops):
* the exact products against numpy's float64 matrix products;
* the bfloat16 roundings against PyTorch's float32 -> bfloat16 conversion on
  values float32 holds exactly, and against hand-made ties (to even);
* the normaliser against scipy.special.logsumexp;
* rank one: z_v = W_up[v, 0] * u_0 exactly, the closed form;
* exact scaling: h -> 2h doubles u and z (powers of two are exact in bf16).
"""
import numpy as np
import torch
from scipy.special import logsumexp

import oracle
import specgen


def bf(x):
    return specgen.f32_to_bf16_bits(np.asarray(x, np.float32))


def bf1(x):
    return bf([x])[0]


def f(bits):
    return specgen.bf16_bits_to_f32(bits).astype(np.float64)


def small(seed=0, N=6, d=96, r=32, V=300):
    return specgen.lowrank_head_inputs(N, d, r, V, seed=seed)


def test_products_match_numpy():
    x = small()
    out = oracle.lowrank_head(x["h"], x["w_down"], x["w_up"], x["temperature"])
    u_ref = f(x["h"]) @ f(x["w_down"]).T
    np.testing.assert_allclose(out["u_exact"], u_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out["u_abs"], np.abs(f(x["h"])) @ np.abs(f(x["w_down"])).T, rtol=1e-13)
    z_ref = f(out["u"]) @ f(x["w_up"]).T       # from the rounded activation (SL1)
    np.testing.assert_allclose(out["z_exact"], z_ref, rtol=1e-12, atol=1e-12)


def test_bf16_rounding_matches_torch_and_ties_go_to_even():
    x = small(seed=1)
    out = oracle.lowrank_head(x["h"], x["w_down"], x["w_up"], x["temperature"])
    # values float32 holds exactly round the same from float32 and from double
    for exact, bits in ((out["u_exact"], out["u"]), (out["z_exact"], out["z"])):
        f32 = exact.astype(np.float32)
        held = f32.astype(np.float64) == exact
        ref = torch.from_numpy(f32[held]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert held.sum() > 0
        assert np.array_equal(bits[held], ref)
        # and every rounding is to a nearest neighbour
        err = np.abs(f(bits) - exact)
        ulp = np.abs(f(bits.astype(np.uint16) + np.uint16(1)) - f(bits))
        assert (err <= 0.5 * ulp + 1e-300).all()
    # hand-made ties: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7 (bf16 has 7
    # fraction bits); even is 1. 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and
    # 1 + 2^-6; even is 1 + 2^-6.
    h = np.zeros((2, 32), np.uint16)
    h[:, 0] = bf1(1.0)
    wd = np.zeros((2, 32), np.uint16)
    wd[0, 0] = bf1(1.0)
    wd[1, 0] = bf1(1.0)
    h[0, 1] = bf1(2.0 ** -8)
    h[1, 1] = bf1(3 * 2.0 ** -8)
    wd[:, 1] = bf1(1.0)
    wu = np.zeros((1, 2), np.uint16)
    wu[0, 0] = bf1(1.0)
    out = oracle.lowrank_head(h, wd, wu, np.ones(2, np.float32))
    assert f(out["u"][0, 0]) == 1.0
    assert f(out["u"][1, 0]) == 1.0 + 2.0 ** -6


def test_lse_matches_scipy():
    x = small(seed=2)
    out = oracle.lowrank_head(x["h"], x["w_down"], x["w_up"], x["temperature"])
    for i, t in enumerate(x["temperature"]):
        if t == 0:
            assert np.isnan(out["lse"][i])
            continue
        inv_t = np.float32(1.0) / np.float32(t)
        xs = (specgen.bf16_bits_to_f32(out["z"][i]) * inv_t).astype(np.float64)
        assert abs(out["lse"][i] - logsumexp(xs)) < 1e-12 * max(1.0, abs(out["lse"][i]))


def test_rank_one_closed_form_and_exact_scaling():
    x = small(seed=3, r=32)
    wd = x["w_down"].copy()
    wd[1:] = 0                       # rank one in effect: only u_0 is nonzero
    out = oracle.lowrank_head(x["h"], wd, x["w_up"], x["temperature"])
    assert (out["u_exact"][:, 1:] == 0).all()
    np.testing.assert_array_equal(out["z_exact"], f(out["u"][:, :1]) * f(x["w_up"][:, 0])[None, :])
    h2 = bf(2.0 * specgen.bf16_bits_to_f32(x["h"]))
    out2 = oracle.lowrank_head(h2, x["w_down"], x["w_up"], x["temperature"])
    base = oracle.lowrank_head(x["h"], x["w_down"], x["w_up"], x["temperature"])
    np.testing.assert_array_equal(out2["u_exact"], 2.0 * base["u_exact"])
    np.testing.assert_array_equal(f(out2["z"]), 2.0 * f(base["z"]))


def test_row_subset_matches_full():
    x = small(seed=4)
    full = oracle.lowrank_head(x["h"], x["w_down"], x["w_up"], x["temperature"])
    sub = oracle.lowrank_head(x["h"], x["w_down"], x["w_up"], x["temperature"], rows=[4, 1])
    for key in ("u", "z"):
        assert np.array_equal(sub[key], full[key][[4, 1]])
    np.testing.assert_array_equal(sub["lse"], full["lse"][[4, 1]])
