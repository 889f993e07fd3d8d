"""GPU parity of the low-rank draft head (spec_lowrank_head) against
oracle.lowrank_head.

Match rule. The GPU accumulates in binary32 on the matrix cores; the oracle
computes the exact values (double) and rounds them to bf16. A binary32 sum
of n terms differs from the exact sum by at most about n * 2^-24 times the
sum of the terms' magnitudes; the longest rounding chain here is at most 2^6
(K / 512 accumulations per wavefront, at most 16 for the K <= 8192 tested,
the sum over 16 wavefronts, and the 32 products inside one MFMA), so the
tests allow c = 2^-16 (4x that) of the magnitude:
* activation u: each bf16 value equals the oracle's rounding, or, where the
  exact value lies within e_j = c * sum|W_down h| of a rounding boundary
  ("flip-possible"), it is within e_j + ulp/2 of the exact value (a binary32
  value within e_j, rounded); near zero that can be several ulps;
* logits z: the same with B_v = sum over flip-possible j of |W_up[v][j]| *
  (2 e_j + ulp(u_j)) (what the activation can differ by) + c * sum|W_up u|,
  against the oracle's z computed from the oracle's rounded u;
* normaliser: |lse_gpu - lse_oracle| <= 1.01 * (1/T) * sum over flip-possible
  v of p_v * (2 B_v + ulp(z_v)) + 2e-6 * max(1, |lse|) (a logit that moves by
  delta moves the normaliser by p_v * delta / T; the second term bounds the
  binary32 exp2 and the eight-term binary32 sums before binary64).
Counts of values that differ from the oracle's rounding are reported.
"""
import numpy as np
import pytest
import torch

import device_draft_verification_amd as sv
import oracle
import specgen

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

C_ACC = 2.0 ** -16


def f64(bits):
    return specgen.bf16_bits_to_f32(bits).astype(np.float64)


def boundary_distance(exact, bits):
    """Distance of the exact values to the nearer rounding boundary around
    their bf16 rounding `bits` (inf where a neighbour does not exist)."""
    b = bits.astype(np.int64)
    v = f64(bits)
    out = np.full(exact.shape, np.inf)
    for step in (-1, 1):
        nb = b + step
        ok = (nb >= 0) & (nb <= 0xFFFF)
        nv = f64(np.where(ok, nb, b).astype(np.uint16))
        fin = ok & np.isfinite(nv) & (nv != v)
        mid = 0.5 * (v + nv)
        out = np.where(fin, np.minimum(out, np.abs(exact - mid)), out)
    return out


def ulp_of(bits):
    b = bits.astype(np.int64)
    up = f64(np.minimum(b + 1, 0xFFFF).astype(np.uint16))
    return np.abs(up - f64(bits))


def adjacent(a, b):
    return np.abs(a.astype(np.int64) - b.astype(np.int64)) == 1


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def run_head(x):
    N, d = x["h"].shape
    r = x["w_down"].shape[0]
    V = x["w_up"].shape[0]
    ctx = sv.spec_lowrank_head_init(N, d, r, V)
    z = torch.empty((N, V), dtype=torch.int16, device="cuda")
    lse = torch.empty(N, dtype=torch.float64, device="cuda")
    u = torch.empty((N, r), dtype=torch.int16, device="cuda")
    sv.spec_lowrank_head(ctx, bf16_dev(x["h"]), bf16_dev(x["w_down"]), bf16_dev(x["w_up"]),
                         torch.from_numpy(x["temperature"]).cuda(), z, lse)
    sv.spec_lowrank_head_copy_activation(ctx, u)
    torch.cuda.synchronize()
    return dict(z=z.cpu().numpy().view(np.uint16), lse=lse.cpu().numpy(),
                u=u.cpu().numpy().view(np.uint16))


def check_rows(gpu, ref, x, rows):
    """Apply the match rule to `rows` (ref holds the oracle for those rows)."""
    flips_u = flips_z = 0
    for n, row in enumerate(rows):
        gu, ou = gpu["u"][row], ref["u"][n]
        e = C_ACC * ref["u_abs"][n]
        fu = boundary_distance(ref["u_exact"][n], ou) <= e          # flip-possible activations
        diff = gu != ou
        near = np.abs(f64(gu) - ref["u_exact"][n]) <= e + 0.5 * ulp_of(gu)
        assert not (diff & ~(fu & near)).any(), ("u", row, np.nonzero(diff & ~(fu & near))[0][:5])
        flips_u += int(diff.sum())
        du = np.where(fu, 2 * e + ulp_of(ou), 0.0)
        B = np.abs(f64(x["w_up"][:, fu])) @ du[fu] + C_ACC * ref["z_abs"][n]
        gz, oz = gpu["z"][row], ref["z"][n]
        fz = boundary_distance(ref["z_exact"][n], oz) <= B
        diffz = gz != oz
        nearz = np.abs(f64(gz) - ref["z_exact"][n]) <= B + 0.5 * ulp_of(gz)
        bad = diffz & ~(fz & nearz)
        assert not bad.any(), ("z", row, np.nonzero(bad)[0][:5], gz[bad][:5], oz[bad][:5])
        flips_z += int(diffz.sum())
        t = x["temperature"][row]
        if not t > 0:
            assert np.isnan(gpu["lse"][row]) and np.isnan(ref["lse"][n])
            continue
        inv_t = float(np.float32(1.0) / np.float32(t))
        xs = f64(oz) * inv_t
        p = np.exp(xs - ref["lse"][n])
        move = (2 * B[fz] + ulp_of(oz[fz]))
        tol = 1.01 * inv_t * float((p[fz] * move).sum()) + 2e-6 * max(1.0, abs(ref["lse"][n]))
        assert abs(gpu["lse"][row] - ref["lse"][n]) <= tol, (row, gpu["lse"][row], ref["lse"][n], tol)
    return flips_u, flips_z


@pytest.mark.parametrize("N,d,r,V", [
    (8, 128, 64, 296),         # single tiles, ragged everywhere
    (130, 256, 64, 2056),      # two row tiles, ragged vocabulary tile, split K
    (64, 1024, 128, 8192),     # several K splits and vocabulary tiles
    # the streaming second product (rank 256 or 512): W_up in 16-row blocks
    (8, 128, 256, 296),        # 19 blocks, the last one half full, one per workgroup
    (300, 256, 512, 2056),     # two 256-row batch tiles, ragged last block
    (37, 512, 512, 65544),     # 4097 blocks over the CUs, rows not a multiple of 16
])
def test_head_parity_small(N, d, r, V):
    x = specgen.lowrank_head_inputs(N, d, r, V, seed=N + d)
    print(f"\n[head N={N} d={d} r={r} V={V}]", flush=True)
    gpu = run_head(x)
    ref = oracle.lowrank_head(x["h"], x["w_down"], x["w_up"], x["temperature"])
    fu, fz = check_rows(gpu, ref, x, np.arange(N))
    print(f"  flips u={fu}/{N * r} z={fz}/{N * V}", flush=True)


def test_head_parity_full_size_sampled():
    """The B=256 draft step of the V=152064 workload with d = 4096 and the
    pages' example rank r = d / 8 = 512; the oracle on a sample of rows."""
    N, d, r, V = 256, 4096, 512, 152064
    x = specgen.lowrank_head_inputs(N, d, r, V, seed=11)
    print(f"\n[head N={N} d={d} r={r} V={V}]", flush=True)
    gpu = run_head(x)
    rows = np.array([0, 5, 77, 128, 200, N - 1])
    ref = oracle.lowrank_head(x["h"], x["w_down"], x["w_up"], x["temperature"], rows=rows)
    fu, fz = check_rows(gpu, ref, x, rows)
    print(f"  flips u={fu}/{rows.size * r} z={fz}/{rows.size * V}", flush=True)
    # every row: finite logits, normaliser NaN exactly for the greedy rows
    assert np.isfinite(f64(gpu["z"])).all()
    assert (np.isnan(gpu["lse"]) == (x["temperature"] == 0)).all()
    again = run_head(x)
    assert np.array_equal(again["z"], gpu["z"]) and np.array_equal(again["u"], gpu["u"])
    assert np.array_equal(again["lse"].view(np.uint64), gpu["lse"].view(np.uint64))


def test_head_feeds_the_verifier():
    """The head's logits are draft rows the verifier can read, and its fused
    normaliser equals the verifier's own normaliser of those rows (same
    definition, different summation order)."""
    B, G, d, r, V = 16, 2, 256, 64, 4096
    x = specgen.lowrank_head_inputs(B * G, d, r, V, seed=3, greedy_fraction=0.0)
    temp = np.repeat(x["temperature"][::G], G)          # one temperature per sequence
    x["temperature"] = temp
    gpu = run_head(x)
    draft = torch.from_numpy(gpu["z"].view(np.int16)).view(torch.bfloat16).cuda().view(B, G, V)
    target = torch.randn(B, G + 1, V, device="cuda").to(torch.bfloat16)
    tokens = torch.zeros(B, G, dtype=torch.int32, device="cuda")
    ctx = sv.spec_verify_init(B, G, V, torch.bfloat16)
    alen = torch.empty(B, dtype=torch.int32, device="cuda")
    toks = torch.empty(B, G + 1, dtype=torch.int32, device="cuda")
    tdev = torch.from_numpy(temp[::G].copy()).cuda()
    sv.spec_verify(ctx, draft, target, tokens, tdev, 0, 0, alen, toks)
    lse = torch.empty(B, 2 * G + 1, dtype=torch.float64, device="cuda")
    sv.spec_verify_copy_lse(ctx, lse)
    torch.cuda.synchronize()
    verifier = lse.cpu().numpy()[:, :G].reshape(-1)
    np.testing.assert_allclose(gpu["lse"], verifier, rtol=0, atol=2e-6 * np.maximum(1, np.abs(verifier)).max())


def test_head_rejects_misaligned_pointers():
    ctx = sv.spec_lowrank_head_init(4, 64, 64, 64)
    h = torch.zeros(4 * 64 + 1, dtype=torch.int16, device="cuda")[1:].view(4, 64)
    ok = lambda *s: torch.zeros(*s, dtype=torch.int16, device="cuda")
    with pytest.raises(sv.SpecVerifyError):
        sv.spec_lowrank_head(ctx, h, ok(64, 64), ok(64, 64), torch.ones(4, device="cuda"),
                             ok(4, 64), torch.zeros(4, dtype=torch.float64, device="cuda"))
