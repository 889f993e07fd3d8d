"""GPU parity of online draft selection: spec_bandit_step through the C ABI
against the oracle's bandit, step by step along whole trajectories.

Match rule:
* the state (play counts and reward sums) is compared bit for bit: it comes
  from integer sums, one correctly rounded double division and one double
  addition per play, identical on both sides;
* the chosen arm must be identical, except where the oracle takes the choice
  with a relative margin below 1e-9 (best vs second-best score, or a
  Marsaglia-Tsang test): the two sides' log / cos / sqrt may differ in the
  last ulp. Such steps are counted as flagged, and both sides then continue
  from the oracle's choice (the played arm is an input of the step).
"""
import numpy as np
import pytest
import torch

import device_draft_verification_amd as sv
import oracle
import specgen
from test_bandit_oracle import sample_accept_len

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

MARGIN = 1e-9
GAMMA = 4


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def check_choice(gpu_arm: torch.Tensor, orc_arm: np.ndarray, margin: np.ndarray) -> int:
    g = gpu_arm.cpu().numpy()
    bad = g != orc_arm
    flagged = bad & (margin < MARGIN)
    assert not (bad & ~flagged).any(), (np.nonzero(bad & ~flagged)[0][:8], g[bad][:8],
                                        orc_arm[bad][:8], margin[bad][:8])
    return int(flagged.sum())


def check_state(ctx, band):
    counts, sums = sv.spec_bandit_get_state(ctx)
    assert np.array_equal(counts, band.counts)
    assert np.array_equal(sums.view(np.uint64), band.sums.view(np.uint64))


def run_trajectory(policy, G, K, B, steps, seed, sentinel_rate=0.03, in_place=False):
    rng = np.random.default_rng(1000 * G + K + policy)
    alphas = rng.uniform(0.15, 0.9, size=(G, K))
    band = oracle.Bandit(policy, groups=G, arms=K, batch=B, gamma=GAMMA)
    ctx = sv.spec_bandit_init(G, K, B, GAMMA, policy)
    out = torch.full((G,), -7, dtype=torch.int32, device="cuda")
    arm_o, mg = band.step(seed=seed, offset=0)
    sv.spec_bandit_step(ctx, None, None, seed, 0, out)
    flagged = check_choice(out, arm_o, mg)
    per = B // G
    grp = np.repeat(np.arange(G), per)
    for t in range(1, steps + 1):
        played = arm_o.copy()
        k = sample_accept_len(rng, alphas[grp, np.repeat(played, per)], GAMMA)
        k[rng.random(B) < sentinel_rate] = -1
        arm_o, mg = band.step(k, played, seed=seed, offset=t)
        if in_place:
            out.copy_(i32(played))
            sv.spec_bandit_step(ctx, i32(k), out, seed, t, out)
        else:
            sv.spec_bandit_step(ctx, i32(k), i32(played), seed, t, out)
        flagged += check_choice(out, arm_o, mg)
        if t % 100 == 0 or t == steps:
            check_state(ctx, band)
    return flagged, band


@pytest.mark.parametrize("policy", [oracle.UCB1, oracle.THOMPSON], ids=["ucb1", "thompson"])
@pytest.mark.parametrize("G,K,B", [(1, 3, 16), (4, 8, 16), (16, 5, 16), (2, 64, 130),
                                   (512, 3, 512)])
def test_bandit_trajectory_parity(policy, G, K, B):
    steps = 200 if G >= 512 else 600
    print(f"\n[bandit policy={policy} G={G} K={K} B={B} steps={steps}]", flush=True)
    flagged, band = run_trajectory(policy, G, K, B, steps, seed=17)
    print(f"  flagged={flagged} plays={int(band.counts.sum())}", flush=True)
    assert flagged <= max(1, steps * G // 1000)


@pytest.mark.parametrize("policy", [oracle.UCB1, oracle.THOMPSON], ids=["ucb1", "thompson"])
def test_bandit_in_place_arm_buffer(policy):
    flagged, _ = run_trajectory(policy, 8, 4, 64, 150, seed=3, in_place=True)
    assert flagged == 0


def test_bandit_bad_arms_and_sentinels():
    G, K, B = 2, 3, 4
    band = oracle.Bandit(oracle.UCB1, groups=G, arms=K, batch=B, gamma=GAMMA)
    ctx = sv.spec_bandit_init(G, K, B, GAMMA, sv.SPEC_BANDIT_UCB1)
    out = torch.zeros(G, dtype=torch.int32, device="cuda")
    band.step()
    sv.spec_bandit_step(ctx, None, None, 0, 0, out)
    for k, played in (([2, -1, -1, -1], [0, 0]), ([4, 4, 4, 4], [3, -2]),
                      ([5, 5, 1, 3], [1, 1]), ([0, 9, 4, -3], [2, 0])):
        arm_o, _ = band.step(np.array(k, np.int32), np.array(played, np.int32))
        sv.spec_bandit_step(ctx, i32(k), i32(played), 0, 0, out)
        assert out.cpu().numpy().tolist() == arm_o.tolist()
        check_state(ctx, band)


@pytest.mark.parametrize("policy", [oracle.UCB1, oracle.THOMPSON], ids=["ucb1", "thompson"])
def test_bandit_set_state_resume_and_reset(policy):
    G, K, B = 3, 5, 6
    rng = np.random.default_rng(8)
    counts = rng.integers(1, 5000, size=(G, K)).astype(np.uint32)
    sums = counts * rng.uniform(0.0, 1.0, size=(G, K))
    band = oracle.Bandit(policy, groups=G, arms=K, batch=B, gamma=GAMMA)
    band.counts[:] = counts
    band.sums[:] = sums
    ctx = sv.spec_bandit_init(G, K, B, GAMMA, policy)
    sv.spec_bandit_set_state(ctx, counts, sums)
    check_state(ctx, band)
    out = torch.zeros(G, dtype=torch.int32, device="cuda")
    for off in range(50):
        arm_o, mg = band.step(seed=99, offset=off)
        sv.spec_bandit_step(ctx, None, None, 99, off, out)
        assert check_choice(out, arm_o, mg) == 0
    with pytest.raises(sv.SpecVerifyError):
        bad = sums.copy()
        bad[0, 0] = counts[0, 0] + 1.0
        sv.spec_bandit_set_state(ctx, counts, bad)
    check_state(ctx, band)  # a rejected state changes nothing
    sv.spec_bandit_set_state(ctx)
    c, s = sv.spec_bandit_get_state(ctx)
    assert not c.any() and not s.any()


def test_bandit_on_a_side_stream():
    G, K, B = 4, 3, 32
    side = torch.cuda.Stream()
    band = oracle.Bandit(oracle.THOMPSON, groups=G, arms=K, batch=B, gamma=GAMMA)
    with torch.cuda.stream(side):
        ctx = sv.spec_bandit_init(G, K, B, GAMMA, sv.SPEC_BANDIT_THOMPSON, stream=side)
        out = torch.zeros(G, dtype=torch.int32, device="cuda")
        k = i32(np.arange(B) % (GAMMA + 1))
        played = i32(np.arange(G) % K)
        for t in range(20):
            sv.spec_bandit_step(ctx, k, played, 5, t, out)
            arm_o, mg = band.step(np.arange(B) % (GAMMA + 1), np.arange(G) % K, seed=5, offset=t)
        side.synchronize()
    assert check_choice(out, arm_o, mg) == 0
    check_state(ctx, band)


def test_bandit_fed_by_the_verifier_on_the_device():
    """The decode loop without host round trips: spec_verify writes accept
    lengths on the device, spec_bandit_step reads them there and picks the
    next draft model for every group. Three draft models of different quality;
    the oracle bandit replays the same steps from the GPU's accept lengths,
    and each step's draft choice must agree."""
    B, G, V, K, groups, steps = 64, 4, 2000, 3, 4, 24
    rng = np.random.default_rng(2026)
    base = rng.normal(0.0, 2.0, size=(B, G + 1, V))
    target_bits = specgen.f32_to_bf16_bits(base.astype(np.float32))
    temp = np.full(B, 0.8, np.float32)
    draft_bits, draft_tok = [], []
    for noise in (0.3, 1.0, 2.5):
        zq = specgen.f32_to_bf16_bits((base[:, :G] + rng.normal(0, noise, (B, G, V))).astype(np.float32))
        draft_bits.append(zq)
        draft_tok.append(np.stack([specgen.gumbel_max_tokens(zq[b], 0.8, rng) for b in range(B)]))

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    stack = torch.stack([bf16(z) for z in draft_bits])                  # [K, B, G, V]
    tok_stack = torch.stack([i32(t) for t in draft_tok])                # [K, B, G]
    target = bf16(target_bits)
    tdev = torch.from_numpy(temp).cuda()
    verify = sv.spec_verify_init(B, G, V, torch.bfloat16)
    bandit = sv.spec_bandit_init(groups, K, B, G, sv.SPEC_BANDIT_UCB1)
    band = oracle.Bandit(oracle.UCB1, groups=groups, arms=K, batch=B, gamma=G)
    arm = torch.zeros(groups, dtype=torch.int32, device="cuda")
    alen = torch.zeros(B, dtype=torch.int32, device="cuda")
    toks = torch.zeros((B, G + 1), dtype=torch.int32, device="cuda")
    rows = torch.arange(B, device="cuda")
    per = B // groups
    sv.spec_bandit_step(bandit, None, None, 1, 0, arm)
    arm_o, _ = band.step(seed=1, offset=0)
    history = []
    for step in range(1, steps + 1):
        # every sequence of a group takes the logits and tokens of its group's draft
        sel = arm.long().repeat_interleave(per)
        ld = stack[sel, rows].contiguous()
        tk = tok_stack[sel, rows].contiguous()
        sv.spec_verify(verify, ld, target, tk, tdev, 7, step, alen, toks)
        played = arm.clone()
        sv.spec_bandit_step(bandit, alen, played, 1, step, arm)
        history.append((alen.clone(), played, arm.clone()))
    torch.cuda.synchronize()
    for step, (al, played, nxt) in enumerate(history, start=1):
        assert played.cpu().numpy().tolist() == arm_o.tolist(), step
        arm_o, mg = band.step(al.cpu().numpy(), played.cpu().numpy(), seed=1, offset=step)
        assert check_choice(nxt, arm_o, mg) == 0
    check_state(bandit, band)
    assert int(band.counts.sum()) == steps * groups
