"""Race check: back-to-back calls on one context with the same inputs and
(seed, offset) give bitwise-identical outputs, 100 times over. The fused draw
hands out tiles through an LDS counter and the sampled tree verifier's parts
exchange shares through device memory, so a race in either would show as a
difference between repeats. Stops at the first difference."""
import numpy as np
import pytest
import torch

import device_draft_verification_amd as sv
import specgen
from gpu_helpers import to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

REPEATS = 100


def test_verification_repeats_bitwise_B256():
    rec = specgen.config(4)
    t = to_device(specgen.generate(rec))
    B, G = rec.batch, rec.gamma
    ctx = sv.spec_verify_init(B, G, rec.vocab, torch.bfloat16)
    assert sv.spec_verify_get_geometry(ctx)["residual_splits"] == 0  # the fused draw
    alen = torch.empty(B, dtype=torch.int32, device="cuda")
    toks = torch.empty(B, G + 1, dtype=torch.int32, device="cuda")
    lse = torch.empty((B, 2 * G + 1), dtype=torch.float64, device="cuda")
    first = None
    for r in range(REPEATS):
        alen.fill_(-7)
        toks.fill_(-7)
        sv.spec_verify(ctx, t["logits_draft"], t["logits_target"], t["draft_tokens"],
                       t["temperature"], 0, 0, alen, toks)
        sv.spec_verify_copy_lse(ctx, lse)
        got = (alen.cpu().numpy(), toks.cpu().numpy(), lse.cpu().numpy().view(np.uint64))
        if first is None:
            first = got
            continue
        for a, b, name in zip(first, got, ("accept_len", "tokens", "lse")):
            assert np.array_equal(a, b), f"repeat {r}: {name} differs"
    print(f"\n[determinism B=256 verification] {REPEATS} calls bitwise equal", flush=True)
    sv.spec_verify_destroy(ctx)


def test_sampled_tree_repeats_bitwise():
    B, M, V = 256, 16, 152064
    trees = specgen.draft_trees(B, M, V, seed=31)
    zt = specgen.tree_target_logits(trees, V, seed=5)
    zq = specgen.tree_target_logits(trees, V, seed=6)
    rng = np.random.default_rng(7)
    temp = rng.uniform(0.3, 1.5, B).astype(np.float32)
    temp[rng.random(B) < 0.1] = 0.0
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    args = (dev(trees["parent"]), dev(trees["token"]), dev(np.full(B, M, np.int32)), bf(zq), bf(zt),
            dev(temp))
    ctx = sv.spec_tree_verify_init(B, M, V, torch.bfloat16)
    L = torch.empty(B, dtype=torch.int32, device="cuda")
    path = torch.empty((B, M), dtype=torch.int32, device="cuda")
    extra = torch.empty(B, dtype=torch.int32, device="cuda")
    first = None
    for r in range(REPEATS):
        L.fill_(-7)
        extra.fill_(-7)
        sv.spec_tree_verify_sample(ctx, *args, 2, 4, L, path, extra)
        got = (L.cpu().numpy(), path.cpu().numpy(), extra.cpu().numpy())
        if first is None:
            assert (got[0] >= 0).all()
            first = got
            continue
        for a, b, name in zip(first, got, ("length", "path", "extra")):
            assert np.array_equal(a, b), f"repeat {r}: {name} differs"
    print(f"\n[determinism sampled trees B={B} M={M}] {REPEATS} calls bitwise equal", flush=True)
    sv.spec_tree_verify_destroy(ctx)
