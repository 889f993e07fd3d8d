"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Sizes: the five workloads at full size (oracle on all sequences for the two
small ones, on a seeded sample of sequences for the three large ones, in the
same launch configuration the benchmark times), plus small cases that span
several vocabulary splits and a ragged tail, and the edge cases of the method.
"""
import concurrent.futures as cf
import math
import os

import numpy as np
import pytest
import torch

import device_draft_verification_amd as sv
import oracle
import specgen
from gpu_helpers import assert_parity, compare, record, run_gpu, to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


def _oracle(d, rows=None, seed=0, offset=0):
    """The oracle on all sequences of d (or on `rows`), cut into slices run on
    host threads (the oracle is single-threaded C; ctypes drops the GIL)."""
    if rows is not None:
        d = _subset(d, rows)
    B = d["logits_target"].shape[0]
    workers = max(1, min(16, os.cpu_count() or 1, B // 8))
    if workers == 1:
        return oracle.verify(d["logits_draft"], d["logits_target"], d["draft_tokens"],
                             d["temperature"], seed=seed, offset=offset, seq_ids=d["seq_ids"])
    cuts = np.linspace(0, B, workers + 1).astype(int)

    def part(i):
        a, b = cuts[i], cuts[i + 1]
        return oracle.verify(d["logits_draft"][a:b], d["logits_target"][a:b],
                             d["draft_tokens"][a:b], d["temperature"][a:b], seed=seed,
                             offset=offset, seq_ids=d["seq_ids"][a:b])

    with cf.ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(part, range(workers)))
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}


def _subset(d, rows):
    rows = np.asarray(rows)
    return dict(logits_draft=np.ascontiguousarray(d["logits_draft"][rows]),
                logits_target=np.ascontiguousarray(d["logits_target"][rows]),
                draft_tokens=np.ascontiguousarray(d["draft_tokens"][rows]),
                temperature=d["temperature"][rows], seq_ids=d["seq_ids"][rows])


def _check(label, gpu, d, seed=0, offset=0, ref=None, check_lse=True):
    """Oracle on every sequence of d, comparison, record, assertion."""
    ref = _oracle(d, seed=seed, offset=offset) if ref is None else ref
    rep = compare(gpu, ref, d["temperature"], data=d, seed=seed, offset=offset,
                  check_lse=check_lse)
    record(label, rep)
    assert_parity(rep, label)
    return rep


# ------------------------------------------------------------------ Philox --

@pytest.mark.parametrize("seed,offset", [(0, 0), (1, 7), (2**64 - 1, 2**63 + 5), (0xDEADBEEF, 2**32)])
def test_philox_words_bitwise(seed, offset):
    B, G = 37, 6
    ctx = sv.spec_verify_init(B, G, 64, torch.float32)
    out = torch.empty((B, G + 1, 4), dtype=torch.int32, device="cuda")
    sv.spec_verify_philox_words(ctx, seed, offset, out)
    got = out.cpu().numpy().view(np.uint32)
    for b in range(B):
        for i in range(G + 1):
            assert np.array_equal(got[b, i], oracle.philox_words(seed, offset, b, i)), (b, i)


# ------------------------------------------------- full-size small configs --

@pytest.mark.parametrize("cfg", [1, 2])
def test_small_config_full_parity(cfg):
    d = specgen.generate(specgen.config(cfg))
    gpu = run_gpu(to_device(d))
    _check(f"{specgen.config(cfg).name} full batch", gpu, d)


# --------------------------------------- splits, ragged tails, odd shapes --

CASES = [
    # (config recipe, overrides)
    (4, dict(batch=12, vocab=20008)),             # 16-byte groups, ragged last split
    (4, dict(batch=12, vocab=20011)),             # V % 8 != 0: element path
    (4, dict(batch=3, vocab=40001, gamma=2)),     # element path, 626 tiles: runs read in a loop
    (1, dict(batch=6, vocab=10003)),              # fp32 element path
    (1, dict(batch=6, vocab=12000, gamma=3)),     # fp32 16-byte groups
    (2, dict(batch=3, vocab=700, gamma=70)),      # more positions than one wavefront
    (4, dict(batch=4, vocab=520, gamma=130)),     # three passes of 64 positions, mixed T
    (2, dict(batch=5, vocab=4096, gamma=0)),      # bonus draw only
    (3, dict(batch=4, vocab=33000)),              # Zipf rows
    (5, dict(batch=9, vocab=257)),                # tiny vocabulary
    (2, dict(batch=2, vocab=1)),                  # V = 1
    (2, dict(batch=2, vocab=5)),                  # V < 8
]


@pytest.mark.parametrize("cfg,over", CASES)
def test_small_shapes_parity(cfg, over):
    rec = specgen.config(cfg).replace(**over)
    d = specgen.generate(rec)
    for seed, offset in [(0, 0), (12345, 3)]:
        gpu = run_gpu(to_device(d), seed=seed, offset=offset)
        _check(f"shape {rec.name} {over} seed={seed}", gpu, d, seed=seed, offset=offset)


@pytest.mark.parametrize("cfg,over", [CASES[i] for i in (0, 1, 2, 3, 5, 6, 7, 10, 11)])
@pytest.mark.parametrize("fused", [1, 0], ids=["fused", "split"])
def test_residual_kernel_choice_parity(cfg, over, fused, monkeypatch):
    """Both residual paths on the same inputs: the fused one-workgroup-per-
    sequence kernel (chosen by default from B = 128) and the split kernels
    (forced), each against the oracle, and against each other bit for bit."""
    monkeypatch.setenv("SPEC_VERIFY_RESIDUAL_FUSED", str(fused))
    rec = specgen.config(cfg).replace(**over)
    d = specgen.generate(rec)
    t = to_device(d)
    ctx = sv.spec_verify_init(rec.batch, rec.gamma, rec.vocab, t["logits_target"].dtype)
    geo = sv.spec_verify_get_geometry(ctx)
    assert (geo["residual_splits"] == 0) == bool(fused)
    gpu = run_gpu(t, seed=7, offset=1, ctx=ctx)
    _check(f"draw path {rec.name} {over} fused={fused}", gpu, d, seed=7, offset=1)
    monkeypatch.setenv("SPEC_VERIFY_RESIDUAL_FUSED", str(1 - fused))
    other = run_gpu(t, seed=7, offset=1)
    assert np.array_equal(other["tokens"], gpu["tokens"])
    assert np.array_equal(other["accept_len"], gpu["accept_len"])


# ------------------------------------------- full-size large configs, sampled --

@pytest.fixture(scope="module", params=[3, 4, 5])
def big(request):
    cfg = request.param
    rec = specgen.config(cfg)
    d = specgen.generate(rec)
    t = to_device(d)
    gpu = run_gpu(t, seed=0, offset=0)
    yield cfg, rec, d, t, gpu
    del t
    torch.cuda.empty_cache()


def test_large_config_full_parity(big):
    """Every sequence of the workload against the oracle (the launch
    configuration the benchmark times)."""
    cfg, rec, d, t, gpu = big
    _check(f"{rec.name} full batch", gpu, d)


def test_large_config_invariants(big):
    """Properties that hold for every sequence, checked on all of them."""
    cfg, rec, d, t, gpu = big
    k = gpu["accept_len"]
    toks = gpu["tokens"]
    G, V = rec.gamma, rec.vocab
    assert np.all((k >= 0) & (k <= G))
    for b in range(rec.batch):
        kb = k[b]
        assert np.array_equal(toks[b, :kb], d["draft_tokens"][b, :kb])
        assert 0 <= toks[b, kb] < V
        assert np.all(toks[b, kb + 1:] == -1)
    lse = gpu["lse"]
    sampled = d["temperature"] > 0
    assert np.all(np.isfinite(lse[sampled]))
    assert np.all(np.isnan(lse[~sampled]))


def test_large_config_deterministic(big):
    cfg, rec, d, t, gpu = big
    again = run_gpu(t, seed=0, offset=0)
    assert np.array_equal(again["accept_len"], gpu["accept_len"])
    assert np.array_equal(again["tokens"], gpu["tokens"])
    assert np.array_equal(again["lse"].view(np.uint64), gpu["lse"].view(np.uint64))


def test_config5_scalar_mode():
    """Scalar-only mode on the oracle's gathered log-probabilities of the
    B=512, gamma=4, V=201088 workload, rounded to fp32: [512, 4, 2]."""
    rec = specgen.config(5)
    d = specgen.generate(rec)
    pairs = oracle.gather_logprobs(d["logits_draft"], d["logits_target"], d["draft_tokens"],
                                   d["temperature"]).astype(np.float32)
    ref = oracle.accept_logprobs(pairs, seed=0, offset=0)
    ctx = sv.spec_verify_init(rec.batch, rec.gamma, rec.vocab, torch.bfloat16)
    lp = torch.from_numpy(pairs).cuda()
    out = torch.full((rec.batch,), -7, dtype=torch.int32, device="cuda")
    sv.spec_accept_logprobs(ctx, lp, 0, 0, out)
    got = out.cpu().numpy()
    diff = np.nonzero(got != ref["accept_len"])[0]
    for b in diff:
        k = min(got[b], ref["accept_len"][b])
        assert np.min(np.abs(ref["acc_margin"][b, :k + 1])) < 1e-5, b
    print(f"\n[{rec.name} scalar mode] mismatched-but-flagged={len(diff)} of {rec.batch}", flush=True)
    # cross-mode: the full call decides the same lengths, up to flagged decisions
    full = run_gpu(to_device(d), with_lse=False)
    cross = np.nonzero(full["accept_len"] != got)[0]
    for b in cross:
        k = min(got[b], full["accept_len"][b])
        assert np.min(np.abs(ref["acc_margin"][b, :k + 1])) < 1e-5, b


# ------------------------------------------------------------- edge cases --

def test_sentinel_sequences():
    rng = np.random.default_rng(8)
    B, G, V = 7, 3, 640
    zq = rng.normal(0, 1, size=(B, G, V)).astype(np.float32)
    zp = rng.normal(0, 1, size=(B, G + 1, V)).astype(np.float32)
    toks = rng.integers(0, V, size=(B, G)).astype(np.int32)
    temp = np.array([1.0, np.nan, -0.5, np.inf, 1.0, 1.0, 0.0], np.float32)
    toks[4, 1] = V
    zp[5, 2, :] = -np.inf
    zp[6, 0, :] = -np.inf  # greedy sequence with an empty target row
    d = dict(logits_draft=zq, logits_target=zp, draft_tokens=toks, temperature=temp,
             seq_ids=np.arange(B))
    gpu = run_gpu(to_device(d))
    ref = _oracle(d)
    assert np.array_equal(gpu["accept_len"], ref["accept_len"])
    assert np.array_equal(gpu["tokens"], ref["tokens"])
    assert list(gpu["accept_len"][1:]) == [-1] * 6


@pytest.mark.parametrize("B,G,V", [(64, 5, 3000), (6, 130, 600)])
def test_identical_rows_accept_all_and_bonus(B, G, V):
    # G = 130: the first rejection is searched over three passes of 64
    # positions, and the bonus row's coefficients come from the third.
    rng = np.random.default_rng(4)
    base = rng.normal(0, 2.0, size=(G + 1, V)).astype(np.float32)
    zp = np.ascontiguousarray(np.broadcast_to(base, (B, G + 1, V)))
    zq = np.ascontiguousarray(zp[:, :G])
    r2 = np.random.default_rng(5)
    toks = np.stack([specgen.gumbel_max_tokens(base[:G], 0.8, r2) for _ in range(B)])
    d = dict(logits_draft=zq, logits_target=zp, draft_tokens=toks,
             temperature=np.full(B, 0.8, np.float32), seq_ids=np.arange(B))
    gpu = run_gpu(to_device(d))
    assert np.all(gpu["accept_len"] == G)
    _check(f"identical rows B={B} G={G} V={V}", gpu, d)


def test_disjoint_support_rejects_all():
    G, V, B = 2, 64, 200
    rng = np.random.default_rng(5)
    zq = np.full((G, V), -np.inf, np.float32)
    zp = np.full((G + 1, V), -np.inf, np.float32)
    zq[:, :32] = rng.normal(0, 1, size=(G, 32))
    zp[:, 32:] = rng.normal(0, 1, size=(G + 1, 32))
    r2 = np.random.default_rng(6)
    toks = np.stack([specgen.gumbel_max_tokens(zq, 1.0, r2) for _ in range(B)])
    d = dict(logits_draft=np.ascontiguousarray(np.broadcast_to(zq, (B, G, V))),
             logits_target=np.ascontiguousarray(np.broadcast_to(zp, (B, G + 1, V))),
             draft_tokens=toks, temperature=np.ones(B, np.float32), seq_ids=np.arange(B))
    gpu = run_gpu(to_device(d))
    assert np.all(gpu["accept_len"] == 0)
    assert np.all(gpu["tokens"][:, 0] >= 32)
    _check("disjoint supports", gpu, d)


def test_greedy_ties_lowest_index():
    rng = np.random.default_rng(6)
    B, G, V = 32, 4, 2048
    zp = rng.integers(-4, 5, size=(B, G + 1, V)).astype(np.float32)  # many exact ties
    zq = rng.normal(0, 1, size=(B, G, V)).astype(np.float32)
    amax = np.argmax(zp, axis=-1)
    toks = amax[:, :G].astype(np.int32).copy()
    flip = rng.random((B, G)) < 0.3
    toks[flip] = (toks[flip] + 1) % V
    d = dict(logits_draft=zq, logits_target=zp, draft_tokens=toks,
             temperature=np.zeros(B, np.float32), seq_ids=np.arange(B))
    gpu = run_gpu(to_device(d))
    ref = _oracle(d)
    assert np.array_equal(gpu["accept_len"], ref["accept_len"])
    assert np.array_equal(gpu["tokens"], ref["tokens"])


def test_statistical_gate_on_gpu():
    """The CI gate (10,000 draws, V = 8, chi-square at 0.01) on the GPU's own
    output, plus parity of every draw with the oracle."""
    from scipy.special import softmax
    from scipy.stats import chisquare
    rng = np.random.default_rng(1234)
    G, V, N, T = 3, 8, 10_000, 0.9
    base = rng.normal(0, 1.2, size=(G + 1, V))
    zp = (base + rng.normal(0, 0.8, size=base.shape)).astype(np.float32)
    zq = base[:G].astype(np.float32)
    r2 = np.random.default_rng(99)
    toks = np.stack([specgen.gumbel_max_tokens(zq, T, r2) for _ in range(N)])
    d = dict(logits_draft=np.ascontiguousarray(np.broadcast_to(zq, (N, G, V))),
             logits_target=np.ascontiguousarray(np.broadcast_to(zp, (N, G + 1, V))),
             draft_tokens=toks, temperature=np.full(N, T, np.float32), seq_ids=np.arange(N))
    gpu = run_gpu(to_device(d), seed=2024, offset=7)
    _check("V=8 gate, 10000 draws", gpu, d, seed=2024, offset=7)
    inv_t = np.float32(1.0) / np.float32(T)
    p = softmax((zp * inv_t).astype(np.float64), axis=-1)
    first = gpu["tokens"][:, 0]
    assert chisquare(np.bincount(first, minlength=V), p[0] * N).pvalue > 0.01


def test_runs_on_a_side_stream_and_times_kernels():
    rec = specgen.config(2).replace(batch=8, vocab=32000)
    d = specgen.generate(rec)
    t = to_device(d)
    s = torch.cuda.Stream()
    ctx = sv.spec_verify_init(rec.batch, rec.gamma, rec.vocab, torch.bfloat16, stream=s)
    sv.spec_verify_enable_timing(ctx, 8)
    alen = torch.empty(rec.batch, dtype=torch.int32, device="cuda")
    toks = torch.empty(rec.batch, rec.gamma + 1, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(s):
        for i in range(3):
            sv.spec_verify(ctx, t["logits_draft"], t["logits_target"], t["draft_tokens"],
                           t["temperature"], 0, 0, alen, toks)
    times = sv.spec_verify_read_timing(ctx, 8)
    assert len(times) == 3
    # B = 8 takes the tile path, whose tile kernel runs the accept step: its
    # own slot reads 0
    assert sv.spec_verify_get_geometry(ctx)["residual_splits"] > 0
    assert all(row[0] > 0 and row[1] == 0 and row[2] > 0 for row in times)
    s.synchronize()
    gpu = dict(accept_len=alen.cpu().numpy(), tokens=toks.cpu().numpy())
    _check("side stream B=8", gpu, d, check_lse=False)
    geo = sv.spec_verify_get_geometry(ctx)
    assert geo["block"] == 256 and geo["row_splits"] >= 1


def test_argument_errors_on_device():
    ctx = sv.spec_verify_init(4, 2, 100, torch.float32)
    lib = sv.load_library()
    ok = torch.zeros((4, 3, 100), device="cuda")
    alen = torch.zeros(4, dtype=torch.int32, device="cuda")
    assert lib.spec_verify(ctx.handle, None, ok.data_ptr(), None, None, 0, 0,
                           alen.data_ptr(), alen.data_ptr()) == sv.binding.SPEC_EINVAL
    with pytest.raises(ValueError):
        sv.spec_verify(ctx, ok, ok, alen, alen, 0, 0, alen, alen)
    with pytest.raises(sv.SpecVerifyError):
        sv.spec_verify_copy_lse(ctx, torch.empty((4, 5), dtype=torch.float64, device="cuda"))


@pytest.mark.parametrize("cfg", [1, 4])
def test_misaligned_base_pointers_take_the_element_path(cfg):
    """Logit buffers whose base is not 16-byte aligned (one element in) run the
    element-load path even though V is a multiple of the 16-byte group."""
    rec = specgen.config(cfg).replace(batch=6, vocab=4096, gamma=3)
    d = specgen.generate(rec)
    t = to_device(d)
    for key in ("logits_draft", "logits_target"):
        x = t[key]
        buf = torch.empty(x.numel() + 1, dtype=x.dtype, device=x.device)
        view = buf[1:].view(x.shape)
        view.copy_(x)
        assert view.data_ptr() % 16 != 0
        t[key] = view
    gpu = run_gpu(t)
    _check(f"misaligned {rec.name}", gpu, d)


def _scalar_compare(lp, seed, offset):
    B, G, _ = lp.shape
    ctx = sv.spec_verify_init(B, G, 8, torch.float32)
    out = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    sv.spec_accept_logprobs(ctx, torch.from_numpy(lp).cuda(), seed, offset, out)
    got = out.cpu().numpy()
    ref = oracle.accept_logprobs(lp, seed=seed, offset=offset)
    for b in np.nonzero(got != ref["accept_len"])[0]:
        k = min(got[b], ref["accept_len"][b])
        m = np.abs(ref["acc_margin"][b, :k + 1])
        assert np.nanmin(m) < 1e-5, (b, got[b], ref["accept_len"][b])
    return got, ref["accept_len"]


def test_scalar_mode_edge_values():
    rng = np.random.default_rng(17)
    B, G = 64, 5
    lp = rng.normal(-3, 2, size=(B, G, 2)).astype(np.float32)
    lp[0, 0, 1] = np.nan           # NaN target log-prob: reject
    lp[1, 0, 0] = np.nan           # NaN draft log-prob: reject
    lp[2, 0, 1] = -np.inf          # p = 0: reject
    lp[3, 0, 0] = -np.inf          # q = 0 with p > 0: accept
    lp[4, :, :] = -np.inf          # both zero: NaN difference, reject
    lp[5, :, 1] = lp[5, :, 0]      # p = q: always accept
    got, ref = _scalar_compare(lp, 5, 9)
    assert list(got[:3]) == [0, 0, 0]
    assert got[3] >= 1
    assert got[4] == 0
    assert got[5] == G
    assert np.array_equal(got, ref)


def test_scalar_mode_gamma_zero_and_large_gamma():
    got, _ = _scalar_compare(np.zeros((7, 0, 2), np.float32), 1, 2)
    assert np.all(got == 0)
    rng = np.random.default_rng(18)
    lp = rng.normal(-2, 0.3, size=(300, 70, 2)).astype(np.float32)
    got, ref = _scalar_compare(lp, 123, 456)
    assert got.max() <= 70


def test_empty_batch_is_a_no_op():
    """B = 0: both calls return success and launch nothing (empty tensors give
    null data pointers, which a zero batch never dereferences); a later call
    on a non-empty context on the same stream still verifies correctly."""
    for G in (0, 3):
        ctx = sv.spec_verify_init(0, G, 1000, torch.bfloat16)
        e = lambda *shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device="cuda")
        alen = e(0, dt=torch.int32)
        sv.spec_verify(ctx, e(0, G, 1000), e(0, G + 1, 1000), e(0, G, dt=torch.int32),
                       e(0, dt=torch.float32), 0, 0, alen, e(0, G + 1, dt=torch.int32))
        sv.spec_accept_logprobs(ctx, e(0, G, 2, dt=torch.float32), 0, 0, alen)
        torch.cuda.synchronize()
        sv.spec_verify_destroy(ctx)
    rec = specgen.config(2).replace(batch=3, vocab=2048)
    d = specgen.generate(rec)
    gpu = run_gpu(to_device(d))
    _check("after empty calls", gpu, d)


def test_graph_capture_replays_match_eager():
    """The whole call records into a HIP graph (its workspace is allocated at
    init and nothing on the path clears memory with a memset node). Replays
    on two input sets copied into the captured buffers, with eager work in
    between, equal eager calls with the same (seed, offset) bit for bit."""
    rec = specgen.config(4).replace(batch=24, vocab=20000)
    sets = [to_device(specgen.generate(rec.replace(seed=s))) for s in (41, 42)]
    B, G = rec.batch, rec.gamma
    static = {k: v.clone() for k, v in sets[0].items()}
    s = torch.cuda.Stream()
    ctx = sv.spec_verify_init(B, G, rec.vocab, torch.bfloat16, stream=s)
    alen = torch.empty(B, dtype=torch.int32, device="cuda")
    toks = torch.empty(B, G + 1, dtype=torch.int32, device="cuda")

    def call():
        sv.spec_verify(ctx, static["logits_draft"], static["logits_target"],
                       static["draft_tokens"], static["temperature"], 9, 5, alen, toks)

    eager = []
    for t in sets:
        for k in static:
            static[k].copy_(t[k])
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            call()
        s.synchronize()
        eager.append((alen.clone(), toks.clone()))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for r, j in enumerate([1, 0, 1, 0]):
        for k in static:
            static[k].copy_(sets[j][k])
        alen.fill_(-7)
        toks.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(alen, eager[j][0]), f"replay {r}"
        assert torch.equal(toks, eager[j][1]), f"replay {r}"
        _ = (sets[j]["logits_target"].float().sum()).item()  # eager work between replays
    del g
    sv.spec_verify_destroy(ctx)


def test_offset_from_device_memory_and_graph_replays_with_fresh_uniforms():
    """spec_verify_offset_ptr equals spec_verify with the same offset bit for
    bit; captured in a HIP graph together with a one-element add that advances
    the offset word, each replay equals the eager call at the next offset."""
    rec = specgen.config(4).replace(batch=24, vocab=20000)
    d = specgen.generate(rec)
    t = to_device(d)
    B, G = rec.batch, rec.gamma
    s = torch.cuda.Stream()
    ctx = sv.spec_verify_init(B, G, rec.vocab, torch.bfloat16, stream=s)
    alen = torch.empty(B, dtype=torch.int32, device="cuda")
    toks = torch.empty(B, G + 1, dtype=torch.int32, device="cuda")
    off = torch.zeros(1, dtype=torch.int64, device="cuda")

    def eager(offset, ptr):
        with torch.cuda.stream(s):
            if ptr:
                off.fill_(offset)
                sv.spec_verify_offset_ptr(ctx, t["logits_draft"], t["logits_target"],
                                          t["draft_tokens"], t["temperature"], 3, off, alen, toks)
            else:
                sv.spec_verify(ctx, t["logits_draft"], t["logits_target"], t["draft_tokens"],
                               t["temperature"], 3, offset, alen, toks)
        s.synchronize()
        return alen.clone(), toks.clone()

    ref = {o: eager(o, False) for o in range(10, 14)}
    for o in (10, 11, (1 << 40) + 7):
        a = eager(o, True)
        b = eager(o, False) if o not in ref else ref[o]
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), o
    assert not all(torch.equal(ref[10][1], ref[o][1]) for o in (11, 12, 13))

    off.fill_(10)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        sv.spec_verify_offset_ptr(ctx, t["logits_draft"], t["logits_target"], t["draft_tokens"],
                                  t["temperature"], 3, off, alen, toks)
        off.add_(1)
    torch.cuda.synchronize()
    off.fill_(10)  # the capture itself ran nothing
    torch.cuda.synchronize()
    for o in range(10, 14):
        alen.fill_(-7)
        toks.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(alen, ref[o][0]), o
        assert torch.equal(toks, ref[o][1]), o
        assert int(off.item()) == o + 1
    del g
    sv.spec_verify_destroy(ctx)


@pytest.mark.parametrize("batch", [8, 128])
def test_dispatch_event_timing_fits_inside_the_call(batch):
    """Per-kernel durations from the events attached to the kernels'
    dispatches (split draw at B = 8, fused draw at B = 128) are positive -- the
    accept step's is 0 on the tile path, whose tile kernel runs it -- and their
    sum is no longer than the whole call timed by events around it."""
    rec = specgen.config(4).replace(batch=batch, vocab=30000)
    t = to_device(specgen.generate(rec))
    B, G = rec.batch, rec.gamma
    ctx = sv.spec_verify_init(B, G, rec.vocab, torch.bfloat16)
    assert (sv.spec_verify_get_geometry(ctx)["residual_splits"] == 0) == (batch >= 128)
    sv.spec_verify_enable_timing(ctx, 4)
    alen = torch.empty(B, dtype=torch.int32, device="cuda")
    toks = torch.empty(B, G + 1, dtype=torch.int32, device="cuda")
    outer = []
    for i in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sv.spec_verify(ctx, t["logits_draft"], t["logits_target"], t["draft_tokens"],
                       t["temperature"], 0, i, alen, toks)
        e1.record()
        outer.append((e0, e1))
    torch.cuda.synchronize()
    times = sv.spec_verify_read_timing(ctx, 4)
    assert len(times) == 4
    for (e0, e1), row in zip(outer, times):
        assert row[0] > 0 and row[2] > 0
        assert (row[1] > 0) == (batch >= 128)  # on the tile path the accept step is in the draw
        assert sum(row) <= e0.elapsed_time(e1) * 1.01 + 1e-3
    sv.spec_verify_destroy(ctx)


def test_first_rejection_in_a_later_pass():
    """G = 130: every position is accepted (identical rows) except position
    j*, where the target gives the draft token zero probability, so k = j*
    for certain; j* falls in the second and third passes of 64 positions and
    the residual draw runs on that position's rows."""
    rng = np.random.default_rng(11)
    G, V = 130, 800
    stars = [64, 100, 127, 128, 129]
    B = len(stars)
    base = rng.normal(0, 1.5, size=(G + 1, V)).astype(np.float32)
    zp = np.ascontiguousarray(np.broadcast_to(base, (B, G + 1, V))).copy()
    zq = np.ascontiguousarray(zp[:, :G]).copy()
    r2 = np.random.default_rng(12)
    toks = np.stack([specgen.gumbel_max_tokens(base[:G], 1.0, r2) for _ in range(B)])
    for b, j in enumerate(stars):
        zp[b, j, toks[b, j]] = -np.inf
    d = dict(logits_draft=zq, logits_target=zp, draft_tokens=toks,
             temperature=np.ones(B, np.float32), seq_ids=np.arange(B))
    gpu = run_gpu(to_device(d))
    ref = _oracle(d)
    assert list(ref["accept_len"]) == stars
    assert list(gpu["accept_len"]) == stars
    _check("first rejection in a later pass", gpu, d, ref=ref)
