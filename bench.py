"""Throughput of batched speculative-sampling verification on one MI355X.

One step = one spec_verify call (row normalisers, accept, residual draw) over
the B=256, gamma=8, V=152064 bf16 workload (target correlated rho=0.8 with the
draft, per-sequence temperature U[0.3, 1.5], 10 % greedy sequences), inputs
resident in HBM before the timed region. Three copies of the inputs are
rotated so no step finds the previous step's rows in the 256 MB last-level
cache. Before the W warm-up steps, untimed calls run for --settle-ms (300 ms
by default) so that the timed steps see settled clocks; the timed region is
exactly K steps. Prints one JSON line. The further sections (outcome law,
low-rank head, trees) each run their operation untimed for
--section-settle-ms (40 ms by default) and W times before their K timed calls.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms T]
                    [--section-settle-ms T] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified sequences/sec and achieved HBM GB/s (% of peak) at B×(γ+1)×V"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
WORKLOAD_CONFIG = 4
# Counter records (rocprofv3 FETCH_SIZE / WRITE_SIZE of the B=256 workload's
# kernels) and the sources each depends on: a record no longer matching its
# sources is reported as null.
_CSRC = "device_draft_verification_amd/csrc/"
TRAFFIC = {
    "row_norm": dict(kernel="row_norm_kernel",
                     file=os.path.join(ROOT, "profiles", "rownorm_B256_g8_V152064_traffic.json"),
                     sources=[_CSRC + "rownorm.hip", _CSRC + "common.hpp", _CSRC + "launch.hpp"]),
    "residual": dict(kernel="residual_fused_kernel",
                     file=os.path.join(ROOT, "profiles", "residual_B256_g8_V152064_traffic.json"),
                     sources=[_CSRC + "residual.hip", _CSRC + "accept.hpp", _CSRC + "philox.hpp",
                              _CSRC + "common.hpp", _CSRC + "launch.hpp"]),
}
PROBE_BYTES = 1 << 30   # read-only probe buffer: four times the last-level cache
PROBE_BLOCKS = 8192


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(name: str = "row_norm") -> str:
    h = hashlib.sha256()
    for rel in TRAFFIC[name]["sources"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(rec, temperature: np.ndarray, accept_len: np.ndarray) -> dict:
    """Bytes each kernel must move for one call (see the kernel headers):
    row normalisers read (2G+1) rows per sampled sequence and G+1 target rows
    per greedy one; the residual kernel reads 2 rows after a rejection, the
    bonus row after a full accept, nothing for greedy sequences; the accept
    kernel gathers 2 logits per position and writes the outcome."""
    s = 2 if rec.dtype == "bf16" else 4
    G, V = rec.gamma, rec.vocab
    sampled = temperature > 0
    greedy = temperature == 0
    k1 = int(sampled.sum()) * (2 * G + 1) * V * s + int(greedy.sum()) * (G + 1) * V * s
    valid = accept_len >= 0
    rejected = sampled & valid & (accept_len < G)
    bonus = sampled & valid & (accept_len == G)
    k3 = int(rejected.sum()) * 2 * V * s + int(bonus.sum()) * V * s
    k2 = rec.batch * (2 * G * s + 4 * G + 4 + 4 * (G + 2))
    return dict(row_norm=k1, accept=k2, residual=k3)


def cpu_baseline(rec, d, budget_s: float = 10.0, cap_s: float = 30.0) -> dict:
    """The oracle, single-threaded, one call per sequence over the same inputs
    (sequence b, offset = pass number), until at least budget_s seconds of CPU
    work have been spent (whole passes over the batch, at most cap_s)."""
    import oracle
    oracle._load()
    n = 0
    passes = 0
    t0 = time.perf_counter()
    while True:
        for b in range(rec.batch):
            sl = slice(b, b + 1)
            oracle.verify(d["logits_draft"][sl], d["logits_target"][sl], d["draft_tokens"][sl],
                          d["temperature"][sl], seed=0, offset=passes, seq_ids=d["seq_ids"][sl])
            n += 1
            if time.perf_counter() - t0 > cap_s:
                break
        passes += 1
        if time.perf_counter() - t0 > budget_s or time.perf_counter() - t0 > cap_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "sequences/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} sequence verifications ({passes} passes over the {rec.batch} "
                      f"sequences of the {rec.name} workload, one oracle call per sequence), "
                      f"{dt:.1f} s on one host core",
            "host_cpu": host_cpu_model(), "nproc": os.cpu_count()}


def tree_sample_bytes(parent, M, length, path, temperature, row_bytes) -> int:
    """Rows one sampled tree walk must read, from its outcome: at each visited
    node the target row (its normaliser, or the argmax at T = 0) and, when it
    has children, the draft row; two rows per rejected child (children are
    tried in node order, so those before the accepted one, and all of the
    last node's); one more row for the final draw when nothing was rejected at
    the last node (a rejection leaves that draw's tile sums ready)."""
    total = 0
    for b in range(parent.shape[0]):
        L = int(length[b])
        if L < 0:
            continue
        nodes = [0] + [int(x) for x in path[b, :L]]
        for i, u in enumerate(nodes):
            kids = [s for s in range(1, M) if parent[b, s] == u]
            total += row_bytes
            if temperature[b] == 0:
                continue
            if kids:
                total += row_bytes
            nxt = nodes[i + 1] if i + 1 < len(nodes) else None
            rejected = [s for s in kids if nxt is None or s < nxt]
            total += 2 * row_bytes * len(rejected)
            if nxt is None and not rejected:
                total += row_bytes
    return total


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_next_rows(rec, d, host: dict, F: int) -> dict:
    """The oracle of each further row, single-threaded, on a bounded sample of
    the same work the GPU lines above time (a few seconds each)."""
    import oracle
    oracle._load()
    B, G = rec.batch, rec.gamma
    res = {}

    def timed(fn, reps=1):
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        return (time.perf_counter() - t0) / reps

    n_seq = min(2, B)
    dt = timed(lambda: oracle.outcomes(d["logits_draft"][:n_seq], d["logits_target"][:n_seq],
                                       d["draft_tokens"][:n_seq], d["temperature"][:n_seq], F))
    res["outcomes"] = {"us_per_sequence": round(dt / n_seq * 1e6, 1),
                       "sample": f"outcome law with F = {F} for {n_seq} sequences of the workload"}
    if "fanout" in host:
        fx = host["fanout"]
        dt = timed(lambda: oracle.outcome_fanout(fx["pk"], fx["probs"], fx["budget"]), reps=5)
        res["outcome_fanout"] = {"us_per_call": round(dt * 1e6, 1),
                                 "sample": f"cache budget of {fx['budget']} entries for all "
                                           f"{fx['pk'].shape[0]} sequences of the workload"}
    if "head" in host:
        hx = host["head"]
        rows = [r for r in (0, 1) if r < hx["h"].shape[0]]
        dt = timed(lambda: oracle.lowrank_head(hx["h"], hx["w_down"], hx["w_up"],
                                               hx["temperature"], rows=rows))
        res["lowrank_head"] = {"us_per_row": round(dt / len(rows) * 1e6, 1),
                               "sample": f"{len(rows)} rows of the N = {hx['h'].shape[0]} head"}
    if "tree" in host:
        tr = host["tree"]
        pr = tr["prune"]
        dt = timed(lambda: oracle.tree_prune(pr["parent"], pr["logq"], float(np.log(1e-3)), 32), 3)
        res["tree_prune"] = {"us_per_call": round(dt * 1e6, 1),
                             "sample": f"{pr['parent'].shape[0]} trees of {pr['parent'].shape[1]} nodes"}
        vt, nt = tr["verify"], tr["target"].shape[0]
        if "draft" in tr:
            temp4 = d["temperature"][:nt]
            dt_s = timed(lambda: oracle.tree_verify_sample(vt["parent"][:nt], vt["token"][:nt],
                                                           np.full(nt, tr["n"], np.int32),
                                                           tr["draft"], tr["target"], temp4))
            res["tree_sample"] = {"us_per_tree": round(dt_s / nt * 1e6, 1),
                                  "sample": f"{nt} trees of {tr['n']} nodes, sampled rule"}
        n_nodes = np.full(nt, tr["n"], np.int32)
        dt = timed(lambda: oracle.tree_verify_greedy(vt["parent"][:nt], vt["token"][:nt], n_nodes,
                                                     tr["target"]))
        res["tree_verify"] = {"us_per_tree": round(dt / nt * 1e6, 1),
                              "sample": f"{nt} trees of {tr['n']} nodes"}
    if G > 0:
        al = np.minimum(np.arange(B, dtype=np.int32) % (G + 1), G)
        for name, pol in (("ucb1", oracle.UCB1), ("thompson", oracle.THOMPSON)):
            bd = oracle.Bandit(pol, B, 3, B, G)
            arm, _ = bd.step(seed=1, offset=0)
            reps = 200
            t0 = time.perf_counter()
            for i in range(reps):
                arm, _ = bd.step(al, arm, seed=1, offset=i + 1)
            res[f"bandit_{name}_groups{B}"] = {
                "us_per_step": round((time.perf_counter() - t0) / reps * 1e6, 1),
                "sample": f"{reps} steps, {B} groups of 3 arms"}
    return res


COPY_BYTES = 1 << 30


def _counter_rows(path: str, counter: str):
    import csv
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                yield r


def derive_traffic(fetch_csv: str, write_csv: str) -> int:
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each kernel in TRAFFIC
    found in the two counter runs, each scaled by what the same counter reads
    for the 1 GiB calibration copy (which moves exactly COPY_BYTES each way)."""
    def per_kernel(path, counter, kernel):
        rows = list(_counter_rows(path, counter))
        # sum over the counter's instances per dispatch
        by_dispatch = {}
        for r in rows:
            key = (r["Dispatch_Id"], r["Kernel_Name"], int(r.get("Grid_Size", 0) or 0))
            by_dispatch[key] = by_dispatch.get(key, 0.0) + float(r["Counter_Value"])
        ks = [v for (d, name, g), v in by_dispatch.items() if kernel in name]
        # the calibration copy is the largest device-to-device copy of the run
        copies = [v for (d, name, g), v in by_dispatch.items() if "copyBuffer" in name]
        copy_kib = max(copies) if copies else None
        return (sum(ks) / len(ks) if ks else None), copy_kib
    written = 0
    for name, t in TRAFFIC.items():
        fk, fc = per_kernel(fetch_csv, "FETCH_SIZE", t["kernel"])
        wk, wc = per_kernel(write_csv, "WRITE_SIZE", t["kernel"])
        if fk is None or wk is None or not fc or not wc:
            continue
        f_scale = COPY_BYTES / (fc * 1024.0)
        w_scale = COPY_BYTES / (wc * 1024.0)
        rec = {"kernel": t["kernel"], "workload": "B256_g8_V152064_bf16_corr",
               "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
               "copy_fetch_kib": fc, "copy_write_kib": wc, "copy_bytes": COPY_BYTES,
               "fetch_scale": f_scale, "write_scale": w_scale,
               "hbm_bytes_per_launch": int(round(fk * 1024.0 * f_scale + wk * 1024.0 * w_scale)),
               "kernel_source_hash": kernel_source_hash(name)}
        os.makedirs(os.path.dirname(t["file"]), exist_ok=True)
        with open(t["file"], "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        written += 1
    return 0 if written else 1


def load_traffic(name: str = "row_norm"):
    """HBM bytes per launch of a kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs, or None when its sources have changed since
    they were taken."""
    path = TRAFFIC[name]["file"]
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(name):
        return None
    return int(t["hbm_bytes_per_launch"])


def hbm_probe(sv, torch, dev, stream, reps: int = 20) -> dict:
    """The read-only probe over a 1 GiB buffer: the practical read ceiling of
    this device, reported beside the vendor figure."""
    buf = torch.ones(PROBE_BYTES // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(PROBE_BLOCKS, dtype=torch.int32, device=dev)
    for _ in range(3):
        sv.spec_hbm_read_probe(buf, sink, PROBE_BLOCKS, stream=stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        sv.spec_hbm_read_probe(buf, sink, PROBE_BLOCKS, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])
    del buf, sink
    return {"bytes": PROBE_BYTES, "us_median": round(float(np.median(us)), 2),
            "gbs": round(PROBE_BYTES / (float(np.median(us)) * 1e-6) / 1e9, 1),
            "blocks": PROBE_BLOCKS, "reps": reps}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--workload", type=int, default=WORKLOAD_CONFIG, choices=[1, 2, 3, 4, 5],
                    help="which of the five workloads to time (default: the B=256 one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed verification calls for about this long before the warm-up "
                         "steps, so that the timed steps run at the clocks of sustained work "
                         "rather than during the ramp from idle")
    ap.add_argument("--section-settle-ms", type=float, default=40.0,
                    help="untimed calls of each further section's operation (outcome law, "
                         "head, trees) for about this long before its warm-up calls")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device-to-device copy first (counter calibration)")
    ap.add_argument("--derive-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) "
                         "into the traffic record under profiles/ and exit")
    args = ap.parse_args()
    if args.derive_traffic:
        return derive_traffic(*args.derive_traffic)
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library's verification path runs "
              "on a single device (multi-GPU sharding is not built)", file=sys.stderr)
        return 2

    import torch
    import device_draft_verification_amd as sv
    import specgen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    sv.load_library()
    dev = torch.device("cuda:0")
    rec = specgen.config(args.workload)
    B, G, V = rec.batch, rec.gamma, rec.vocab
    t0 = time.perf_counter()
    d = specgen.generate(rec)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    draft0, target0 = to_dev(d["logits_draft"]), to_dev(d["logits_target"])
    copies = [(draft0, target0)] + [(draft0.clone(), target0.clone()) for _ in range(args.copies - 1)]
    tokens = torch.from_numpy(d["draft_tokens"]).to(dev)
    temp = torch.from_numpy(d["temperature"]).to(dev)
    alen = torch.empty(B, dtype=torch.int32, device=dev)
    toks = torch.empty(B, G + 1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    ctx = sv.spec_verify_init(B, G, V, target0.dtype, stream=stream)
    geo = sv.spec_verify_get_geometry(ctx)

    def step(i):
        zq, zp = copies[i % len(copies)]
        sv.spec_verify(ctx, zq, zp, tokens, temp, 0, i, alen, toks)

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # Clock settling: untimed calls before the warm-up. Measured on this part,
    # a run of 5 warm-up and 20 timed steps from idle saw the row kernel at
    # 199-209 us and the residual draw at 27.5-28.8 us, against 187 and 25.6 us
    # once the clocks had settled; the JSON line reports what was run.
    settle_calls = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(16):
            step((1 << 40) + settle_calls)
            settle_calls += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3

    def warm(fn):
        """Untimed calls of a further section's operation: --section-settle-ms
        of them (indices from 2^40 up), then the W warm-up calls (indices 0 ..
        W - 1), so that its timed calls see the clocks of its own sustained
        work, as the verification steps do."""
        t0, n = time.perf_counter(), 0
        while (time.perf_counter() - t0) * 1e3 < args.section_settle_ms:
            for _ in range(4):
                fn((1 << 40) + n)
                n += 1
            torch.cuda.synchronize()
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K steps, bracketed by events on the launch stream.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    # The same K steps again, right after the timed region (same clocks), with
    # the library's per-kernel HIP events recorded on the stream the kernels
    # are launched on (each event adds a few us between kernels, so the step
    # time above is taken without them).
    sv.spec_verify_enable_timing(ctx, args.steps)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(args.warmup + i)
    per_kernel = np.array(sv.spec_verify_read_timing(ctx, args.steps))  # [K, 3] ms
    sv.spec_verify_enable_timing(ctx, 0)
    k1_med, k3_med = float(np.median(per_kernel[:, 0])), float(np.median(per_kernel[:, 2]))

    # Distribution of single calls: each bracketed by its own event pair.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(args.steps, 100))]
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        step(args.warmup + i)
        e1.record(stream)
    torch.cuda.synchronize()
    call_us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])

    # Scalar-only mode at B = 512, gamma = 4 (the [512, 4, 2] fp32 pairs the
    # B=512 workload specifies); the pair values do not change the work.
    sc_b, sc_g = 512, 4
    sc_ctx = sv.spec_verify_init(sc_b, sc_g, 8, torch.float32, stream=stream)
    sc_lp = torch.randn(sc_b, sc_g, 2, device=dev) - 2.0
    sc_out = torch.empty(sc_b, dtype=torch.int32, device=dev)
    for i in range(args.warmup):
        sv.spec_accept_logprobs(sc_ctx, sc_lp, 0, i, sc_out)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        sv.spec_accept_logprobs(sc_ctx, sc_lp, 0, i, sc_out)
    end.record(stream)
    torch.cuda.synchronize()
    scalar_us = start.elapsed_time(end) * 1e3 / args.steps
    sv.spec_verify_destroy(sc_ctx)

    # Online draft selection (K = 3 draft models): one spec_bandit_step per
    # decoding step, reading the last call's accept lengths on the device.
    # Launch-latency bound (a few hundred bytes); reported in us per step.
    step(0)
    bandit_us = {}
    for pol_name, pol in (("ucb1", sv.SPEC_BANDIT_UCB1), ("thompson", sv.SPEC_BANDIT_THOMPSON)):
        for groups in (1, B):
            bctx = sv.spec_bandit_init(groups, 3, B, G, pol, stream=stream) if G > 0 else None
            if bctx is None:
                continue
            arm = torch.zeros(groups, dtype=torch.int32, device=dev)
            sv.spec_bandit_step(bctx, None, None, 1, 0, arm)
            for i in range(args.warmup):
                sv.spec_bandit_step(bctx, alen, arm, 1, i + 1, arm)
            torch.cuda.synchronize()
            start.record(stream)
            for i in range(args.steps):
                sv.spec_bandit_step(bctx, alen, arm, 1, args.warmup + i + 1, arm)
            end.record(stream)
            torch.cuda.synchronize()
            bandit_us[f"{pol_name}_groups{groups}"] = round(start.elapsed_time(end) * 1e3 / args.steps, 2)
            sv.spec_bandit_destroy(bctx)


    # Algorithmic bytes per call: outputs are a pure function of (inputs, seed,
    # offset), so each timed call's accept lengths are recomputed untimed.
    k1_bytes = k3_bytes = k2_bytes = 0
    for i in range(args.steps):
        step(args.warmup + i)
        torch.cuda.synchronize()
        ab = algorithmic_bytes(rec, d["temperature"], alen.cpu().numpy())
        k1_bytes += ab["row_norm"]
        k2_bytes += ab["accept"]
        k3_bytes += ab["residual"]
    k1_bytes /= args.steps
    k2_bytes /= args.steps
    k3_bytes /= args.steps
    k1_ms, k2_ms, k3_ms = per_kernel.mean(axis=0)

    # Verification-outcome law with F = 16 tokens per length, after a call on
    # input copy 0: one more pass over the same logits the row kernel reads.
    F_OUT = 16
    o_tok = torch.empty(B, G + 1, F_OUT, dtype=torch.int32, device=dev)
    o_prob = torch.empty(B, G + 1, F_OUT, dtype=torch.float32, device=dev)
    o_pk = torch.empty(B, G + 1, dtype=torch.float32, device=dev)
    o_mass = torch.empty(B, G + 1, dtype=torch.float32, device=dev)
    step(0)
    zq0, zp0 = copies[0]

    def outcomes():
        sv.spec_verify_outcomes(ctx, zq0 if G else None, zp0, tokens if G else None, F_OUT,
                                o_tok, o_prob, o_pk, o_mass)

    warm(lambda i: outcomes())
    start.record(stream)
    for _ in range(args.steps):
        outcomes()
    end.record(stream)
    torch.cuda.synchronize()
    outcome_ms = start.elapsed_time(end) / args.steps
    outcome_bytes = algorithmic_bytes(rec, d["temperature"], alen.cpu().numpy())["row_norm"]
    outcome_gbs = outcome_bytes / (outcome_ms * 1e-3) / 1e9

    # Speculation-cache budget per length from that law: FANOUT_BUDGET entries
    # per sequence (no figure on the pages; 64 is four per length at G = 8, in
    # units of the lists' F = 16).
    FANOUT_BUDGET = 64
    f_n = torch.empty(B, G + 1, dtype=torch.int32, device=dev)
    f_hit = torch.empty(B, dtype=torch.float64, device=dev)

    def fanout():
        sv.spec_outcome_fanout(o_pk, o_prob, FANOUT_BUDGET, f_n, f_hit, stream)

    outcomes()
    warm(lambda i: fanout())
    start.record(stream)
    for _ in range(args.steps):
        fanout()
    end.record(stream)
    torch.cuda.synchronize()
    fanout_ms = start.elapsed_time(end) / args.steps
    fanout_hit = f_hit.cpu().numpy()

    # Low-rank draft head for one draft step of this batch: N = B rows,
    # hidden d = 4096, rank r = d / 8 = 512 (the pages' example ratio), this
    # workload's vocabulary; random bf16 weights made on the device.
    hd, hr = 4096, 512
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    hh = torch.randn(B, hd, device=dev, generator=gen).to(torch.bfloat16)
    wd = (torch.randn(hr, hd, device=dev, generator=gen) / hd ** 0.5).to(torch.bfloat16)
    wu = (torch.randn(V, hr, device=dev, generator=gen) * (2.5 / hr ** 0.5)).to(torch.bfloat16)
    hz = torch.empty(B, V, dtype=torch.bfloat16, device=dev)
    hl = torch.empty(B, dtype=torch.float64, device=dev)
    hctx = sv.spec_lowrank_head_init(B, hd, hr, V, stream=stream)
    warm(lambda i: sv.spec_lowrank_head(hctx, hh, wd, wu, temp, hz, hl))
    start.record(stream)
    for _ in range(args.steps):
        sv.spec_lowrank_head(hctx, hh, wd, wu, temp, hz, hl)
    end.record(stream)
    torch.cuda.synchronize()
    head_ms = start.elapsed_time(end) / args.steps
    head_bytes = 2 * (V * hr + B * V + hr * hd + B * hd)
    head_flops = 2 * B * (hd * hr + hr * V)
    sv.spec_lowrank_head_destroy(hctx)
    host = {}
    if not args.no_cpu_baseline:
        host["fanout"] = dict(pk=o_pk.cpu().numpy(), probs=o_prob.cpu().numpy(),
                              budget=FANOUT_BUDGET)
        bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
        host["head"] = dict(h=bits(hh), w_down=bits(wd), w_up=bits(wu),
                            temperature=d["temperature"][:B].copy())
    del hh, wd, wu, hz

    # Draft trees of this batch and vocabulary: pruning 64-node trees, and
    # greedy verification of 16-node trees (target rows read once by the
    # argmax pass; random bf16 logits made on the device).
    tp = specgen.draft_trees(B, 64, V, seed=1)
    t_par, t_lq = torch.from_numpy(tp["parent"]).to(dev), torch.from_numpy(tp["logq"]).to(dev)
    p_cum = torch.empty(B, 64, dtype=torch.float64, device=dev)
    p_ni = torch.empty(B, 64, dtype=torch.int32, device=dev)
    p_np = torch.empty(B, 64, dtype=torch.int32, device=dev)
    p_cnt = torch.empty(B, dtype=torch.int32, device=dev)

    def prune():
        sv.spec_tree_prune(t_par, t_lq, float(np.log(1e-3)), 32, p_cum, p_ni, p_np, p_cnt,
                           stream=stream)

    warm(lambda i: prune())
    start.record(stream)
    for _ in range(args.steps):
        prune()
    end.record(stream)
    torch.cuda.synchronize()
    prune_us = start.elapsed_time(end) * 1e3 / args.steps
    tm = 16
    tv = specgen.draft_trees(B, tm, V, seed=2)
    v_par, v_tok = torch.from_numpy(tv["parent"]).to(dev), torch.from_numpy(tv["token"]).to(dev)
    v_n = torch.full((B,), tm, dtype=torch.int32, device=dev)
    v_tgt = (torch.randn(B, tm, V, device=dev, generator=gen) * 2.5).to(torch.bfloat16)
    v_len = torch.empty(B, dtype=torch.int32, device=dev)
    v_path = torch.empty(B, tm, dtype=torch.int32, device=dev)
    v_extra = torch.empty(B, dtype=torch.int32, device=dev)
    tctx = sv.spec_tree_verify_init(B, tm, V, torch.bfloat16, stream=stream)
    warm(lambda i: sv.spec_tree_verify_greedy(tctx, v_par, v_tok, v_n, v_tgt, v_len, v_path, v_extra))
    start.record(stream)
    for _ in range(args.steps):
        sv.spec_tree_verify_greedy(tctx, v_par, v_tok, v_n, v_tgt, v_len, v_path, v_extra)
    end.record(stream)
    torch.cuda.synchronize()
    tree_ms = start.elapsed_time(end) / args.steps
    tree_bytes = B * tm * V * 2
    # Sampled verification of the same trees (multi-step speculative
    # sampling) at the workload's temperatures, with random bf16 draft rows.
    v_q = (torch.randn(B, tm, V, device=dev, generator=gen) * 2.5).to(torch.bfloat16)
    warm(lambda i: sv.spec_tree_verify_sample(tctx, v_par, v_tok, v_n, v_q, v_tgt, temp, 0, i,
                                              v_len, v_path, v_extra))
    start.record(stream)
    for i in range(args.steps):
        sv.spec_tree_verify_sample(tctx, v_par, v_tok, v_n, v_q, v_tgt, temp, 0, args.warmup + i,
                                   v_len, v_path, v_extra)
    end.record(stream)
    torch.cuda.synchronize()
    tree_s_ms = start.elapsed_time(end) / args.steps
    tree_s_bytes = tree_sample_bytes(tv["parent"], tm, v_len.cpu().numpy(), v_path.cpu().numpy(),
                                     d["temperature"], V * 2)
    host_tree_draft = v_q[:4].view(torch.int16).cpu().numpy().view(np.uint16)
    del v_q
    sv.spec_tree_verify_destroy(tctx)
    if not args.no_cpu_baseline:
        host["tree"] = dict(prune=tp, verify=tv, n=tm,
                            target=v_tgt[:4].view(torch.int16).cpu().numpy().view(np.uint16),
                            draft=host_tree_draft)
    del v_tgt
    k1_gbs = k1_bytes / (k1_ms * 1e-3) / 1e9
    k3_gbs = k3_bytes / (k3_ms * 1e-3) / 1e9
    call_gbs = (k1_bytes + k2_bytes + k3_bytes) / (ms_per_step * 1e-3) / 1e9
    value = B / (ms_per_step * 1e-3)
    log(f"per step {ms_per_step * 1e3:.1f} us: row_norm {k1_ms * 1e3:.1f} us ({k1_gbs:.0f} GB/s), "
        f"accept {k2_ms * 1e3:.1f} us, residual {k3_ms * 1e3:.1f} us ({k3_gbs:.0f} GB/s); "
        f"whole call {call_gbs:.0f} GB/s")

    on_workload = args.workload == WORKLOAD_CONFIG
    traffic = load_traffic("row_norm") if on_workload else None
    traffic_k3 = load_traffic("residual") if on_workload and geo["residual_splits"] == 0 else None
    probe = hbm_probe(sv, torch, dev, stream)
    pg = probe["gbs"]
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "sequences/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"calls": settle_calls, "ms": round(settle_ms, 1),
                   "section_ms": args.section_settle_ms},
        "ms_per_step": round(ms_per_step, 5),
        "call_us": {"median": round(float(np.median(call_us)), 2),
                    "p10": round(float(np.percentile(call_us, 10)), 2),
                    "p90": round(float(np.percentile(call_us, 90)), 2), "calls": int(call_us.size)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if rec.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": rec.name, "batch": B, "gamma": G, "vocab": V,
                   "logits": rec.dtype,
                   "greedy_fraction": round(float((d["temperature"] == 0).mean()), 3),
                   "parallelism": "none"},
        "hbm_gbs_whole_call": round(call_gbs, 1),
        "hbm_frac_whole_call": round(call_gbs / HBM_PEAK_GBS, 4),
        "kernels": {
            "row_norm": {"us": round(k1_ms * 1e3, 2), "us_median": round(k1_med * 1e3, 2),
                         "bytes": int(k1_bytes),
                         "gbs": round(k1_gbs, 1), "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
                         "frac_probe": round(k1_gbs / pg, 4), "traffic": traffic,
                         "splits": geo["row_splits"]},
            "accept": {"us": round(k2_ms * 1e3, 2), "bytes": int(k2_bytes)},
            "residual": {"us": round(k3_ms * 1e3, 2), "us_median": round(k3_med * 1e3, 2),
                         "bytes": int(k3_bytes),
                         "gbs": round(k3_gbs, 1), "frac": round(k3_gbs / HBM_PEAK_GBS, 4),
                         "frac_probe": round(k3_gbs / pg, 4), "traffic": traffic_k3,
                         "splits": geo["residual_splits"]},
        },
        "hbm_probe": probe,
        "scalar_mode": {"us_per_call": round(scalar_us, 2), "batch": sc_b, "gamma": sc_g,
                        "bytes": sc_b * sc_g * 8 + sc_b * 4,
                        "sequences_per_s": round(sc_b / (scalar_us * 1e-6), 1)},
        "bandit": {"arms": 3, "us_per_step": bandit_us},
        "tree": {"prune_nodes": 64, "prune_us": round(prune_us, 2), "verify_nodes": tm,
                 "verify_us": round(tree_ms * 1e3, 2), "verify_bytes": int(tree_bytes),
                 "verify_gbs": round(tree_bytes / (tree_ms * 1e-3) / 1e9, 1),
                 "verify_frac": round(tree_bytes / (tree_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "sample_us": round(tree_s_ms * 1e3, 2),
                 "sample_bytes_last_call": int(tree_s_bytes),
                 "sample_gbs": round(tree_s_bytes / (tree_s_ms * 1e-3) / 1e9, 1)},
        "lowrank_head": {"rows": B, "hidden": hd, "rank": hr, "vocab": V,
                         "us_per_call": round(head_ms * 1e3, 2), "bytes": int(head_bytes),
                         "gbs": round(head_bytes / (head_ms * 1e-3) / 1e9, 1),
                         "tflops": round(head_flops / (head_ms * 1e-3) / 1e12, 1),
                         "frac_hbm": round(head_bytes / (head_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "outcomes": {"top_f": F_OUT, "us_per_call": round(outcome_ms * 1e3, 2),
                     "bytes": int(outcome_bytes), "gbs": round(outcome_gbs, 1),
                     "frac": round(outcome_gbs / HBM_PEAK_GBS, 4),
                     "fanout": {"budget": FANOUT_BUDGET, "us_per_call": round(fanout_ms * 1e3, 2),
                                "hit_rate_mean": round(float(fanout_hit.mean()), 4)}},
        "roofline": {"bound": "hbm", "achieved": round(k1_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "row_norm_kernel"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(rec, d)
        out["cpu_baseline"]["rows"] = cpu_next_rows(rec, d, host, F_OUT)
    sv.spec_verify_destroy(ctx)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
