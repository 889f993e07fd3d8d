"""Helpers shared by the GPU parity tests: device upload, one verification call
through the C ABI, the comparison with the oracle under the match rules, and
the record of the per-case counts.

Match rules (the verification's tolerance):
* accept lengths and emitted tokens are compared exactly. The only exceptions
  are decisions the oracle itself takes with a log-margin below 1e-5, and even
  then the GPU's answer must be the other valid one:
  - an accept decision at the position where the two lengths part,
    i = min(k_gpu, k_oracle), with |(lp_i - lq_i) - log u_i| < 1e-5. The GPU's
    emitted prefix must still be its drafts up to its own k, its pads -1, and
    its extra token the oracle's draw at that k (or, when that draw itself has a
    margin below 1e-5, the token across the nearer bin edge);
  - the residual / bonus draw at the same k, with the oracle's log-margin (the
    log-ratio distance of u * S to the chosen bin's edges) below 1e-5: the
    GPU's token must be the one across the nearer edge, which has positive
    residual mass.
  Each such sequence is counted as excused; counts of excusals never exceed the
  oracle's own low-margin decisions, which are counted beside them;
* greedy sequences (T == 0) and rejected sequences (-1) must match exactly;
* every sequence must be well formed whatever the oracle says: accept length
  in [0, G] (or -1 with all tokens -1), drafts up to k, a token in [0, V) at
  k, -1 after;
* row log-normalisers: |lse_gpu - lse_oracle| <= 1e-5 * max(1, |lse_oracle|).
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import device_draft_verification_amd as sv
import oracle

MARGIN = 1e-5
LSE_REL = 1e-5

_REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORD_PATH = os.environ.get("SPEC_PARITY_RECORD",
                             os.path.join(_REPO, "gpurun_out", "parity_counts.json"))


def to_device(d: dict, dev="cuda"):
    def logits(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)
    return dict(
        logits_draft=logits(d["logits_draft"]),
        logits_target=logits(d["logits_target"]),
        draft_tokens=torch.from_numpy(np.ascontiguousarray(d["draft_tokens"], np.int32)).to(dev),
        temperature=torch.from_numpy(np.ascontiguousarray(d["temperature"], np.float32)).to(dev),
    )


def run_gpu(t: dict, seed=0, offset=0, ctx=None, with_lse=True):
    zp = t["logits_target"]
    B, G1, V = zp.shape
    G = G1 - 1
    own = ctx is None
    if own:
        ctx = sv.spec_verify_init(B, G, V, zp.dtype)
    alen = torch.full((B,), -7, dtype=torch.int32, device=zp.device)
    toks = torch.full((B, G + 1), -7, dtype=torch.int32, device=zp.device)
    sv.spec_verify(ctx, t["logits_draft"] if G else None, zp, t["draft_tokens"] if G else None,
                   t["temperature"], seed, offset, alen, toks)
    out = dict()
    if with_lse:
        lse = torch.empty((B, 2 * G + 1), dtype=torch.float64, device=zp.device)
        sv.spec_verify_copy_lse(ctx, lse)
        torch.cuda.synchronize()
        out["lse"] = lse.cpu().numpy()
    torch.cuda.synchronize()
    out["accept_len"] = alen.cpu().numpy()
    out["tokens"] = toks.cpu().numpy()
    if own:
        sv.spec_verify_destroy(ctx)
    return out


def _well_formed(gl, gt, draft, G, V):
    """The output of one sequence is a valid verification outcome."""
    if gl == -1:
        return bool(np.all(gt == -1))
    if not 0 <= gl <= G:
        return False
    return (np.array_equal(gt[:gl], draft[:gl]) and 0 <= gt[gl] < V
            and bool(np.all(gt[gl + 1:] == -1)))


def _parted_outcome_valid(data, j, T, seed, offset, gl, rl, token) -> bool:
    """The GPU took the other side of the oracle's low-margin accept decision
    at position min(gl, rl). Its outcome is valid iff the oracle, taking that
    same side, reaches the GPU's length and draws its token (or the token
    across the nearer bin edge of a draw that has a margin below 1e-5)."""
    G = data["logits_target"].shape[1] - 1
    sid = int(data["seq_ids"][j]) if "seq_ids" in data else j
    if gl < rl:
        # rejected where the oracle accepted: the draw at gl decides
        u = oracle.uniform_res(seed, offset, sid, gl)
        qrow = data["logits_draft"][j, gl] if gl < G else None
        tok, tm, ta = oracle.draw_at(qrow, data["logits_target"][j, gl], T, u)
    else:
        # accepted where the oracle rejected: the oracle accepts position rl
        # too (u = 0) and runs on with its own uniforms
        words = [oracle.philox_words(seed, offset, sid, i) for i in range(G + 1)]
        ua = np.array([oracle.uniform24(int(w[0])) for w in words])
        ur = np.array([oracle.uniform24(int(w[1])) for w in words])
        ua[rl] = 0.0
        o = oracle.verify_sequence(data["logits_draft"][j], data["logits_target"][j],
                                   data["draft_tokens"][j], T, ua, ur)
        if o["accept_len"] != gl:
            return False
        tok, tm, ta = int(o["tokens"][gl]), o["res_margin"], o["res_alt"]
    return token == tok or (tm < MARGIN and ta >= 0 and token == ta)


def compare(gpu: dict, ref: dict, temperature, rows=None, check_lse=True, data=None,
            seed=0, offset=0):
    """Compare GPU outputs (indexed by `rows`, default all) with oracle outputs
    of the same sequences. `data` holds the inputs of those sequences (indexed
    like `ref`: logits_draft, logits_target, draft_tokens, seq_ids) and the
    call's (seed, offset); without it a parted accept length cannot be
    validated and is a failure. Returns a report dict; report["fails"] lists
    the sequences that break the match rules."""
    temperature = np.asarray(temperature)
    n = len(ref["accept_len"])
    rows = np.arange(n) if rows is None else np.asarray(rows)
    rep = dict(n=n, exact=0, excused_accept=0, excused_resample=0, fails=[],
               low_margin_accept=0, low_margin_resample=0, lse_max_abs=0.0, lse_max_rel=0.0)
    G = ref["tokens"].shape[1] - 1
    V = None if data is None else data["logits_target"].shape[-1]
    for j in range(n):
        b = rows[j]
        gl, rl = int(gpu["accept_len"][b]), int(ref["accept_len"][j])
        gt, rt = gpu["tokens"][b], ref["tokens"][j]
        greedy = temperature[j] == 0
        sampled_ok = rl >= 0 and not greedy
        if sampled_ok:
            am = np.abs(ref["acc_margin"][j])
            if np.any(am[~np.isnan(am)] < MARGIN):
                rep["low_margin_accept"] += 1
            if ref["res_margin"][j] < MARGIN:
                rep["low_margin_resample"] += 1
        if data is not None and not _well_formed(gl, gt, data["draft_tokens"][j], G, V):
            rep["fails"].append((int(b), "malformed", gl, gt.tolist()))
            continue
        if gl == rl and np.array_equal(gt, rt):
            rep["exact"] += 1
        elif gl == rl and sampled_ok:
            k = rl
            prefix_ok = np.array_equal(gt[:k], rt[:k]) and np.all(gt[k + 1:] == -1)
            alt = int(ref["res_alt"][j])
            if prefix_ok and ref["res_margin"][j] < MARGIN and alt >= 0 and gt[k] == alt:
                rep["excused_resample"] += 1
            else:
                rep["fails"].append((int(b), "token", gl, gt.tolist(), rt.tolist(),
                                     float(ref["res_margin"][j]), alt))
        else:
            if gl < 0 or rl < 0 or greedy or G == 0 or data is None:
                rep["fails"].append((int(b), "length", gl, rl, gt.tolist(), rt.tolist()))
                continue
            k = min(gl, rl)
            m = abs(float(ref["acc_margin"][j, k]))
            ok = m < MARGIN
            if ok:
                ok = _parted_outcome_valid(data, j, float(temperature[j]), seed, offset, gl, rl,
                                           int(gt[gl]))
            if ok:
                rep["excused_accept"] += 1
            else:
                rep["fails"].append((int(b), "accept", gl, rl, m, gt.tolist(), rt.tolist()))
        if check_lse and "lse" in gpu and rl >= 0 and not greedy:
            lg, lr = gpu["lse"][b], ref["lse"][j]
            ok = ~np.isnan(lr)
            if ok.any():
                err = np.abs(lg[ok] - lr[ok])
                rel = err / np.maximum(1.0, np.abs(lr[ok]))
                rep["lse_max_abs"] = max(rep["lse_max_abs"], float(err.max()))
                rep["lse_max_rel"] = max(rep["lse_max_rel"], float(rel.max()))
    return rep


def assert_parity(rep: dict, label=""):
    assert not rep["fails"], f"{label}: {len(rep['fails'])} mismatches, first {rep['fails'][:3]}"
    assert rep["excused_accept"] <= rep["low_margin_accept"], label
    assert rep["excused_resample"] <= rep["low_margin_resample"], label
    assert rep["lse_max_rel"] <= LSE_REL, f"{label}: LSE rel err {rep['lse_max_rel']}"


def record(label: str, rep: dict, **extra):
    """Print one comparison's counts and add them to the JSON record (one
    entry per label, rewritten by a later run of the same case)."""
    row = dict(compared=rep["n"], exact=rep["exact"], excused_accept=rep["excused_accept"],
               excused_resample=rep["excused_resample"], mismatched=len(rep["fails"]),
               oracle_low_margin_accept=rep["low_margin_accept"],
               oracle_low_margin_resample=rep["low_margin_resample"],
               lse_max_abs=rep["lse_max_abs"], lse_max_rel=rep["lse_max_rel"], **extra)
    print(f"\n[{label}] " + " ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
                                   for k, v in row.items()), flush=True)
    try:
        os.makedirs(os.path.dirname(RECORD_PATH), exist_ok=True)
        try:
            with open(RECORD_PATH) as f:
                doc = json.load(f)
        except (OSError, ValueError):
            doc = {}
        doc[label] = row
        tmp = RECORD_PATH + ".tmp"
        with open(tmp, "w") as f:
            json.dump(doc, f, indent=1, sort_keys=True)
        os.replace(tmp, RECORD_PATH)
    except OSError as e:  # the record is a by-product; the assertions decide
        print(f"parity record not written: {e}", flush=True)
