"""Helpers shared by the GPU parity tests: device upload, one verification call
through the C ABI, and the comparison with the oracle under the match rules.

Match rules (the verification's tolerance):
* accept lengths and emitted tokens are compared exactly, except a decision the
  oracle itself takes with a log-margin below 1e-5: such a sequence is counted
  as "flagged" and excluded;
  - accept decisions: margin m_i = (lp_i - lq_i) - log u_i, any position
    i <= min(k_gpu, k_oracle);
  - the residual / bonus draw: margin = log-ratio distance of u * S to the
    edges of the chosen bin;
* greedy sequences (T == 0) and rejected sequences (-1) must match exactly;
* row log-normalisers: |lse_gpu - lse_oracle| <= 1e-5 * max(1, |lse_oracle|).
"""
from __future__ import annotations

import numpy as np
import torch

import device_draft_verification_amd as sv

MARGIN = 1e-5
LSE_REL = 1e-5


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


def compare(gpu: dict, ref: dict, temperature, rows=None, check_lse=True):
    """Compare GPU outputs (indexed by `rows`, default all) with oracle outputs
    of the same sequences. Returns a report dict; report["fails"] lists the
    sequences that break the match rules."""
    temperature = np.asarray(temperature)
    n = len(ref["accept_len"])
    rows = np.arange(n) if rows is None else np.asarray(rows)
    rep = dict(n=n, exact=0, flagged_accept=0, flagged_resample=0, fails=[],
               lse_max_abs=0.0, lse_max_rel=0.0)
    G = ref["tokens"].shape[1] - 1
    for j in range(n):
        b = rows[j]
        gl, rl = int(gpu["accept_len"][b]), int(ref["accept_len"][j])
        gt, rt = gpu["tokens"][b], ref["tokens"][j]
        greedy = temperature[j] == 0
        if gl == rl and np.array_equal(gt, rt):
            rep["exact"] += 1
        elif gl == rl and rl >= 0:
            k = rl
            prefix_ok = np.array_equal(gt[:k], rt[:k]) and np.all(gt[k + 1:] == -1)
            if prefix_ok and not greedy and ref["res_margin"][j] < MARGIN:
                rep["flagged_resample"] += 1
            else:
                rep["fails"].append((int(b), "token", gl, gt.tolist(), rt.tolist(),
                                     float(ref["res_margin"][j])))
        else:
            if gl < 0 or rl < 0 or greedy or G == 0:
                rep["fails"].append((int(b), "length", gl, rl, gt.tolist(), rt.tolist()))
                continue
            k = min(gl, rl)
            m = np.abs(ref["acc_margin"][j, :k + 1])
            if np.any(m < MARGIN):
                rep["flagged_accept"] += 1
            else:
                rep["fails"].append((int(b), "accept", gl, rl, float(np.nanmin(m))))
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
    assert rep["lse_max_rel"] <= LSE_REL, f"{label}: LSE rel err {rep['lse_max_rel']}"
