"""Helpers of the GPU parity tests: seeded inputs, oracle expectations, the
library call, and the comparison rule.

Comparison rule (reading R14 of the design doc): accepted lengths, emitted tokens
and status must match the oracle exactly on every sequence that is not
flagged (a uniform within 1e-6 of a decision threshold); disagreements are
allowed only on flagged sequences and must stay below 0.01% of the sequences
checked; the normalised distribution of the last draw must match within 1e-5
absolute on every sequence.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle.verify as ov
from draft_token_verification_softmax_amd import SV_MODE_SAMPLE, SV_MODE_TREE_GREEDY, SpecVerify
from draft_token_verification_softmax_amd import workloads as wl

RESID_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(arr: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def draw_drafts(inp, check=None, planted=None):
    """The draft model's tokens: x[b, j] ~ q'_j drawn with the workload's own
    uniforms (via the oracle's adjusted distribution) for the sequences in
    `check`; the draft row's argmax elsewhere (cheap, always in q's support).
    planted: optional probability of replacing x by the target's argmax
    (greedy tests)."""
    B, k = inp["u"].shape
    d64 = wl.rows_f64(inp["draft"], inp["dtype"])
    x = np.zeros((B, k), dtype=np.int32)
    for b in range(B):
        for j in range(k):
            if check is None or b in check:
                q = ov.transform_row(d64[b, j], inp["T"], inp["top_k"], inp["top_p"])
                x[b, j] = ov.draw_from(q, inp["draw_u"][b, j])
            else:
                x[b, j] = int(np.argmax(d64[b, j]))
    return x


def run_chain(inp, x, mode, want_resid=None, B=None, max_batch=None):
    B = inp["target"].shape[0] if B is None else B
    k = x.shape[1]
    V = inp["target"].shape[-1]
    sample = mode == SV_MODE_SAMPLE
    if want_resid is None:
        want_resid = sample
    sv = SpecVerify(mode=mode, dtype=inp["dtype"], max_batch=max(B, 1) if max_batch is None else max_batch,
                    k=k, vocab=V,
                    temperature=inp.get("T", 1.0), top_k=inp.get("top_k", 0),
                    top_p=inp.get("top_p", 1.0))
    tgt = dev(inp["target"][:B], inp["dtype"])
    dft = dev(inp["draft"][:B], inp["dtype"]) if sample else None
    xt = dev(x[:B].astype(np.int32))
    u = dev(inp["u"][:B]) if sample else None
    ur = dev(inp["ur"][:B]) if sample else None
    out = sv.run(tgt, dft, xt, u, ur, want_resid_probs=want_resid)
    torch.cuda.synchronize()
    res = {key: (v.cpu().numpy() if v is not None else None) for key, v in out.items()}
    sv.close()
    return res


def oracle_chain(inp, x, mode, idx):
    T64 = wl.rows_f64(inp["target"][idx], inp["dtype"])
    D64 = wl.rows_f64(inp["draft"][idx], inp["dtype"]) if mode == SV_MODE_SAMPLE else None
    name = "sample" if mode == SV_MODE_SAMPLE else "greedy"
    acc, toks, st, flagged, resid = ov.run_chain_batch(
        name, T64, D64, x[idx], inp["u"][idx], inp["ur"][idx], inp.get("T", 1.0),
        inp.get("top_k", 0), inp.get("top_p", 1.0), want_resid=(mode == SV_MODE_SAMPLE))
    return dict(accepted_len=acc, out_tokens=toks, seq_status=st, flagged=flagged, resid=resid)


def compare_chain(gpu, orc, idx, label=""):
    """Apply the comparison rule; returns a small report dict."""
    idx = list(idx)
    mism, unflagged = [], []
    for r, b in enumerate(idx):
        same = (gpu["accepted_len"][b] == orc["accepted_len"][r]
                and np.array_equal(gpu["out_tokens"][b], orc["out_tokens"][r])
                and gpu["seq_status"][b] == orc["seq_status"][r])
        if not same:
            mism.append(b)
            if not orc["flagged"][r]:
                unflagged.append((b, int(gpu["accepted_len"][b]), gpu["out_tokens"][b].tolist(),
                                  int(gpu["seq_status"][b]), int(orc["accepted_len"][r]),
                                  orc["out_tokens"][r].tolist(), int(orc["seq_status"][r])))
    report = dict(checked=len(idx), mismatches=len(mism), flagged=int(np.sum(orc["flagged"])))
    if orc.get("resid") is not None and gpu.get("resid_probs") is not None:
        diff = np.abs(gpu["resid_probs"][idx].astype(np.float64) - orc["resid"])
        report["resid_max_abs"] = float(diff.max()) if diff.size else 0.0
    say(label, report)
    assert not unflagged, f"{label}: unflagged mismatches (b, gpu n, gpu toks, gpu st, orc n, orc toks, orc st): {unflagged[:5]}"
    assert len(mism) <= 1e-4 * len(idx), f"{label}: {len(mism)} flagged mismatches of {len(idx)}"
    if "resid_max_abs" in report:
        assert report["resid_max_abs"] <= RESID_TOL, report
    return report


def run_tree(tr, tokens, B=None):
    B = tr["target"].shape[0] if B is None else B
    N = tr["parents"].shape[1]
    V = tr["target"].shape[-1]
    sv = SpecVerify(mode=SV_MODE_TREE_GREEDY, dtype=tr["dtype"], max_batch=max(B, 1), k=N, vocab=V)
    out = sv.run(dev(tr["target"][:B], tr["dtype"]), draft_tokens=dev(tokens[:B].astype(np.int32)),
                 parents=dev(tr["parents"][:B].astype(np.int32)))
    torch.cuda.synchronize()
    res = {key: (v.cpu().numpy() if v is not None else None) for key, v in out.items()}
    sv.close()
    return res


def tree_tokens_via_oracle(tr):
    T64 = wl.rows_f64(tr["target"], tr["dtype"])
    g = np.argmax(T64, axis=-1)   # first maximal index, the tie rule the oracle uses
    return wl.tree_tokens(tr, g), T64
