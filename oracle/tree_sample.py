"""Plain CPU oracle for modified rejection sampling over a token tree.

TEST INFRASTRUCTURE ONLY (same import rule as oracle/verify.py): only tests/,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
it.  It shares no code with the HIP library.

Source: the edgeinferencenotes.hashnode.dev speculative-decoding / EAGLE-3
article.  "One decode round, end to end": the draft grows a tree, the target
scores every node in one pass under an ancestor-only mask, the accept-or-
correct rule of "The core idea: draft, then check" is applied down the
branches, the single longest agreed path is committed and one correction is
resampled at the first rejected token; the emitted text follows the target
exactly ("Why it changes nothing about the output").

The pages do not say how several children of one node are tried.  Readings
(numbered as in the design doc):
  R24  multi-sibling rule.  At an accepted node u with adjusted target p'_u
       and draft q'_u (the distribution u's children were drawn from), the
       children of u (nodes whose parent is u) are tried in increasing index
       order against a running target r, initially p'_u:
         accept child c (token x) iff (q(x) > 0 and u_c < min(1, r(x)/q(x)))
                                   or (q(x) = 0 and r(x) > 0);
         on rejection r <- max(0, r - q'_u) renormalised (if that is all zero,
         r is left as it was).
       The first accepted child becomes the new node and the walk continues
       there; if no child is accepted, or u has none, the walk stops and one
       token y is drawn from r (inverse CDF with the tree's uniform, R8).
       With one child per node this is the chain rule exactly.  It keeps the
       emitted tokens distributed as the target when the children of a node
       are drawn independently from q'_u.
  R25  inputs.  Row i of the target is the target's distribution for node i's
       children, row i of the draft the draft's; u[i] is node i's uniform
       (u[0] unused); one uniform ur per tree.  Adjustments (temperature,
       top-k, top-p) as reading R5 on every row used.
  R26  bad data.  A token outside [0, V) is rejected like any other
       rejection (status bit 1).  A node whose parent index is not in [0, i)
       is never a child of anything (status bit 2); node 0 is the root
       whatever parents[0] holds (bit 2 if it is not -1).  A target row, or
       the draft row of a node with at least one child, holding NaN / +inf
       or only -inf makes the tree emit nothing (bit 4).
  R27  outputs as the greedy tree: n = depth of the final node; tokens = the
       path's tokens (root excluded) then y; nodes = root .. final node
       (nodes[i] is the node whose row produced tokens[i]); resid = the
       normalised r that y was drawn from.  Flagged (reading R14): an accept
       test with ratio < 1 and |u - ratio| < 1e-6, a draw within 1e-6 of a
       boundary, or a nucleus cut margin below 1e-6 whose marginal token was
       tested or drawn.
"""
from __future__ import annotations

import numpy as np

from .verify import (FLAG_BAND, STATUS_BAD_LOGITS, STATUS_BAD_PARENT, STATUS_BAD_TOKEN,
                     inverse_cdf, row_is_valid, transform_row)


def tree_children(parents):
    """R26: children[u] = nodes i >= 1 with parents[i] == u and 0 <= parents[i] < i,
    in increasing index order; also returns the status bits of the structure."""
    N = len(parents)
    status = 0
    if int(parents[0]) != -1:
        status |= STATUS_BAD_PARENT
    children = [[] for _ in range(N)]
    for i in range(1, N):
        par = int(parents[i])
        if 0 <= par < i:
            children[par].append(i)
        else:
            status |= STATUS_BAD_PARENT
    return children, status


def tree_sample(target_rows, draft_rows, parents, tokens, uniforms, resid_uniform,
                temperature: float, top_k: int = 0, top_p: float = 1.0):
    """One tree, readings R24-R27.  Returns a dict with n, tokens, nodes,
    status, resid, flagged and the margins behind the flag."""
    T = np.asarray(target_rows, dtype=np.float64)
    D = np.asarray(draft_rows, dtype=np.float64)
    N, V = T.shape
    out = {"n": 0, "tokens": [], "nodes": [], "status": 0, "resid": np.zeros(V),
           "flagged": False, "accept_margins": [], "cdf_margin": np.inf}
    children, status = tree_children(parents)
    rows_ok = all(row_is_valid(T[i]) for i in range(N)) and \
        all(row_is_valid(D[u]) for u in range(N) if children[u])
    if not rows_ok:
        out["status"] = STATUS_BAD_LOGITS
        return out

    cuts = []
    decided = set()
    path = [0]
    cur = 0
    while True:
        p, cut = transform_row(T[cur], temperature, top_k, top_p, want_cut=True)
        cuts.append(cut)
        r = p
        nxt = None
        if children[cur]:
            q, qcut = transform_row(D[cur], temperature, top_k, top_p, want_cut=True)
            cuts.append(qcut)
            for c in children[cur]:
                x = int(tokens[c])
                if not (0 <= x < V):
                    status |= STATUS_BAD_TOKEN
                    accept = False
                else:
                    decided.add(x)
                    a, b = r[x], q[x]
                    u = np.float64(uniforms[c])      # float32 inputs widen exactly
                    if b > 0.0:
                        ratio = a / b
                        accept = u < min(1.0, ratio)
                        if ratio < 1.0:
                            out["accept_margins"].append(abs(u - ratio))
                    else:
                        accept = a > 0.0
                if accept:
                    nxt = c
                    break
                res = np.maximum(0.0, r - q)
                s = res.sum()
                if s > 0.0:
                    r = res / s
        if nxt is None:
            break
        path.append(nxt)
        cur = nxt

    y, cdf_margin = inverse_cdf(r, np.float64(resid_uniform))
    decided.add(y)
    out["n"] = len(path) - 1
    out["tokens"] = [int(tokens[i]) for i in path[1:]] + [y]
    out["nodes"] = list(path)
    out["status"] = status
    out["resid"] = r / np.cumsum(r)[-1]
    out["cdf_margin"] = cdf_margin
    flagged = any(m < FLAG_BAND for m in out["accept_margins"]) or cdf_margin < FLAG_BAND
    for c in cuts:
        if c is None:
            continue
        if (c["margin_lo"] < FLAG_BAND and c["last_kept"] in decided) or \
           (c["margin_hi"] < FLAG_BAND and c["next_token"] in decided):
            flagged = True
    out["flagged"] = bool(flagged)
    return out


def run_tree_sample_batch(target, draft, parents, tokens, uniforms, resid_uniforms,
                          temperature=1.0, top_k=0, top_p=1.0, want_resid=False, which=None):
    """tree_sample for the trees of a batch (all, or the indices in `which`).
    Returns accepted_len [B], out_tokens [B, N], out_nodes [B, N] (-1 padded),
    seq_status [B], flagged [B] and, with want_resid, resid [B, V]."""
    target = np.asarray(target)
    B, N, V = target.shape
    acc = np.zeros(B, dtype=np.int32)
    toks = np.full((B, N), -1, dtype=np.int32)
    nodes = np.full((B, N), -1, dtype=np.int32)
    st = np.zeros(B, dtype=np.int32)
    flagged = np.zeros(B, dtype=bool)
    resid = np.zeros((B, V)) if want_resid else None
    for b in (range(B) if which is None else which):
        o = tree_sample(target[b], draft[b], parents[b], tokens[b], uniforms[b],
                        resid_uniforms[b], temperature, top_k, top_p)
        acc[b] = o["n"]
        toks[b, :len(o["tokens"])] = o["tokens"]
        nodes[b, :len(o["nodes"])] = o["nodes"]
        st[b] = o["status"]
        flagged[b] = o["flagged"]
        if want_resid:
            resid[b] = o["resid"]
    return acc, toks, nodes, st, flagged, resid
