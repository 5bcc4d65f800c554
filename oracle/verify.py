"""Plain CPU oracle for the verification step of speculative decoding.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and the
two share no code.

Everything here is NumPy float64, written for a reader who checks it against
the pages by eye: one logits row at a time, no blocking, no fusion.  bf16 and
fp32 inputs convert to float64 exactly.

Sources (the pages this follows):
  [Olifant]  "Towards Green Text Generation: Memory-Based Speculative
             Decoding" -- section 1 (draft k, verify k+1 positions, keep the
             longest prefix that agrees with the verifier's greedy choices) and
             section 2.4 "Verifier and Acceptance" (logits at positions
             ctx-1 .. ctx+k-1 compared greedily with the drafts; acceptance at
             token-ID level).
  [Explainer] edgeinferencenotes.hashnode.dev speculative-decoding / EAGLE-3
             article -- "The core idea: draft, then check" (accept outright if
             p >= q, else with probability p/q; at the first rejection resample
             from the leftover mass; bonus token when all are accepted; at
             least one and at most k+1 tokens per pass), "Why it changes
             nothing about the output" (temperature / top-k / nucleus by
             adjusting both distributions before the test) and "One decode
             round, end to end" (token tree, accept-or-correct applied down
             the branches, longest agreed path plus one correction).

Readings of points the pages leave open are numbered R1..R16 and listed in
the design doc; each function names the ones it uses.

Parity status: every function here is pinned by tests under tests/ against
facts the pages or mathematics fix (hand examples, exact enumeration of the
emitted-token distribution, chi-square, closed forms, library routines,
brute force).  The one thing no page fixes is *which* token a given uniform
selects inside a distribution; that choice (inverse CDF in vocabulary order,
reading R8) is oracle-defined and only its distribution is pinned.
"""
from __future__ import annotations

import numpy as np

# Per-sequence status bits (same meaning as the library's seq_status output).
STATUS_BAD_TOKEN = 1    # a drafted / tree token outside [0, V): treated as rejected
STATUS_BAD_PARENT = 2   # a malformed parent index: that node is unreachable
STATUS_BAD_LOGITS = 4   # a NaN / +inf / all -inf row: the sequence emits nothing

FLAG_BAND = 1e-6        # a decision whose uniform lies this close to its threshold is "flagged"


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

def row_is_valid(z: np.ndarray) -> bool:
    """Reading R16: a row with NaN or +inf, or with no finite maximum, is invalid."""
    if np.isnan(z).any() or np.isposinf(z).any():
        return False
    return bool(np.isfinite(z).any())


# --------------------------------------------------------------------------
# C1: adjusting a distribution before the test
# --------------------------------------------------------------------------

def rank_order(values: np.ndarray) -> np.ndarray:
    """Indices sorted by (value descending, index ascending) -- the tie rule of
    readings R5 and R7 (lower index first)."""
    idx = np.arange(values.shape[0])
    return np.lexsort((idx, -values))


def transform_row(logits: np.ndarray, temperature: float, top_k: int = 0,
                  top_p: float = 1.0, want_cut: bool = False):
    """Turn one row of logits into the adjusted distribution used by the test.

    [Explainer] "Why it changes nothing about the output": temperature, top-k
    and nucleus sampling are handled by adjusting both distributions before
    the accept test.  Reading R5 fixes the order and ties:

      1. z = logits / T                       (float64 division, R6)
      2. top_k > 0: keep exactly top_k entries under (z desc, index asc);
         the rest get probability 0
      3. softmax over the kept entries: m = max z, e = exp(z - m), P = e / sum e
      4. top_p < 1: order by (P desc, index asc) -- computed as (z desc,
         index asc), the same order in exact arithmetic; keep the entry at rank r iff
         the mass strictly before rank r is < top_p (the smallest prefix whose
         mass reaches top_p; rank 0 is always kept); renormalise

    Returns the float64 distribution (and, with want_cut, a dict describing
    the nucleus cut for the margin report of reading R14).
    """
    z = np.asarray(logits, dtype=np.float64) / np.float64(temperature)
    V = z.shape[0]
    keep = np.ones(V, dtype=bool)
    if top_k > 0 and top_k < V:
        order = rank_order(z)
        keep[:] = False
        keep[order[:top_k]] = True
    zk = np.where(keep, z, -np.inf)
    m = zk.max()
    e = np.exp(zk - m)              # exp(-inf) = 0 for dropped entries
    P = e / e.sum()
    cut = None
    if top_p < 1.0:
        # rank by z (exp is strictly increasing, so this is the probability
        # order of exact arithmetic; ranking the rounded float64 P could tie
        # two distinct logits)
        order = rank_order(zk)
        Ps = P[order]
        csum = np.cumsum(Ps)                       # inclusive, sequential float64
        before = np.concatenate(([0.0], csum[:-1]))  # mass strictly before each rank
        kept_sorted = before < np.float64(top_p)
        R = int(np.nonzero(kept_sorted)[0].max())  # last kept rank
        nuc = np.zeros(V, dtype=bool)
        nuc[order[kept_sorted]] = True
        P = np.where(nuc, P, 0.0)
        P = P / P.sum()
        cut = {
            "last_kept": int(order[R]),
            "margin_lo": float(np.float64(top_p) - before[R]),
            "next_token": int(order[R + 1]) if R + 1 < V else -1,
            "margin_hi": float(csum[R] - np.float64(top_p)) if R + 1 < V else np.inf,
            "size": R + 1,
        }
    if want_cut:
        return P, cut
    return P


# --------------------------------------------------------------------------
# inverse-CDF draw (readings R8, R9)
# --------------------------------------------------------------------------

def inverse_cdf(weights: np.ndarray, uniform: float):
    """y = min{v : C_v > uniform * S'} with C the running sum of ``weights``
    in vocabulary order and S' = C[V-1]; clamped to the last v with a
    positive weight.  Returns (y, margin), margin = distance of the uniform
    from the nearest boundary of y's interval in normalised units."""
    C = np.cumsum(np.asarray(weights, dtype=np.float64))
    S = C[-1]
    t = np.float64(uniform) * S
    y = int(np.searchsorted(C, t, side="right"))
    if y >= C.shape[0]:
        y = int(np.nonzero(weights > 0)[0].max())
    lo = C[y - 1] if y > 0 else 0.0
    margin = min(np.float64(uniform) - lo / S, C[y] / S - np.float64(uniform))
    return y, float(margin)


# --------------------------------------------------------------------------
# C2: greedy chain verification
# --------------------------------------------------------------------------

def greedy_chain(target_rows: np.ndarray, draft_tokens: np.ndarray):
    """Greedy longest-agreed-prefix rule.

    [Olifant] section 1 and section 2.4: the verifier scores all k+1 positions
    in one pass, and the logits at positions ctx-1 .. ctx+k-1 are compared
    greedily with the drafts; a token is accepted iff it equals the
    verifier's own greedy choice (token-ID level).  Row j of ``target_rows``
    is the verifier's prediction for draft position j; row k is the bonus row.

      g_j = argmax row j (lowest index on ties, R7)
      n   = first j < k with x_j != g_j, else k
      emit x_0..x_{n-1}, g_n

    Returns (n, tokens, status).
    """
    T = np.asarray(target_rows, dtype=np.float64)
    k = T.shape[0] - 1
    V = T.shape[1]
    if not all(row_is_valid(T[j]) for j in range(k + 1)):
        return 0, [], STATUS_BAD_LOGITS
    status = 0
    g = [int(np.argmax(T[j])) for j in range(k + 1)]   # np.argmax: first maximal index
    n = k
    for j in range(k):
        x = int(draft_tokens[j])
        if not (0 <= x < V):
            status |= STATUS_BAD_TOKEN
            n = j
            break
        if x != g[j]:
            n = j
            break
    tokens = [int(t) for t in draft_tokens[:n]] + [g[n]]
    return n, tokens, status


# --------------------------------------------------------------------------
# C3: modified rejection sampling over a chain
# --------------------------------------------------------------------------

def sample_chain(target_rows, draft_rows, draft_tokens, uniforms, resid_uniform,
                 temperature: float, top_k: int = 0, top_p: float = 1.0):
    """Modified rejection sampling for one sequence.

    [Explainer] "The core idea: draft, then check": with p the target's and q
    the draft's probability of a drafted token, accept it outright if p >= q
    and otherwise with probability p/q (R2: accept iff u < min(1, p/q));
    at the first rejection drop the rest and resample one token from the
    leftover mass max(0, p - q), renormalised; if all k are accepted, emit
    one bonus token from the target's last row (R10).  p and q are the
    adjusted distributions of C1 (R5).

      for j in 0..k-1:  a = p'_j(x_j), b = q'_j(x_j)
                        accept iff (b > 0 and u_j < min(1, a/b)) or (b = 0 and a > 0)   (R3)
      n = first rejected j, else k
      r = max(0, p'_n - q'_n)  (n < k; if sum r = 0 use p'_n, R9)   or   r = p'_k (n = k)
      y = inverse_cdf(r, ur)   (R8)
      emit x_0..x_{n-1}, y

    Returns a dict with n, tokens, status, resid (the normalised r used),
    flagged (reading R14) and the individual margins.
    """
    T = np.asarray(target_rows, dtype=np.float64)
    D = np.asarray(draft_rows, dtype=np.float64)
    k = T.shape[0] - 1
    V = T.shape[1]
    out = {"n": 0, "tokens": [], "status": 0, "resid": np.zeros(V), "flagged": False,
           "accept_margins": [], "cdf_margin": np.inf, "cut_flags": []}
    rows_ok = all(row_is_valid(T[j]) for j in range(k + 1)) and \
        all(row_is_valid(D[j]) for j in range(k))
    if not rows_ok:
        out["status"] = STATUS_BAD_LOGITS
        return out

    want_cut = top_p < 1.0
    p_rows, q_rows, p_cuts, q_cuts = [], [], [], []
    for j in range(k + 1):
        P, c = transform_row(T[j], temperature, top_k, top_p, want_cut=True)
        p_rows.append(P)
        p_cuts.append(c)
    for j in range(k):
        Q, c = transform_row(D[j], temperature, top_k, top_p, want_cut=True)
        q_rows.append(Q)
        q_cuts.append(c)

    status = 0
    n = k
    for j in range(k):
        x = int(draft_tokens[j])
        if not (0 <= x < V):
            status |= STATUS_BAD_TOKEN
            n = j
            break
        a = p_rows[j][x]
        b = q_rows[j][x]
        u = np.float64(uniforms[j])          # float32 inputs widen exactly
        if b > 0.0:
            ratio = a / b
            accept = u < min(1.0, ratio)
            if ratio < 1.0:
                out["accept_margins"].append(abs(u - ratio))
        else:
            accept = a > 0.0
        if not accept:
            n = j
            break

    if n < k:
        r = np.maximum(0.0, p_rows[n] - q_rows[n])
        if r.sum() == 0.0:
            r = p_rows[n].copy()
    else:
        r = p_rows[k].copy()
    y, cdf_margin = inverse_cdf(r, np.float64(resid_uniform))
    out["resid"] = r / np.cumsum(r)[-1]
    out["cdf_margin"] = cdf_margin
    out["n"] = n
    out["status"] = status
    out["tokens"] = [int(t) for t in draft_tokens[:n]] + [y]

    # reading R14: flag decisions whose uniform lies within FLAG_BAND of a threshold
    flagged = any(m < FLAG_BAND for m in out["accept_margins"]) or cdf_margin < FLAG_BAND
    if want_cut:
        decided = set(int(t) for t in draft_tokens[:min(n + 1, k)] if 0 <= int(t) < V) | {y}
        rows = [p_cuts[j] for j in range(n + 1)] + [q_cuts[j] for j in range(min(n + 1, k))]
        for c in rows:
            if (c["margin_lo"] < FLAG_BAND and c["last_kept"] in decided) or \
               (c["margin_hi"] < FLAG_BAND and c["next_token"] in decided):
                flagged = True
                out["cut_flags"].append(c)
    out["flagged"] = bool(flagged)
    return out


# --------------------------------------------------------------------------
# C4: greedy token-tree verification
# --------------------------------------------------------------------------

def tree_greedy(target_rows, parents, tokens):
    """Greedy verification of a flattened token tree.

    [Explainer] "One decode round, end to end": the tree is scored in one
    target pass, the accept-or-correct rule is applied down the branches, the
    single longest agreed path is committed and one correction is added.  In
    the greedy case a node is accepted iff its parent is accepted and its
    token equals the target's argmax at the parent.

      node 0 is the root (its token is ignored); parents[i] < i for i >= 1
      row i of ``target_rows`` is the target's distribution for node i's children
      g_i = argmax row i (lowest index on ties, R7)
      acc(0) = true;  acc(i) = acc(parents[i]) and tokens[i] == g_{parents[i]}
      d* = accepted node of maximum depth, smallest index on ties (R12)
      emit the tokens on the path root -> d* (root excluded), then g_{d*} (R13)

    Returns (n, path_tokens, path_nodes, status): n = depth(d*), path_tokens
    has n+1 entries (the last is the correction), path_nodes has n+1 entries
    (root first; path_nodes[i] is the node whose row produced path_tokens[i]).
    """
    T = np.asarray(target_rows, dtype=np.float64)
    N, V = T.shape
    if not all(row_is_valid(T[i]) for i in range(N)):
        return 0, [], [], STATUS_BAD_LOGITS
    status = 0
    g = [int(np.argmax(T[i])) for i in range(N)]
    acc = [False] * N
    depth = [0] * N
    acc[0] = True
    if int(parents[0]) != -1:
        status |= STATUS_BAD_PARENT
    for i in range(1, N):
        par = int(parents[i])
        if not (0 <= par < i):
            status |= STATUS_BAD_PARENT
            continue
        depth[i] = depth[par] + 1
        t = int(tokens[i])
        if not (0 <= t < V):
            status |= STATUS_BAD_TOKEN
            continue
        acc[i] = acc[par] and t == g[par]
    best = 0
    for i in range(1, N):
        if acc[i] and depth[i] > depth[best]:
            best = i
    path = [best]
    while path[-1] != 0:
        path.append(int(parents[path[-1]]))
    path.reverse()
    n = depth[best]
    path_tokens = [int(tokens[i]) for i in path[1:]] + [g[best]]
    return n, path_tokens, path, status


# --------------------------------------------------------------------------
# batch wrappers: the library's output layout
# --------------------------------------------------------------------------

def run_chain_batch(mode: str, target, draft, draft_tokens, uniforms, resid_uniforms,
                    temperature=1.0, top_k=0, top_p=1.0, want_resid=False):
    """Apply C2 ("greedy") or C3 ("sample") to every sequence of a batch.

    target: [B, k+1, V] float64-convertible; draft: [B, k, V] or None.
    Returns accepted_len [B], out_tokens [B, k+1] (-1 padded), seq_status [B],
    flagged [B] and, with want_resid, resid [B, V] float64.
    """
    target = np.asarray(target)
    B, K1, V = target.shape
    k = K1 - 1
    acc = np.zeros(B, dtype=np.int32)
    toks = np.full((B, k + 1), -1, dtype=np.int32)
    st = np.zeros(B, dtype=np.int32)
    flagged = np.zeros(B, dtype=bool)
    resid = np.zeros((B, V)) if want_resid else None
    for b in range(B):
        if mode == "greedy":
            n, t, s = greedy_chain(target[b], draft_tokens[b])
        else:
            o = sample_chain(target[b], draft[b], draft_tokens[b], uniforms[b],
                             resid_uniforms[b], temperature, top_k, top_p)
            n, t, s = o["n"], o["tokens"], o["status"]
            flagged[b] = o["flagged"]
            if want_resid:
                resid[b] = o["resid"]
        acc[b] = n
        toks[b, :len(t)] = t
        st[b] = s
    return acc, toks, st, flagged, resid


def run_tree_batch(target, parents, tokens):
    """Apply C4 to every tree of a batch.  target: [B, N, V].
    Returns accepted_len [B], out_tokens [B, N], out_nodes [B, N] (-1 padded), seq_status [B]."""
    target = np.asarray(target)
    B, N, V = target.shape
    acc = np.zeros(B, dtype=np.int32)
    toks = np.full((B, N), -1, dtype=np.int32)
    nodes = np.full((B, N), -1, dtype=np.int32)
    st = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n, t, p, s = tree_greedy(target[b], parents[b], tokens[b])
        acc[b] = n
        toks[b, :len(t)] = t
        nodes[b, :len(p)] = p
        st[b] = s
    return acc, toks, nodes, st


def draw_from(probs: np.ndarray, uniform: float) -> int:
    """Draw one index from a distribution with one uniform (inverse CDF, R8).
    Used by tests to play the draft model: x_j ~ q'_j (reading R15)."""
    return inverse_cdf(probs, uniform)[0]
