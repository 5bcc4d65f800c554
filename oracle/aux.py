"""Plain CPU oracle for the steps on either side of verification.

TEST INFRASTRUCTURE ONLY (same import rule as oracle/verify.py): only tests/,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
it.  It shares no code with the HIP library.

Sources:
  [Olifant]  "Towards Green Text Generation: Memory-Based Speculative
             Decoding" -- Appendix A: acceptance is the fraction of drafted
             tokens the verifier accepts; MAL (mean accepted length) is the
             mean number of draft tokens accepted per verification step.
             Section 2.4: upon rejection the KV cache is truncated to the
             accepted prefix.
  [Explainer] edgeinferencenotes.hashnode.dev speculative-decoding / EAGLE-3
             article -- "One decode round, end to end": a pass commits the
             accepted draft tokens plus one (the committed count per target
             pass); the flattened tree is scored under a tree attention mask
             that lets each candidate see only its own ancestors (and the
             context), never sibling branches; the longest agreed path is
             committed and the rest collapse.
  [Calculator] "Speculative Decoding Speedup Calculator" -- alpha is the
             probability that the target accepts a given draft token, an
             empirical number measured on one's own prompts; E, cost and
             speedup as in oracle/calculator.py.

Readings (numbered as in the design doc):
  R20  alpha measured from a batch of verification results = accepted draft
       tokens / tested draft tokens, where a sequence with n accepted of k
       tested min(n + 1, k) tokens (the ones up to and including its first
       rejection).  Under the calculator's model (every tested token accepted
       independently with probability alpha) this is the maximum-likelihood
       estimate.  No tested token (k = 0 or no sequence): alpha = 0.
  R21  sequences whose status has the bad-logits bit emitted nothing and are
       left out of every statistic.
  R22  the tree attention mask row of node i holds i and its ancestors (the
       root included); a node whose parent chain is malformed (some parent
       not in [0, i) for its node i) is unreachable: its row holds only itself
       and its depth is -1.  Node 0 is the root whatever parents[0] holds (the
       verification flags a root parent other than -1).
  R23  commit map: node i of the accepted root-to-d* path moves to position
       depth(i) (root 0); every other node collapses (-1).  A sequence that
       emitted nothing (n outside [0, N) or a path node outside [0, N))
       commits nothing.

Parity status: pinned by hand-worked examples (tests/golden/aux.json), the
mask recursion and popcount invariants, brute-force ancestor enumeration,
and, for alpha, recovery of the true value on simulated constant-alpha
sequences (statistical).
"""
from __future__ import annotations

import numpy as np

from .calculator import best_gamma, expected_tokens_closed, speedup

STATUS_BAD_LOGITS = 4
GAMMA_SCAN = range(1, 13)


def accept_stats(accepted_len, k: int, draft_cost: float, seq_status=None) -> dict:
    """Acceptance statistics of one batch and the calculator fed with the
    measured alpha.

    [Olifant] Appendix A: acceptance = accepted / drafted, MAL = accepted per
    verification step.  [Explainer]: committed tokens per pass = MAL + 1.
    [Calculator]: alpha (R20), E(alpha, k), speedup(alpha, gamma, c) for
    gamma = 1..12 and the best gamma (smallest on ties).
    """
    n = np.asarray(accepted_len, dtype=np.int64)
    keep = np.ones(n.shape, dtype=bool)
    if seq_status is not None:
        keep = (np.asarray(seq_status) & STATUS_BAD_LOGITS) == 0       # R21
    n = n[keep]
    seqs = int(n.size)
    accepted = int(n.sum())
    drafted = seqs * int(k)
    tested = int(np.minimum(n + 1, k).sum())                              # R20
    out = {
        "sequences": seqs, "accepted": accepted, "drafted": drafted, "tested": tested,
        "acceptance": accepted / drafted if drafted else 0.0,
        "mal": accepted / seqs if seqs else 0.0,
        "tokens_per_step": (accepted + seqs) / seqs if seqs else 0.0,
        "alpha": accepted / tested if tested else 0.0,
    }
    a = out["alpha"]
    out["expected_tokens"] = expected_tokens_closed(a, int(k))
    out["speedups"] = [speedup(a, g, draft_cost) for g in GAMMA_SCAN]
    g_best, s_best = best_gamma(a, draft_cost)
    out["gamma_best"] = g_best
    out["speedup_best"] = s_best
    return out


def tree_ancestors(parents):
    """R22: per node, its depth (-1 if unreachable) and the set holding the
    node and its ancestors, by walking the parent chain to the root."""
    parents = [int(x) for x in parents]
    N = len(parents)
    depth, sets = [], []
    for i in range(N):
        chain = [i]
        ok = True
        j = i
        while j != 0:
            par = parents[j]
            if not (0 <= par < j):
                ok = False
                break
            chain.append(par)
            j = par
        if ok:
            depth.append(len(chain) - 1)
            sets.append(set(chain))
        else:
            depth.append(-1)
            sets.append({i})
    return depth, sets


def tree_attention_mask(parents):
    """[Explainer] tree attention mask: row i lets node i see itself and its
    ancestors only.  Returns (mask [N, ceil(N/32)] uint32 words, bit j of row
    i set iff j is in the set; depth [N])."""
    depth, sets = tree_ancestors(parents)
    N = len(depth)
    W = (N + 31) // 32
    mask = np.zeros((N, W), dtype=np.uint32)
    for i in range(N):
        for j in sets[i]:
            mask[i, j // 32] |= np.uint32(1 << (j % 32))
    return mask, np.array(depth, dtype=np.int32)


def tree_commit_map(path_nodes, n: int, N: int):
    """R23: commit_pos[i] = position of node i on the accepted path (the
    root at 0, the node at depth d at d) for the n + 1 path nodes; -1 for
    every node that collapses.  An n outside [0, N), or a path node outside
    [0, N) (a sequence that emitted nothing), commits nothing."""
    pos = np.full(N, -1, dtype=np.int32)
    if not (0 <= int(n) < N) or any(not (0 <= int(path_nodes[d]) < N) for d in range(int(n) + 1)):
        return pos
    for d in range(int(n) + 1):
        pos[int(path_nodes[d])] = d
    return pos
