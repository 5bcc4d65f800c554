"""Seeded synthetic workloads for draft-token verification.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the verification arithmetic: no temperature, softmax,
top-k, top-p, argmax or acceptance.  The two places where a workload needs
such a computation -- the draft model's own draw of x_j from its adjusted
distribution, and the planted tree matches that equal the target's argmax
at the parent -- take that computation from the caller as a function.

Workloads (the pages run natural-language prompts through a 32000-token
Mistral-7B verifier and 8B-class targets with ~60-node token trees; those
models and datasets are not available, so these seeded logits stand in for
the verifier's and the draft model's outputs):

  1  chain, B=1,   k=4, V=32000,  fp32: t ~ N(0, 3^2), d = t + N(0, 1^2), T=1
  2  chain, B=16,  k=5, V=32000,  bf16: t ~ N(0, 3^2) with 5 distinct tokens
     per row boosted by +8, d = t + N(0, 1.5^2), T=1
  3  chain, B=64,  k=8, V=128256, bf16: t = per row sorted N(0, 2^2) plus
     -ln(rank), randomly permuted; d = t + N(0, 1^2); T=0.7, top-k 50
  4  tree,  B=8,   N=60 nodes (root included), depth <= 6, <= 4 children,
     V=128256, bf16 t ~ N(0, 3^2) per node
  5  chain, B=256, k=4, V=152064, fp32: t ~ N(0, 2.5^2), d = 0.8 t + N(0, 1^2);
     T=0.8, top-p 0.9
  6  sampled tree, the shape of workload 4 with draft rows d = t + N(0, 1^2)
     per node and tokens drawn by the caller from the draft row at the parent

Draft logits are made from the unrounded target before both are rounded to
the storage dtype (bf16 with round-to-nearest-even).
"""
from __future__ import annotations

import numpy as np

CONFIGS = {
    1: dict(kind="chain", B=1, k=4, V=32000, dtype="f32", T=1.0, top_k=0, top_p=1.0,
            rounds=1000, recipe="gauss", sd=3.0, noise=1.0),
    2: dict(kind="chain", B=16, k=5, V=32000, dtype="bf16", T=1.0, top_k=0, top_p=1.0,
            recipe="boosted", sd=3.0, noise=1.5, n_boost=5, boost=8.0),
    3: dict(kind="chain", B=64, k=8, V=128256, dtype="bf16", T=0.7, top_k=50, top_p=1.0,
            recipe="zipf", sd=2.0, noise=1.0),
    4: dict(kind="tree", B=8, N=60, V=128256, dtype="bf16", max_depth=6, max_children=4,
            rho=0.5, sd=3.0),
    5: dict(kind="chain", B=256, k=4, V=152064, dtype="f32", T=0.8, top_k=0, top_p=0.9,
            recipe="gauss", sd=2.5, noise=1.0, draft_scale=0.8),
    # the sampling twin of workload 4 (tree_sample_inputs)
    6: dict(kind="tree_sample", B=8, N=60, V=128256, dtype="bf16", T=1.0, max_depth=6,
            max_children=4, sd=3.0, noise=1.0),
}

DEFAULT_SEED = {c: 1000 + c for c in CONFIGS}


def bf16_from_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even) and
    return the bit patterns as uint16.  Values are assumed finite and in the
    normal range of bf16."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    u = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    f32 = u.view(np.float64).astype(np.float32)   # exact: at most 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_from_f64(x64)
    return x64.astype(np.float32)


def _target_f64(rng, cfg, rows_shape, V):
    recipe = cfg.get("recipe", "gauss")
    shape = rows_shape + (V,)
    if recipe == "gauss":
        return rng.normal(0.0, cfg["sd"], size=shape)
    if recipe == "boosted":
        t = rng.normal(0.0, cfg["sd"], size=shape)
        flat = t.reshape(-1, V)
        nb = cfg["n_boost"]
        for r in range(flat.shape[0]):
            idx = rng.choice(V, size=nb, replace=False)
            flat[r, idx] += cfg["boost"]
        return t
    if recipe == "zipf":
        flat = rng.normal(0.0, cfg["sd"], size=(int(np.prod(rows_shape)), V))
        flat = -np.sort(-flat, axis=1)                       # descending
        flat -= np.log(np.arange(1, V + 1, dtype=np.float64))  # log-rank decay
        flat = rng.permuted(flat, axis=1)
        return flat.reshape(shape)
    raise ValueError(recipe)


def chain_inputs(config: int, seed: int | None = None, B: int | None = None,
                 V: int | None = None, k: int | None = None, dtype: str | None = None,
                 noise: float | None = None):
    """Seeded inputs of a chain workload (configs 1, 2, 3, 5), optionally with
    smaller B / V / k, or another draft noise sd, for parity cases.

    Returns a dict:
      target  [B, k+1, V]  float32, or uint16 bf16 bit patterns
      draft   [B, k, V]    same dtype
      draw_u  [B, k]       float64 uniforms the draft model uses to draw x_j
      u       [B, k]       float32 accept-test uniforms in [0, 1)
      ur      [B]          float32 residual / bonus uniforms in [0, 1)
      plus the scalar settings (T, top_k, top_p, dtype, B, k, V).
    """
    cfg = dict(CONFIGS[config])
    assert cfg["kind"] == "chain"
    B = cfg["B"] if B is None else B
    V = cfg["V"] if V is None else V
    k = cfg["k"] if k is None else k
    dtype = cfg["dtype"] if dtype is None else dtype
    if noise is not None:
        cfg["noise"] = noise
    rng = np.random.default_rng(DEFAULT_SEED[config] if seed is None else seed)
    t64 = _target_f64(rng, cfg, (B, k + 1), V)
    d64 = cfg.get("draft_scale", 1.0) * t64[:, :k] + rng.normal(0.0, cfg["noise"], size=(B, k, V))
    draw_u = rng.random(size=(B, k))
    u = rng.random(size=(B, k), dtype=np.float32)
    ur = rng.random(size=(B,), dtype=np.float32)
    return dict(target=_store(t64, dtype), draft=_store(d64, dtype), draw_u=draw_u, u=u, ur=ur,
                T=cfg["T"], top_k=cfg["top_k"], top_p=cfg["top_p"], dtype=dtype, B=B, k=k, V=V)


def draft_tokens(draft_rows_f64_fn, draw_u: np.ndarray) -> np.ndarray:
    """x[b, j] = draw(b, j, draw_u[b, j]) with ``draft_rows_f64_fn(b, j, w)``
    supplied by the caller (the draft model's sampler)."""
    B, k = draw_u.shape
    x = np.zeros((B, k), dtype=np.int32)
    for b in range(B):
        for j in range(k):
            x[b, j] = draft_rows_f64_fn(b, j, float(draw_u[b, j]))
    return x


def tree_inputs(config: int = 4, seed: int | None = None, B: int | None = None,
                N: int | None = None, V: int | None = None, dtype: str | None = None):
    """Seeded inputs of a token-tree workload.

    Shape: node 0 is the root; for i = 1..N-1 the parent is uniform over the
    earlier nodes whose depth is below max_depth and that have fewer than
    max_children children.  For every node with children, with probability
    rho one random child is marked to carry the target's argmax at the parent
    (a planted match); the other children get distinct random tokens from a
    pre-drawn pool that excludes that argmax.  Tokens are filled in by
    ``tree_tokens`` once the caller has computed the argmax per node.

    Returns a dict with target [B, N, V], parents [B, N] int32, and the
    plant/pool arrays ``tree_tokens`` needs.
    """
    cfg = dict(CONFIGS[config])
    assert cfg["kind"] == "tree"
    B = cfg["B"] if B is None else B
    N = cfg["N"] if N is None else N
    V = cfg["V"] if V is None else V
    dtype = cfg["dtype"] if dtype is None else dtype
    md, mc = cfg["max_depth"], cfg["max_children"]
    rng = np.random.default_rng(DEFAULT_SEED[config] if seed is None else seed)
    t64 = rng.normal(0.0, cfg["sd"], size=(B, N, V))
    parents = np.full((B, N), -1, dtype=np.int32)
    plant = np.full((B, N), -1, dtype=np.int32)
    pool = np.zeros((B, N, mc + 1), dtype=np.int64)
    for b in range(B):
        depth = [0] * N
        nchild = [0] * N
        children = [[] for _ in range(N)]
        for i in range(1, N):
            elig = [j for j in range(i) if depth[j] < md and nchild[j] < mc]
            par = elig[int(rng.integers(len(elig)))]
            parents[b, i] = par
            depth[i] = depth[par] + 1
            nchild[par] += 1
            children[par].append(i)
        for p in range(N):
            if children[p] and rng.random() < cfg["rho"]:
                plant[b, p] = children[p][int(rng.integers(len(children[p])))]
            pool[b, p] = rng.choice(V, size=mc + 1, replace=False)
    return dict(target=_store(t64, dtype), parents=parents, plant=plant, pool=pool,
                dtype=dtype, B=B, N=N, V=V)


def tree_tokens(tree: dict, argmax_rows: np.ndarray) -> np.ndarray:
    """Fill in the tree's tokens given the caller's argmax per node row
    (``argmax_rows`` [B, N])."""
    parents, plant, pool = tree["parents"], tree["plant"], tree["pool"]
    B, N = parents.shape
    tokens = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        for p in range(N):
            kids = [i for i in range(1, N) if parents[b, i] == p]
            if not kids:
                continue
            g = int(argmax_rows[b, p])
            others = [int(t) for t in pool[b, p] if int(t) != g]
            o = 0
            for c in kids:
                if c == plant[b, p]:
                    tokens[b, c] = g
                else:
                    tokens[b, c] = others[o]
                    o += 1
    return tokens


def rows_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored rows -> float64 (exact) for consumers that need real values."""
    if dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def tree_sample_inputs(seed: int = 1006, B: int = 8, N: int = 60, V: int = 128256,
                       dtype: str = "bf16", T: float = 1.0, sd: float = 3.0, noise: float = 1.0,
                       max_depth: int = 6, max_children: int = 4):
    """Seeded inputs of a sampled token tree (the sampling twin of workload 4).

    The tree shape follows ``tree_inputs`` (parent uniform over the earlier
    nodes below max_depth with fewer than max_children children).  Target
    rows t ~ N(0, sd^2) per node, draft rows d = t + N(0, noise^2) (made
    before rounding to the storage dtype); uniforms u [B, N] and ur [B] for
    the tests, and draw_u [B, N] with which the caller draws node i's token
    from the draft's adjusted distribution at its parent (the draft model's
    own draw, done by the caller).
    """
    rng = np.random.default_rng(seed)
    t64 = rng.normal(0.0, sd, size=(B, N, V))
    d64 = t64 + rng.normal(0.0, noise, size=(B, N, V))
    parents = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        depth = [0] * N
        nchild = [0] * N
        for i in range(1, N):
            elig = [j for j in range(i) if depth[j] < max_depth and nchild[j] < max_children]
            par = elig[int(rng.integers(len(elig)))]
            parents[b, i] = par
            depth[i] = depth[par] + 1
            nchild[par] += 1
    u = rng.random((B, N)).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    draw_u = rng.random((B, N))
    return dict(target=_store(t64, dtype), draft=_store(d64, dtype), parents=parents, u=u, ur=ur,
                draw_u=draw_u, dtype=dtype, T=T, B=B, N=N, V=V)
