"""Checks that pin the oracle to facts other than itself.

Each ``pin_*`` function takes the oracle's verify module (and, for the
calculator, its calculator module) as an argument and raises AssertionError
when a pin does not hold.  The same functions run against the real oracle
(tests/test_oracle_*.py) and against source-level mutants of it
(tests/test_oracle_mutations.py), which shows that a plausible slip in the
oracle -- a dropped term, a flipped sign, an off-by-one, swapped operands --
breaks at least one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special
import scipy.stats

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rows(rows):
    return np.array([[float(v) for v in r] for r in rows], dtype=np.float64)


# ---------------------------------------------------------------- greedy chain

def pin_greedy_golden(ov):
    for c in _load("greedy_chain.json")["cases"]:
        n, toks, st = ov.greedy_chain(_rows(c["rows"]), np.array(c["drafts"]))
        assert (n, list(toks), st) == (c["n"], c["tokens"], c["status"]), (c["name"], n, toks, st)


def pin_greedy_invariants(ov, trials=300, seed=0):
    """Output-preserving by construction ([Olifant] section 2.4): the emitted
    tokens are exactly the verifier's greedy chain g_0..g_n, 1 <= len <= k+1,
    and the stop is at the first disagreement."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        k = int(rng.integers(1, 7))
        V = int(rng.integers(2, 6))
        rows = rng.integers(0, 3, size=(k + 1, V)).astype(np.float64)   # many ties
        g = rows.argmax(axis=1)
        x = np.where(rng.random(k) < 0.7, g[:k], rng.integers(0, V, size=k))
        n, toks, st = ov.greedy_chain(rows, x)
        assert st == 0 and 1 <= len(toks) <= k + 1 and len(toks) == n + 1
        assert list(toks) == [int(v) for v in g[:n + 1]]
        assert all(x[j] == g[j] for j in range(n))
        assert n == k or x[n] != g[n]


# ---------------------------------------------------------------- tree

def pin_tree_golden(ov):
    for c in _load("tree_greedy.json")["cases"]:
        n, toks, nodes, st = ov.tree_greedy(_rows(c["rows"]), np.array(c["parents"]), np.array(c["tokens"]))
        got = (n, list(toks), list(nodes), st)
        want = (c["n"], c["path_tokens"], c["path_nodes"], c["status"])
        assert got == want, (c["name"], got, want)


def pin_tree_path_equals_chain(ov, trials=200, seed=1):
    """A path-shaped tree (parents[i] = i-1) is a chain: same answer as C2."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        k = int(rng.integers(1, 8))
        V = int(rng.integers(2, 5))
        rows = rng.integers(0, 3, size=(k + 1, V)).astype(np.float64)
        x = rng.integers(0, V, size=k)
        n_c, t_c, _ = ov.greedy_chain(rows, x)
        parents = np.arange(-1, k)
        tokens = np.concatenate(([0], x))
        n_t, t_t, nodes, _ = ov.tree_greedy(rows, parents, tokens)
        assert (n_c, list(t_c)) == (n_t, list(t_t))
        assert list(nodes) == list(range(n_t + 1))


def pin_tree_bruteforce(ov, trials=300, seed=2):
    """Enumerate every root-to-node path; a path is accepted iff each edge's
    token equals np.argmax of its parent's row.  Deepest accepted node,
    smallest index on ties."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        N = int(rng.integers(1, 13))
        V = int(rng.integers(2, 5))
        rows = rng.normal(size=(N, V))
        parents = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, N)])
        tokens = rng.integers(0, V, size=N)
        best, best_depth, best_path = 0, 0, [0]
        for i in range(N):
            path = [i]
            while path[-1] != 0:
                path.append(int(parents[path[-1]]))
            path.reverse()
            ok = all(tokens[path[d + 1]] == np.argmax(rows[path[d]]) for d in range(len(path) - 1))
            if ok and len(path) - 1 > best_depth:
                best, best_depth, best_path = i, len(path) - 1, path
        n, toks, nodes, st = ov.tree_greedy(rows, parents, tokens)
        assert n == best_depth and list(nodes) == best_path
        assert list(toks) == [int(tokens[i]) for i in best_path[1:]] + [int(np.argmax(rows[best]))]


# ---------------------------------------------------------------- C1 transform

def pin_transform_softmax(ov, trials=50, seed=3):
    """Without filters the adjusted distribution is the textbook softmax of logits/T."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        V = int(rng.integers(2, 300))
        l = rng.normal(0, 4, size=V)
        T = float(rng.choice([1.0, 0.7, 1.3, 0.25]))
        P = ov.transform_row(l, T)
        assert np.max(np.abs(P - scipy.special.softmax(l / T))) < 1e-14


def pin_transform_topk(ov, trials=50, seed=4):
    """top-k keeps the k largest (np.argpartition on tie-free rows) and is the
    softmax restricted to them."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        V = int(rng.integers(5, 300))
        K = int(rng.integers(1, V))
        l = rng.normal(0, 3, size=V)
        T = float(rng.choice([1.0, 0.7]))
        P = ov.transform_row(l, T, top_k=K)
        top = set(np.argpartition(-l, K - 1)[:K].tolist())
        assert set(np.nonzero(P > 0)[0].tolist()) == top
        idx = np.array(sorted(top))
        assert np.max(np.abs(P[idx] - scipy.special.softmax(l[idx] / T))) < 1e-14


def pin_transform_golden(ov):
    for c in _load("transform.json")["cases"]:
        P = ov.transform_row(np.array(c["logits"], dtype=np.float64), c["T"], c["top_k"], c["top_p"])
        kept = sorted(np.nonzero(P > 0)[0].tolist())
        assert kept == c["kept"], (c, kept)
        l = np.array(c["logits"], dtype=np.float64)
        idx = np.array(kept)
        # on the kept set the result is the softmax of logits/T restricted to it
        assert np.max(np.abs(P[idx] - scipy.special.softmax(l[idx] / c["T"]))) < 1e-14


def pin_topp_minimal(ov, trials=200, seed=5):
    """Nucleus: the kept set is a top-ranked prefix whose mass reaches top_p,
    and dropping its last member would leave less than top_p (smallest such
    prefix).  Checked by brute force over prefixes of a full sort."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        V = int(rng.integers(2, 40))
        l = rng.normal(0, 2, size=V)
        p = float(rng.uniform(0.05, 0.99))
        P = ov.transform_row(l, 1.0, top_p=p)
        full = scipy.special.softmax(l)
        order = sorted(range(V), key=lambda v: (-full[v], v))
        kept = set(np.nonzero(P > 0)[0].tolist())
        r = len(kept)
        assert kept == set(order[:r])
        mass = sum(full[v] for v in order[:r])
        assert mass >= p - 1e-12 or r == V
        assert sum(full[v] for v in order[:r - 1]) < p + 1e-12
        assert abs(P.sum() - 1.0) < 1e-12
        assert np.max(np.abs(P[list(kept)] - full[list(kept)] / mass)) < 1e-13


# ---------------------------------------------------------------- inverse CDF

def pin_inverse_cdf_golden(ov):
    g = _load("inverse_cdf.json")
    w = np.array(g["weights"])
    for u, y in g["cases"]:
        assert ov.inverse_cdf(w, u)[0] == y, (u, y)


# ---------------------------------------------------------------- C3: exact enumeration

def _threshold(pred):
    """sup{u in [0, 1) : pred(u)} for a predicate true on [0, t) and false on [t, 1)."""
    if not pred(0.0):
        return 0.0
    if pred(np.nextafter(1.0, 0.0)):
        return 1.0
    lo, hi = 0.0, 1.0
    for _ in range(62):
        mid = 0.5 * (lo + hi)
        if pred(mid):
            lo = mid
        else:
            hi = mid
    return hi


def _step_measure(f, V):
    """Lebesgue measure of {u in [0,1) : f(u) = v} for v = 0..V-1, for a
    non-decreasing step function f."""
    bounds = []
    for v in range(V):
        bounds.append(_threshold(lambda u, v=v: f(u) <= v))
    return np.diff(np.concatenate(([0.0], np.maximum.accumulate(bounds))))


SETTINGS = [dict(T=1.0, top_k=0, top_p=1.0), dict(T=0.7, top_k=0, top_p=1.0),
            dict(T=1.0, top_k=3, top_p=1.0), dict(T=1.0, top_k=0, top_p=0.7),
            dict(T=0.8, top_k=5, top_p=0.8)]


def first_token_distribution(ov, tgt, dft, T, top_k, top_p):
    """Exact law of the first emitted token for k = 1, computed by treating
    the oracle as a black box: x ranges over the draft's support weighted by
    q'(x); the accept region in u and the residual draw's regions in ur are
    found by bisection (both are intervals / monotone steps)."""
    V = tgt.shape[1]
    q = ov.transform_row(dft[0], T, top_k, top_p)

    def run(x, u, ur):
        return ov.sample_chain(tgt, dft, [x], [u], ur, T, top_k, top_p)

    law = np.zeros(V)
    resid = None
    for x in range(V):
        if q[x] == 0.0:
            continue
        t = _threshold(lambda u: run(x, u, 0.5)["n"] == 1)
        law[x] += q[x] * t
        if t < 1.0:
            if resid is None:
                u_rej = np.nextafter(1.0, 0.0)
                resid = _step_measure(lambda ur: run(x, u_rej, ur)["tokens"][0], V)
            law += q[x] * (1.0 - t) * resid
    return law


def pin_enumeration(ov, seed=6, reps=3):
    """Distribution preservation ([Explainer] "Why it changes nothing about the
    output"): the first emitted token is distributed exactly as the adjusted
    target p'_0, for any draft, with and without temperature / top-k / top-p."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for s in SETTINGS:
        for _ in range(reps):
            V = 8
            tgt = rng.normal(0, 1.5, size=(2, V))
            dft = rng.normal(0, 1.5, size=(1, V))
            law = first_token_distribution(ov, tgt, dft, **s)
            p = ov.transform_row(tgt[0], s["T"], s["top_k"], s["top_p"])
            worst = max(worst, float(np.max(np.abs(law - p))))
    assert worst < 1e-12, worst
    return worst


# ---------------------------------------------------------------- C3: chi-square

def pin_chisq(ov, trials=20000, seed=7, setting=None, alpha=1e-3):
    """Brute-force trials on V=8, k=2: frequency of the first emitted token
    against p'_0, and of the second emitted token given acceptance at 0
    against p'_1, by chi-square at significance alpha."""
    rng = np.random.default_rng(seed)
    s = setting or SETTINGS[0]
    V = 8
    tgt = rng.normal(0, 1.0, size=(3, V))
    dft = tgt[:2] + rng.normal(0, 1.0, size=(2, V))
    q = [ov.transform_row(dft[j], s["T"], s["top_k"], s["top_p"]) for j in range(2)]
    p = [ov.transform_row(tgt[j], s["T"], s["top_k"], s["top_p"]) for j in range(3)]
    first = np.zeros(V)
    second = np.zeros(V)
    for _ in range(trials):
        x = [ov.draw_from(q[j], rng.random()) for j in range(2)]
        o = ov.sample_chain(tgt, dft, x, rng.random(2), rng.random(), s["T"], s["top_k"], s["top_p"])
        first[o["tokens"][0]] += 1
        if o["n"] >= 1:
            second[o["tokens"][1]] += 1
    for counts, probs in ((first, p[0]), (second, p[1])):
        support = probs > 0
        assert counts[~support].sum() == 0
        exp = probs[support] * counts.sum()
        pval = scipy.stats.chisquare(counts[support], exp).pvalue
        assert pval > alpha, (counts, exp, pval)


# ---------------------------------------------------------------- C3 vs calculator E

def pin_constant_alpha(ov, calc, trials=2500, alpha=0.6, seed=8):
    """Rows with sum_v min(p, q) = alpha exactly (q on tokens 0..V-2,
    p = alpha q + (1-alpha) delta_{V-1}); drafts x_j ~ q.  The mean number of
    tokens per pass, mean(n + 1), must match the calculator's
    E = 1 + alpha + ... + alpha^gamma within 4 standard errors."""
    rng = np.random.default_rng(seed)
    V = 8
    for gamma in range(1, 9):
        q = np.zeros((gamma, V))
        p = np.zeros((gamma + 1, V))
        for j in range(gamma):
            w = rng.random(V - 1) + 0.2
            q[j, :V - 1] = w / w.sum()
            p[j] = alpha * q[j]
            p[j, V - 1] += 1.0 - alpha
        p[gamma] = np.full(V, 1.0 / V)
        with np.errstate(divide="ignore"):
            tl, dl = np.log(p), np.log(q)
        counts = []
        for _ in range(trials):
            x = [ov.draw_from(q[j], rng.random()) for j in range(gamma)]
            o = ov.sample_chain(tl, dl, x, rng.random(gamma), rng.random(), 1.0)
            counts.append(o["n"] + 1)
        counts = np.array(counts, dtype=np.float64)
        E = calc.expected_tokens_closed(alpha, gamma)
        se = counts.std(ddof=1) / math.sqrt(trials)
        assert abs(counts.mean() - E) < 4 * se + 1e-12, (gamma, counts.mean(), E, se)


# ---------------------------------------------------------------- special cases

def pin_special_cases(ov, seed=9):
    rng = np.random.default_rng(seed)
    V = 12
    # (a) identical target and draft rows: every draft is accepted, n = k
    for s in SETTINGS:
        k = 4
        rows = rng.normal(0, 2, size=(k + 1, V))
        for _ in range(50):
            q = [ov.transform_row(rows[j], s["T"], s["top_k"], s["top_p"]) for j in range(k)]
            x = [ov.draw_from(q[j], rng.random()) for j in range(k)]
            o = ov.sample_chain(rows, rows[:k], x, rng.random(k), rng.random(), s["T"], s["top_k"], s["top_p"])
            assert o["n"] == k
    # (b) top_k = 1 sampling reproduces greedy verification, for any drafts
    for _ in range(200):
        k = int(rng.integers(1, 6))
        tgt = rng.integers(0, 4, size=(k + 1, V)).astype(np.float64)
        dft = rng.integers(0, 4, size=(k, V)).astype(np.float64)
        x = rng.integers(0, V, size=k)
        o = ov.sample_chain(tgt, dft, x, rng.random(k), rng.random(), 0.9, top_k=1)
        n, toks, _ = ov.greedy_chain(tgt, x)
        assert (o["n"], o["tokens"]) == (n, toks)
    # (c) one-hot draft at x: accept with probability p'(x); the residual is
    #     p' with x removed, renormalised
    for s in SETTINGS:
        tgt = rng.normal(0, 1.5, size=(2, V))
        x = int(rng.integers(0, V))
        dft = np.full((1, V), -np.inf)
        dft[0, x] = 0.0
        p = ov.transform_row(tgt[0], s["T"], s["top_k"], s["top_p"])

        def run(u, ur):
            return ov.sample_chain(tgt, dft, [x], [u], ur, s["T"], s["top_k"], s["top_p"])
        t = _threshold(lambda u: run(u, 0.5)["n"] == 1)
        assert abs(t - p[x]) < 1e-15
        if p[x] < 1.0:
            law = _step_measure(lambda ur: run(np.nextafter(1.0, 0.0), ur)["tokens"][0], V)
            want = p.copy()
            want[x] = 0.0
            want /= want.sum()
            assert np.max(np.abs(law - want)) < 1e-12


def pin_residual_properties(ov, trials=100, seed=10):
    """After a rejection the normalised residual is >= 0, sums to 1 and lives
    on {p' > q'}; after full acceptance it is p'_k itself."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        V = int(rng.integers(3, 50))
        k = 2
        s = SETTINGS[int(rng.integers(len(SETTINGS)))]
        tgt = rng.normal(0, 2, size=(k + 1, V))
        dft = rng.normal(0, 2, size=(k, V))
        x = rng.integers(0, V, size=k)
        o = ov.sample_chain(tgt, dft, x, rng.random(k), rng.random(), s["T"], s["top_k"], s["top_p"])
        r = o["resid"]
        assert np.all(r >= 0) and abs(r.sum() - 1) < 1e-12
        p = ov.transform_row(tgt[o["n"]], s["T"], s["top_k"], s["top_p"])
        if o["n"] < k:
            q = ov.transform_row(dft[o["n"]], s["T"], s["top_k"], s["top_p"])
            if np.any(p > q):
                assert set(np.nonzero(r > 0)[0]) <= set(np.nonzero(p > q)[0])
        else:
            assert np.max(np.abs(r - p)) < 1e-15
        assert r[o["tokens"][-1]] > 0


def pin_flags(ov):
    """Reading R14: a uniform within 1e-6 of its accept threshold flags the
    sequence; one far from every threshold does not."""
    V = 4
    tgt = np.log(np.array([[0.1, 0.2, 0.3, 0.4], [0.25, 0.25, 0.25, 0.25]]))
    dft = np.log(np.array([[0.4, 0.3, 0.2, 0.1]]))
    # x = 1: a = 0.2, b = 0.3, threshold 2/3
    near = ov.sample_chain(tgt, dft, [1], [2.0 / 3.0 + 3e-7], 0.3, 1.0)
    far = ov.sample_chain(tgt, dft, [1], [0.2], 0.3, 1.0)
    assert near["flagged"] and not far["flagged"]
    assert far["n"] == 1 and near["n"] == 0


def pin_flag_rules(ov):
    """Reading R14's other flag rules, on hand-worked exact binary weights
    (tests/golden/flags.json): the inverse-CDF margin in normalised units
    (and the flag it raises, in a residual whose mass is 1/2, not 1), and the
    nucleus cut margins on both sides of top_p, which flag a sequence only
    when the marginal token is tested or drawn."""
    g = _load("flags.json")
    ic = g["inverse_cdf"]
    w = np.array(ic["weights"])
    for c in ic["cases"]:
        y, m = ov.inverse_cdf(w, c["u"])
        assert y == c["y"] and abs(m - c["margin"]) < 1e-12, ("inverse_cdf", c, y, m)
    cd = g["chain_draw"]
    for c in cd["cases"]:
        o = ov.sample_chain(_rows(cd["target"]), _rows(cd["draft"]), cd["x"], cd["u"], c["ur"], 1.0)
        assert (o["n"], o["tokens"]) == (c["n"], c["tokens"]), ("chain_draw", c, o["n"], o["tokens"])
        assert abs(o["cdf_margin"] - c["cdf_margin"]) < 1e-12, ("chain_draw margin", c, o["cdf_margin"])
        assert o["flagged"] == c["flagged"], ("chain_draw flag", c)
    nc = g["nucleus_cut"]
    for c in nc["cases"]:
        _, cut = ov.transform_row(np.array(nc["logits"]), 1.0, 0, c["top_p"], want_cut=True)
        for key in ("last_kept", "next_token", "size"):
            assert cut[key] == c[key], ("nucleus_cut", key, c, cut)
        for key in ("margin_lo", "margin_hi"):
            assert abs(cut[key] - c[key]) < 1e-12, ("nucleus_cut", key, c, cut)
    ch = g["nucleus_chain"]
    rows = np.array([ch["logits"], ch["logits"]])
    for c in ch["cases"]:
        o = ov.sample_chain(rows, rows[:1], c["x"], c["u"], c["ur"], 1.0, 0, c["top_p"])
        assert (o["n"], o["tokens"]) == (c["n"], c["tokens"]), ("nucleus_chain", c, o["n"], o["tokens"])
        assert o["flagged"] == c["flagged"], ("nucleus_chain flag", c)
    r1 = g["ratio_one"]
    row = np.array(r1["row"])
    o = ov.sample_chain(np.array([row, row]), row[None, :], [1], [r1["u"]], r1["chain"]["ur"], 1.0)
    c = r1["chain"]
    assert (o["n"], o["tokens"], o["flagged"]) == (c["n"], c["tokens"], c["flagged"]), ("ratio one", o)


# ---------------------------------------------------------------- calculator

def pin_calculator(calc):
    g = _load("calculator.json")
    for w in g["worked_examples"]:
        assert round(calc.speedup(w["alpha"], w["gamma"], w["c"]), 2) == w["speedup_2dp"], w
    for e in g["expected_tokens"]:
        assert abs(calc.expected_tokens_closed(e["alpha"], e["gamma"]) - e["E"]) < 1e-12
        assert abs(calc.expected_tokens_series(e["alpha"], e["gamma"]) - e["E"]) < 1e-12
    for b in g["break_even_percent"]:
        assert round(100 * calc.break_even_acceptance(b["k"])) == b["percent"]
    # closed form and series agree everywhere (the page's self-check)
    for a in np.linspace(0, 0.99, 34):
        for gm in range(0, 13):
            assert abs(calc.expected_tokens_closed(a, gm) - calc.expected_tokens_series(a, gm)) < 1e-12
    # speed-up rises to a peak and then falls (the page's gamma scan; ties such
    # as alpha=0.5, c=0.2 at gamma 1 and 2 happen), and the scan's answer is the
    # first of the best of the 12 values
    for a in (0.5, 0.7, 0.8, 0.9):
        for c in (0.05, 0.1, 0.2):
            s = [calc.speedup(a, gm, c) for gm in range(1, 13)]
            peak = int(np.argmax(s))
            assert all(s[i] <= s[i + 1] + 1e-12 for i in range(peak)) and \
                all(s[i] >= s[i + 1] - 1e-12 for i in range(peak, 11))
            gbest, sbest = calc.best_gamma(a, c)
            assert gbest == peak + 1 and sbest == max(s)
    # no drafting cost: more drafts never hurt; expensive drafts: gamma = 1
    assert calc.best_gamma(0.8, 0.0)[0] == 12
    assert calc.best_gamma(0.3, 0.9)[0] == 1
    assert calc.step_cost(4, 0.1) == 1.4


ALL_ORACLE_PINS = [
    pin_greedy_golden, pin_greedy_invariants, pin_tree_golden, pin_tree_path_equals_chain,
    pin_tree_bruteforce, pin_transform_softmax, pin_transform_topk, pin_transform_golden,
    pin_topp_minimal, pin_inverse_cdf_golden, pin_enumeration, pin_special_cases,
    pin_residual_properties, pin_flags, pin_flag_rules,
]


# ---------------------------------------------------------------- acceptance statistics, tree mask, commit map

def _frac(x):
    return None if x is None else x[0] / x[1]


def pin_aux_golden(ax):
    g = _load("aux.json")
    for c in g["stats"]:
        r = ax.accept_stats(c["n"], c["k"], c["c"], c["status"])
        for key in ("accepted", "drafted", "tested", "sequences"):
            assert r[key] == c[key], (c["name"], key, r[key])
        for key in ("acceptance", "mal", "tokens_per_step", "alpha", "expected_tokens"):
            if c[key] is not None:
                assert abs(r[key] - _frac(c[key])) <= 1e-15, (c["name"], key, r[key])
    for c in g["masks"]:
        if "chain" in c:
            m, d = ax.tree_attention_mask([-1] + list(range(c["chain"] - 1)))
            assert [int(w) for w in m[c["row"]]] == c["words"] and int(d[c["row"]]) == c["depth_last"], c["name"]
        else:
            m, d = ax.tree_attention_mask(c["parents"])
            assert [[int(w) for w in row] for row in m] == c["rows"], (c["name"], m)
            assert [int(x) for x in d] == c["depth"], (c["name"], d)
    for c in g["commits"]:
        pos = ax.tree_commit_map(c["path"], c["n"], c["N"])
        assert [int(x) for x in pos] == c["pos"], (c["name"], pos)


def _random_tree(rng, N, bad=False):
    par = [-1]
    for i in range(1, N):
        par.append(int(rng.integers(0, i)))
    if bad and N > 3:
        par[int(rng.integers(2, N))] = N + 5          # out of range: that node and its subtree unreachable
    return par


def pin_mask_recursion(ax):
    """Row i = row(parent i) with bit i added, for every reachable node; the
    row of a node has depth + 1 bits; siblings never see each other; an
    unreachable node sees only itself."""
    rng = np.random.default_rng(123)
    for t in range(60):
        N = int(rng.integers(1, 90))
        par = _random_tree(rng, N, bad=(t % 4 == 3))
        m, d = ax.tree_attention_mask(par)
        bits = lambda i: {j for j in range(N) if (int(m[i, j // 32]) >> (j % 32)) & 1}
        for i in range(N):
            bi = bits(i)
            if d[i] < 0:
                assert bi == {i}, (par, i)
                continue
            assert len(bi) == d[i] + 1, (par, i)
            if i == 0:
                assert bi == {0}
            else:
                assert d[par[i]] >= 0 and bi == bits(par[i]) | {i}, (par, i)
                for s in range(1, N):
                    if s != i and par[s] == par[i]:
                        assert s not in bi, (par, i, s)


def pin_commit_inverse(ax):
    """The commit map inverts the accepted path: path node d goes to d, the
    other nodes collapse."""
    rng = np.random.default_rng(7)
    for _ in range(40):
        N = int(rng.integers(2, 50))
        par = _random_tree(rng, N)
        leaf = int(rng.integers(0, N))
        path = [leaf]
        while path[-1] != 0:
            path.append(par[path[-1]])
        path.reverse()
        pos = ax.tree_commit_map(path, len(path) - 1, N)
        assert sorted(int(x) for x in pos if x >= 0) == list(range(len(path)))
        for d, node in enumerate(path):
            assert pos[node] == d
        assert int((pos < 0).sum()) == N - len(path)


def pin_alpha_recovery(ax, calc):
    """Sequences drawn from the calculator's own model (each tested draft
    accepted independently with probability alpha, stop at the first
    rejection, at most k): the measured alpha recovers alpha within 4
    standard errors, and mean tokens per step matches E(alpha, k)."""
    rng = np.random.default_rng(2024)
    for alpha, k in ((0.3, 3), (0.7, 5), (0.9, 8)):
        S = 200000
        u = rng.random((S, k))
        fail = u >= alpha
        n = np.where(fail.any(axis=1), fail.argmax(axis=1), k)
        r = ax.accept_stats(n, k, 0.05)
        se = math.sqrt(alpha * (1 - alpha) / r["tested"])
        assert abs(r["alpha"] - alpha) < 4 * se, (alpha, k, r["alpha"])
        tps_se = float(np.std(n + 1)) / math.sqrt(S)
        assert abs(r["tokens_per_step"] - calc.expected_tokens_closed(alpha, k)) < 4 * tps_se, (alpha, k)
        assert abs(r["expected_tokens"] - calc.expected_tokens_closed(r["alpha"], k)) < 1e-15


# ---------------------------------------------------------------- tree sampling (readings R24-R27)

def _tree_logits(rows):
    with np.errstate(divide="ignore"):
        return np.log(np.array(rows, dtype=np.float64))


def pin_tree_sample_golden(ts):
    """Hand-worked trees (tests/golden/tree_sample.json)."""
    for c in _load("tree_sample.json")["cases"]:
        o = ts.tree_sample(_tree_logits(c["target"]), _tree_logits(c["draft"]), np.array(c["parents"]),
                           np.array(c["tokens"]), np.array(c["u"]), c["ur"], 1.0)
        got = (o["n"], o["tokens"], o["nodes"], o["status"])
        want = (c["n"], c["out_tokens"], c["out_nodes"], c["status"])
        assert got == want, (c["name"], got, want)
        assert np.allclose(o["resid"], c["resid"], rtol=0, atol=1e-12), (c["name"], o["resid"])


def pin_tree_sample_flags(ts):
    """Reading R14 in a sampled tree (tests/golden/flags.json): a child's
    uniform near its accept threshold, and the draw near a boundary of the
    running residual (after a rejection) or of a leaf's target row (after an
    acceptance), flag the tree; the same walks with the uniforms moved off
    the thresholds do not."""
    g = _load("flags.json")["tree"]
    for c in g["cases"]:
        o = ts.tree_sample(_rows(g["target"]), _rows(g["draft"]), np.array(g["parents"]),
                           np.array(g["tokens"]), np.array([0.0, c["u1"]]), c["ur"], 1.0)
        assert (o["n"], o["tokens"]) == (c["n"], c["tokens"]), ("tree flags", c, o["n"], o["tokens"])
        assert o["flagged"] == c["flagged"], ("tree flags", c)
    r1 = _load("flags.json")["ratio_one"]
    row = np.array(r1["row"])
    leaf = np.zeros(4)
    o = ts.tree_sample(np.array([row, leaf]), np.array([row, leaf]), np.array([-1, 0]), np.array([0, 1]),
                       np.array([0.0, r1["u"]]), r1["tree"]["ur"], 1.0)
    c = r1["tree"]
    assert (o["n"], o["tokens"], o["flagged"]) == (c["n"], c["tokens"], c["flagged"]), ("tree ratio one", o)


def pin_tree_sample_is_chain(ts, ov, trials=150, seed=11):
    """A path-shaped tree (one child per node) is the chain: node i + 1 carries
    draft token i, target and draft row i are the chain's rows i, node i + 1's
    uniform is the chain's u_i.  Same tokens, length, status and residual."""
    rng = np.random.default_rng(seed)
    for t in range(trials):
        s = SETTINGS[t % len(SETTINGS)]
        k = int(rng.integers(1, 6))
        V = int(rng.integers(3, 9))
        tgt = rng.normal(0, 1.5, size=(k + 1, V))
        dft = tgt[:k] + rng.normal(0, 1.0, size=(k, V))
        q = [ov.transform_row(dft[j], s["T"], s["top_k"], s["top_p"]) for j in range(k)]
        x = [ov.draw_from(q[j], rng.random()) if rng.random() < 0.9 else int(rng.integers(0, V))
             for j in range(k)]
        u = rng.random(k)
        ur = rng.random()
        c = ov.sample_chain(tgt, dft, x, u, ur, s["T"], s["top_k"], s["top_p"])
        parents = np.arange(-1, k)
        tokens = np.array([0] + list(x))
        draft_rows = np.vstack([dft, np.zeros((1, V))])
        o = ts.tree_sample(tgt, draft_rows, parents, tokens, np.concatenate(([0.0], u)), ur,
                           s["T"], s["top_k"], s["top_p"])
        assert (o["n"], o["tokens"], o["status"]) == (c["n"], c["tokens"], c["status"]), (t, o, c)
        assert o["nodes"] == list(range(o["n"] + 1))
        assert np.allclose(o["resid"], c["resid"], rtol=0, atol=1e-14), (t, o["resid"], c["resid"])


def tree_first_token_law(ts, ov, tgt, dft, m, T, top_k, top_p):
    """Exact law of the first emitted token of a root with m leaf children
    whose tokens are drawn independently from q'_root, with the oracle as a
    black box: every token tuple weighted by its draft probability; child i's
    accept region in u_i (earlier children forced to reject) and the residual
    draw's regions in ur found by bisection."""
    V = tgt.shape[1]
    q = ov.transform_row(dft[0], T, top_k, top_p)
    parents = np.array([-1] + [0] * m)
    never = np.nextafter(1.0, 0.0)

    def run(xs, us, ur):
        return ts.tree_sample(tgt, dft, parents, np.array([0] + list(xs)), np.array([0.0] + list(us)),
                              ur, T, top_k, top_p)

    law = np.zeros(V)
    resid = None
    support = [v for v in range(V) if q[v] > 0.0]
    for xs in np.array(np.meshgrid(*[support] * m, indexing="ij")).reshape(m, -1).T:
        w = float(np.prod([q[x] for x in xs]))
        surv = 1.0
        for i in range(m):
            def acc_i(u, i=i):
                us = [never] * i + [u] + [never] * (m - i - 1)
                o = run(xs, us, 0.5)
                return o["n"] >= 1 and o["nodes"][1] == i + 1
            th = _threshold(acc_i)
            law[xs[i]] += w * surv * th
            surv *= 1.0 - th
            if surv == 0.0:
                break
        if surv > 0.0:
            if resid is None:
                resid = _step_measure(lambda ur: run(xs, [never] * m, ur)["tokens"][0], V)
            law += w * surv * resid
    return law


def pin_tree_sample_enumeration(ts, ov, seed=12, cases=((2, 6), (3, 5))):
    """Distribution preservation over a tree ([Explainer] "Why it changes
    nothing about the output", applied down the branches): whatever the draft,
    the first emitted token of a root with m independently drafted children
    follows p'_root exactly, under temperature, top-k and top-p."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for j, (m, V) in enumerate(cases):
        for s in (SETTINGS[j % len(SETTINGS)], SETTINGS[(j + 3) % len(SETTINGS)]):
            tgt = rng.normal(0, 1.5, size=(m + 1, V))
            dft = rng.normal(0, 1.5, size=(m + 1, V))
            law = tree_first_token_law(ts, ov, tgt, dft, m, s["T"], s["top_k"], s["top_p"])
            p = ov.transform_row(tgt[0], s["T"], s["top_k"], s["top_p"])
            worst = max(worst, float(np.max(np.abs(law - p))))
    assert worst < 1e-12, worst
    return worst


def pin_tree_sample_chisq(ts, ov, trials=6000, seed=13, alpha=1e-3):
    """Brute force on a depth-3 tree (V = 8, two or three children per inner
    node, children drawn from the draft row of their parent): the first
    emitted token follows p'_root, and the second, given that the walk went
    to the root's first child c, follows p'_c."""
    rng = np.random.default_rng(seed)
    V = 8
    parents = np.array([-1, 0, 0, 0, 1, 1, 2, 4, 4])
    N = len(parents)
    tgt = rng.normal(0, 1.0, size=(N, V))
    dft = tgt + rng.normal(0, 1.0, size=(N, V))
    q = [ov.transform_row(dft[i], 1.0) for i in range(N)]
    p = [ov.transform_row(tgt[i], 1.0) for i in range(N)]
    first = np.zeros(V)
    second = np.zeros(V)
    for _ in range(trials):
        tokens = np.array([0] + [ov.draw_from(q[parents[i]], rng.random()) for i in range(1, N)])
        o = ts.tree_sample(tgt, dft, parents, tokens, rng.random(N), rng.random(), 1.0)
        first[o["tokens"][0]] += 1
        if o["n"] >= 1 and o["nodes"][1] == 1:
            second[o["tokens"][1]] += 1
    for counts, probs in ((first, p[0]), (second, p[1])):
        assert counts.sum() > 500
        pval = scipy.stats.chisquare(counts, probs * counts.sum()).pvalue
        assert pval > alpha, (counts, probs * counts.sum(), pval)


def pin_tree_sample_status(ts):
    """R26: a NaN in a target row, or in the draft row of a node with a child,
    empties the output; the draft row of a leaf is never read."""
    V = 4
    parents = np.array([-1, 0, 1])
    tgt = np.zeros((3, V))
    dft = np.zeros((3, V))
    toks = np.array([0, 1, 2])
    u = np.full(3, 0.5)
    ok = ts.tree_sample(tgt, dft, parents, toks, u, 0.5, 1.0)
    assert ok["status"] == 0 and len(ok["tokens"]) == ok["n"] + 1
    d2 = dft.copy(); d2[2, 1] = np.nan          # leaf's draft row: not read
    assert ts.tree_sample(tgt, d2, parents, toks, u, 0.5, 1.0)["status"] == 0
    d1 = dft.copy(); d1[1, 1] = np.nan          # node 1 has a child
    o = ts.tree_sample(tgt, d1, parents, toks, u, 0.5, 1.0)
    assert o["status"] == 4 and o["tokens"] == [] and o["nodes"] == []
    t2 = tgt.copy(); t2[2, :] = -np.inf          # a target row with no finite logit
    assert ts.tree_sample(t2, dft, parents, toks, u, 0.5, 1.0)["status"] == 4
