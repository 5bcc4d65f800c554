"""Planted mistakes in a copy of the oracle's source must fail a pin (CPU only).

Each mutant is a one-line slip a careful author could make -- a flipped
ratio, a wrong sign, an off-by-one, a dropped term, a wrong tie rule.  The
mutated source is executed into a fresh module and the pins of
oracle_pins.py run against it; the test passes when some pin rejects it.
"""
import types

import pytest

import oracle.calculator as calc
import oracle.verify as real
import oracle_pins as pins

SRC = open(real.__file__).read()

MUTANTS = [
    ("accept ratio inverted", "ratio = a / b", "ratio = b / a"),
    ("accept test reversed", "accept = u < min(1.0, ratio)", "accept = u > min(1.0, ratio)"),
    ("residual sign flipped", "r = np.maximum(0.0, p_rows[n] - q_rows[n])",
     "r = np.maximum(0.0, q_rows[n] - p_rows[n])"),
    ("resample from p, not the residual", "r = np.maximum(0.0, p_rows[n] - q_rows[n])", "r = p_rows[n].copy()"),
    ("clip dropped from the residual", "r = np.maximum(0.0, p_rows[n] - q_rows[n])",
     "r = np.abs(p_rows[n] - q_rows[n])"),
    ("bonus from the wrong row", "        r = p_rows[k].copy()", "        r = p_rows[k - 1].copy()"),
    ("target row off by one in the test", "a = p_rows[j][x]", "a = p_rows[j + 1][x]"),
    ("no stop at the first rejection", "        if not accept:\n            n = j\n            break",
     "        if not accept:\n            n = j"),
    ("zero-q draft always rejected", "            accept = a > 0.0", "            accept = False"),
    ("empty-residual fallback not p", "        if r.sum() == 0.0:\n            r = p_rows[n].copy()",
     "        if r.sum() == 0.0:\n            r = np.ones(V)"),
    ("inverse CDF takes the left boundary", 'side="right"', 'side="left"'),
    ("temperature multiplies", "/ np.float64(temperature)", "* np.float64(temperature)"),
    ("ties go to the higher index", "np.lexsort((idx, -values))", "np.lexsort((-idx, -values))"),
    ("nucleus keeps <= top_p", "kept_sorted = before < np.float64(top_p)", "kept_sorted = before <= np.float64(top_p)"),
    ("nucleus uses inclusive mass", "before = np.concatenate(([0.0], csum[:-1]))", "before = csum"),
    ("nucleus not renormalised", "        P = np.where(nuc, P, 0.0)\n        P = P / P.sum()",
     "        P = np.where(nuc, P, 0.0)"),
    ("top-k keeps one too many", "keep[order[:top_k]] = True", "keep[order[:top_k + 1]] = True"),
    ("greedy compares with the next row", "        if x != g[j]:", "        if x != g[j + 1 if j + 1 <= k else j]:"),
    ("greedy correction from row 0", "    tokens = [int(t) for t in draft_tokens[:n]] + [g[n]]",
     "    tokens = [int(t) for t in draft_tokens[:n]] + [g[0]]"),
    ("tree ignores the ancestors", "acc[i] = acc[par] and t == g[par]", "acc[i] = t == g[par]"),
    ("tree compares with its own row", "acc[i] = acc[par] and t == g[par]", "acc[i] = acc[par] and t == g[i]"),
    ("tree depth ties go to the larger index", "if acc[i] and depth[i] > depth[best]:",
     "if acc[i] and depth[i] >= depth[best]:"),
    ("inverse-CDF margin not normalised",
     "margin = min(np.float64(uniform) - lo / S, C[y] / S - np.float64(uniform))",
     "margin = min(np.float64(uniform) - lo, C[y] - np.float64(uniform))"),
    ("inverse-CDF margin misses the upper edge",
     "margin = min(np.float64(uniform) - lo / S, C[y] / S - np.float64(uniform))",
     "margin = np.float64(uniform) - lo / S"),
    ("draw margin left out of the flag",
     'flagged = any(m < FLAG_BAND for m in out["accept_margins"]) or cdf_margin < FLAG_BAND',
     'flagged = any(m < FLAG_BAND for m in out["accept_margins"])'),
    ("accept margins left out of the flag",
     'flagged = any(m < FLAG_BAND for m in out["accept_margins"]) or cdf_margin < FLAG_BAND',
     'flagged = cdf_margin < FLAG_BAND'),
    ("upper cut margin dropped",
     '"margin_hi": float(csum[R] - np.float64(top_p)) if R + 1 < V else np.inf,',
     '"margin_hi": np.inf,'),
    ("lower cut margin measured from the wrong rank",
     '"margin_lo": float(np.float64(top_p) - before[R]),',
     '"margin_lo": float(np.float64(top_p) - before[R - 1]),'),
    ("cut flag ignores whether the marginal token is decided",
     '(c["margin_lo"] < FLAG_BAND and c["last_kept"] in decided)',
     '(c["margin_lo"] < FLAG_BAND)'),
    ("cut flag checks the wrong token",
     '(c["margin_hi"] < FLAG_BAND and c["next_token"] in decided)',
     '(c["margin_hi"] < FLAG_BAND and c["last_kept"] in decided)'),
    ("accept margin kept for ratios of 1 and above",
     '            if ratio < 1.0:\n                out["accept_margins"].append(abs(u - ratio))',
     '            out["accept_margins"].append(abs(u - ratio))'),
    ("drawn token not counted as decided",
     "if 0 <= int(t) < V) | {y}", "if 0 <= int(t) < V)"),
    ("tree correction from the parent", "path_tokens = [int(tokens[i]) for i in path[1:]] + [g[best]]",
     "path_tokens = [int(tokens[i]) for i in path[1:]] + [g[path[-2] if len(path) > 1 else best]]"),
]

CALC_SRC = open(calc.__file__).read()
CALC_MUTANTS = [
    ("E exponent off by one", "alpha ** (gamma + 1)", "alpha ** gamma"),
    ("cost drops the target pass", "return gamma * c + 1.0", "return gamma * c"),
    ("series one term short", "for _ in range(gamma + 1):", "for _ in range(gamma):"),
    ("break-even inverted", "return k / (k + 1.0)", "return (k + 1.0) / k"),
    ("scan keeps the last tie", "if s > best_s:", "if s >= best_s:"),
]


def _quick_pins():
    return [
        pins.pin_greedy_golden, pins.pin_tree_golden, pins.pin_transform_golden,
        pins.pin_inverse_cdf_golden, pins.pin_flags, pins.pin_flag_rules, pins.pin_greedy_invariants,
        pins.pin_tree_path_equals_chain, pins.pin_tree_bruteforce, pins.pin_transform_softmax,
        pins.pin_transform_topk, pins.pin_topp_minimal, pins.pin_special_cases,
        pins.pin_residual_properties,
        lambda m: pins.pin_enumeration(m, reps=1),
        lambda m: pins.pin_chisq(m, trials=6000),
        lambda m: pins.pin_constant_alpha(m, calc, trials=800),
    ]


def _load_mutant(src, old, new, name):
    assert src.count(old) == 1, ("mutation site not unique", old)
    mod = types.ModuleType("mutant_" + name.replace(" ", "_"))
    exec(compile(src.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_verify_mutant_is_caught(name, old, new):
    mod = _load_mutant(SRC, old, new, name)
    for pin in _quick_pins():
        try:
            pin(mod)
        except Exception:
            return
    pytest.fail("mutant survived every pin: " + name)


@pytest.mark.parametrize("name,old,new", CALC_MUTANTS, ids=[m[0] for m in CALC_MUTANTS])
def test_calculator_mutant_is_caught(name, old, new):
    mod = _load_mutant(CALC_SRC, old, new, name)
    with pytest.raises(Exception):
        pins.pin_calculator(mod)


import oracle.aux as aux_real

AUX_SRC = open(aux_real.__file__).read()
AUX_MUTANTS = [
    ("tested counts only the accepted", "tested = int(np.minimum(n + 1, k).sum())", "tested = int(n.sum())"),
    ("tested ignores the cap at k", "tested = int(np.minimum(n + 1, k).sum())", "tested = int((n + 1).sum())"),
    ("acceptance over tested tokens", '"acceptance": accepted / drafted if drafted else 0.0',
     '"acceptance": accepted / tested if tested else 0.0'),
    ("MAL counts the correction token", '"mal": accepted / seqs if seqs else 0.0',
     '"mal": (accepted + seqs) / seqs if seqs else 0.0'),
    ("bad-logits sequences kept", "keep = (np.asarray(seq_status) & STATUS_BAD_LOGITS) == 0",
     "keep = np.ones(n.shape, dtype=bool)"),
    ("mask row misses the node itself", "        chain = [i]\n", "        chain = []\n"),
    ("mask stops below the root", "        while j != 0:", "        while parents[j] != 0 and j != 0:"),
    ("depth counts the node itself", "            depth.append(len(chain) - 1)", "            depth.append(len(chain))"),
    ("commit positions off by one", "        pos[int(path_nodes[d])] = d", "        pos[int(path_nodes[d])] = d + 1"),
    ("commit drops the last path node", "    for d in range(int(n) + 1):", "    for d in range(int(n)):"),
]


def _load_aux_mutant(old, new, name):
    assert AUX_SRC.count(old) == 1, ("mutation site not unique", old)
    mod = types.ModuleType("oracle.mutant_aux_" + name.replace(" ", "_"))
    mod.__dict__["__package__"] = "oracle"
    exec(compile(AUX_SRC.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", AUX_MUTANTS, ids=[m[0] for m in AUX_MUTANTS])
def test_aux_mutant_is_caught(name, old, new):
    mod = _load_aux_mutant(old, new, name)
    for pin in (pins.pin_aux_golden, pins.pin_mask_recursion, pins.pin_commit_inverse,
                lambda m: pins.pin_alpha_recovery(m, calc)):
        try:
            pin(mod)
        except Exception:
            return
    pytest.fail("mutant survived every pin: " + name)


import oracle.tree_sample as ts_real

TS_SRC = open(ts_real.__file__).read()
TS_MUTANTS = [
    ("running target not replaced by the residual", "                if s > 0.0:\n                    r = res / s",
     "                if s > 0.0:\n                    pass"),
    ("residual not clamped at zero", "                res = np.maximum(0.0, r - q)", "                res = np.abs(r - q)"),
    ("residual subtracts the target", "                res = np.maximum(0.0, r - q)", "                res = np.maximum(0.0, q - r)"),
    ("test against p'_u instead of the running target", "                    a, b = r[x], q[x]",
     "                    a, b = p[x], q[x]"),
    ("children tried in reverse order", "            for c in children[cur]:", "            for c in reversed(children[cur]):"),
    ("walk stops after the first accepted child", "        path.append(nxt)\n        cur = nxt",
     "        path.append(nxt)\n        cur = nxt\n        break"),
    ("the draw after a full walk uses the parent's row", "        p, cut = transform_row(T[cur]",
     "        p, cut = transform_row(T[path[-2] if len(path) > 1 else cur]"),
    ("bad parent still a child", "        if 0 <= par < i:", "        if par < i:"),
    ("leaf draft rows read", "        all(row_is_valid(D[u]) for u in range(N) if children[u])",
     "        all(row_is_valid(D[u]) for u in range(N))"),
    ("uniform of the parent used", "                    u = np.float64(uniforms[c])",
     "                    u = np.float64(uniforms[cur])"),
    ("tree draw margin left out of the flag",
     'flagged = any(m < FLAG_BAND for m in out["accept_margins"]) or cdf_margin < FLAG_BAND',
     'flagged = any(m < FLAG_BAND for m in out["accept_margins"])'),
    ("tree accept margins left out of the flag",
     'flagged = any(m < FLAG_BAND for m in out["accept_margins"]) or cdf_margin < FLAG_BAND',
     'flagged = cdf_margin < FLAG_BAND'),
    ("tree accept margin kept for ratios above 1",
     "                        if ratio < 1.0:\n                            out[\"accept_margins\"].append(abs(u - ratio))",
     "                        out[\"accept_margins\"].append(abs(u - ratio))"),
]


def _load_ts_mutant(old, new, name):
    assert TS_SRC.count(old) == 1, ("mutation site not unique", old)
    mod = types.ModuleType("oracle.mutant_ts_" + name.replace(" ", "_"))
    mod.__dict__["__package__"] = "oracle"
    exec(compile(TS_SRC.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", TS_MUTANTS, ids=[m[0] for m in TS_MUTANTS])
def test_tree_sample_mutant_is_caught(name, old, new):
    mod = _load_ts_mutant(old, new, name)
    for pin in (pins.pin_tree_sample_golden, pins.pin_tree_sample_flags,
                lambda m: pins.pin_tree_sample_is_chain(m, real),
                pins.pin_tree_sample_status, lambda m: pins.pin_tree_sample_enumeration(m, real),
                lambda m: pins.pin_tree_sample_chisq(m, real, trials=3000)):
        try:
            pin(mod)
        except Exception:
            return
    pytest.fail("mutant survived every pin: " + name)
