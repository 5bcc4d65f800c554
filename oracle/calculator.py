"""Leviathan improvement-factor model, as the speedup calculator page states it.

TEST INFRASTRUCTURE ONLY (see oracle/verify.py for the import rule).

Source: "Speculative Decoding Speedup Calculator" (induwara.lk), the three
steps it lists -- step 1 expected tokens per step E, step 2 cost per step,
step 3 speedup = E / cost (Leviathan et al. Theorem 3.8) -- and its gamma scan
over 1..12.  Break-even acceptance: [Olifant] section 5.1, Equation (1).

Inputs: alpha = per-token acceptance probability, gamma = draft tokens per
step, c = cost of one draft pass in units of one target pass.
"""
from __future__ import annotations


def expected_tokens_closed(alpha: float, gamma: int) -> float:
    """Step 1, closed form: E = (1 - alpha^(gamma+1)) / (1 - alpha).
    At alpha = 1 the limit gamma + 1 is returned (reading R17)."""
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def expected_tokens_series(alpha: float, gamma: int) -> float:
    """Step 1, as the series 1 + alpha + ... + alpha^gamma (the page's self-check)."""
    total = 0.0
    term = 1.0
    for _ in range(gamma + 1):
        total += term
        term *= alpha
    return total


def step_cost(gamma: int, c: float) -> float:
    """Step 2: the draft runs gamma times at cost c, plus one target pass."""
    return gamma * c + 1.0


def speedup(alpha: float, gamma: int, c: float) -> float:
    """Step 3: improvement factor E / (gamma * c + 1)."""
    return expected_tokens_closed(alpha, gamma) / step_cost(gamma, c)


def best_gamma(alpha: float, c: float, lo: int = 1, hi: int = 12):
    """Scan gamma = lo..hi and return (gamma*, speedup); smallest gamma on ties (R18)."""
    best_g, best_s = lo, speedup(alpha, lo, c)
    for g in range(lo + 1, hi + 1):
        s = speedup(alpha, g, c)
        if s > best_s:
            best_g, best_s = g, s
    return best_g, best_s


def break_even_acceptance(k: int) -> float:
    """[Olifant] section 5.1, Equation (1): acceptance needed to break even when
    verifying k drafts costs as much as generating them, about k / (k + 1)."""
    return k / (k + 1.0)
