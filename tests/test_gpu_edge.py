"""Edge cases, degenerate inputs, determinism and the emitted-token law on the GPU."""
import numpy as np
import pytest
import scipy.stats
import torch

import oracle.verify as ov
from draft_token_verification_softmax_amd import SV_MODE_GREEDY, SV_MODE_SAMPLE, SpecVerify
from draft_token_verification_softmax_amd import workloads as wl
from gpu_common import compare_chain, draw_drafts, oracle_chain, run_chain, run_tree, say

pytestmark = pytest.mark.gpu


def test_empty_batch_is_a_no_op():
    say("empty batch")
    sv = SpecVerify(mode=SV_MODE_SAMPLE, dtype="f32", max_batch=4, k=3, vocab=100)
    e = torch.empty(0, 4, 100, device="cuda")
    out = sv.run(e, torch.empty(0, 3, 100, device="cuda"), torch.empty(0, 3, dtype=torch.int32, device="cuda"),
                 torch.empty(0, 3, device="cuda"), torch.empty(0, device="cuda"))
    torch.cuda.synchronize()
    assert out["accepted_len"].numel() == 0


@pytest.mark.parametrize("mode", ["greedy", "sample", "topk", "topp"])
def test_bad_logits_and_tokens(mode):
    say("bad logits/tokens", mode)
    inp = wl.chain_inputs(2, seed=21, B=8, V=3000, k=4, dtype="f32")
    if mode == "topk":
        inp["top_k"] = 20
    if mode == "topp":
        inp["top_p"] = 0.8
    x = draw_drafts(inp)
    t, d = inp["target"], inp["draft"]
    t[0, 1, 17] = np.nan              # NaN in a target row
    d[1, 2, 5] = np.inf               # +inf in a draft row
    t[2, 0, :] = -np.inf              # a row with no finite value
    t[3, 2, :100] = -np.inf           # -inf entries are allowed
    x[4, 0] = 3000                    # token outside the vocabulary
    x[5, 0] = -7
    x[7, 2] = 4000                    # after an earlier rejection it is never reached
    t[6, 3, 2999] = -np.nan           # negative NaN at the last position
    m = SV_MODE_GREEDY if mode == "greedy" else SV_MODE_SAMPLE
    gpu = run_chain(inp, x, m)
    orc = oracle_chain(inp, x, m, list(range(8)))
    compare_chain(gpu, orc, range(8), f"bad inputs {mode}")
    assert gpu["seq_status"][0] == 4 and gpu["seq_status"][2] == 4
    if mode != "greedy":
        assert gpu["seq_status"][1] == 4
    assert (gpu["seq_status"][4] & 1) and (gpu["seq_status"][5] & 1)
    assert gpu["seq_status"][6] == 4
    assert np.all(gpu["out_tokens"][0] == -1) and gpu["accepted_len"][0] == 0


@pytest.mark.parametrize("N", [20, 64, 100])
def test_tree_bad_rows(N):
    # a NaN, a +inf and an all -inf target row each make their tree invalid;
    # -inf entries alone do not (trees of up to 64 nodes take the kernel's
    # one-wave path, larger ones the block path)
    say("tree bad rows", N)
    tr = wl.tree_inputs(4, seed=40 + N, B=5, N=N, V=2000)
    t = tr["target"]                  # bf16 bit patterns
    t[0, 3, 17] = 0x7FC0              # NaN
    t[1, N - 1, 5] = 0x7F80           # +inf
    t[2, 0, :] = 0xFF80               # -inf
    t[3, 1, :50] = 0xFF80
    T64 = wl.rows_f64(t, tr["dtype"])
    tokens = wl.tree_tokens(tr, np.argmax(np.where(np.isnan(T64), -np.inf, T64), axis=-1))
    gpu = run_tree(tr, tokens)
    acc, toks, nodes, st = ov.run_tree_batch(T64, tr["parents"], tokens)
    assert list(st[:3]) == [4, 4, 4] and st[3] != 4
    assert np.array_equal(gpu["seq_status"], st)
    assert np.array_equal(gpu["accepted_len"], acc)
    assert np.array_equal(gpu["out_tokens"], toks) and np.array_equal(gpu["out_nodes"], nodes)


def test_tree_bad_parents_and_tokens():
    say("tree bad parents")
    tr = wl.tree_inputs(4, seed=5, B=4, N=20, V=2000)
    T64 = wl.rows_f64(tr["target"], tr["dtype"])
    tokens = wl.tree_tokens(tr, np.argmax(T64, axis=-1))
    tr["parents"][0, 5] = 7            # parent after the node
    tr["parents"][1, 0] = 3            # root with a parent
    tr["parents"][2, 9] = -4
    tokens[3, 4] = 99999
    gpu = run_tree(tr, tokens)
    acc, toks, nodes, st = ov.run_tree_batch(T64, tr["parents"], tokens)
    assert np.array_equal(gpu["seq_status"], st) and st[0] == 2 and st[3] == 1
    assert np.array_equal(gpu["accepted_len"], acc)
    assert np.array_equal(gpu["out_tokens"], toks) and np.array_equal(gpu["out_nodes"], nodes)


def test_topk_one_equals_greedy():
    say("top-k 1 == greedy")
    inp = wl.chain_inputs(2, seed=8, B=32, V=4000, k=5, dtype="bf16")
    T64 = wl.rows_f64(inp["target"], "bf16")
    rng = np.random.default_rng(0)
    g = np.argmax(T64, axis=-1)
    x = np.where(rng.random((32, 5)) < 0.8, g[:, :5], rng.integers(0, 4000, (32, 5))).astype(np.int32)
    inp["top_k"] = 1
    inp["T"] = 0.9
    s = run_chain(inp, x, SV_MODE_SAMPLE)
    gr = run_chain(inp, x, SV_MODE_GREEDY)
    assert np.array_equal(s["accepted_len"], gr["accepted_len"])
    assert np.array_equal(s["out_tokens"], gr["out_tokens"])


def test_topk_at_least_vocab_is_off():
    say("top-k >= V")
    inp = wl.chain_inputs(2, seed=9, B=16, V=500, k=3, dtype="bf16")
    x = draw_drafts(inp)
    a = run_chain(inp, x, SV_MODE_SAMPLE)
    inp["top_k"] = 500
    b = run_chain(inp, x, SV_MODE_SAMPLE)
    assert np.array_equal(a["out_tokens"], b["out_tokens"])
    assert np.array_equal(a["resid_probs"], b["resid_probs"])


@pytest.mark.parametrize("top_k,top_p,max_batch", [(0, 1.0, None), (5, 1.0, None), (0, 0.6, None),
                                                   (0, 0.6, 4096)])
def test_identical_rows_accept_everything(top_k, top_p, max_batch):
    """Every draft accepted: the bonus draw from the last target row (with a
    context sized for a large batch, the nucleus residual masses come from
    the queue of kept entries, here with no draft row)."""
    say("q == p", top_k, top_p, max_batch)
    inp = wl.chain_inputs(2, seed=13, B=16, V=2000, k=4, dtype="bf16")
    inp["draft"] = inp["target"][:, :4].copy()
    inp["top_k"], inp["top_p"] = top_k, top_p
    x = draw_drafts(inp)
    g = run_chain(inp, x, SV_MODE_SAMPLE, max_batch=max_batch)
    assert np.all(g["accepted_len"] == 4)
    orc = oracle_chain(inp, x, SV_MODE_SAMPLE, list(range(16)))
    compare_chain(g, orc, range(16), "q == p")


@pytest.mark.parametrize("top_p,top_k", [(1.0, 0), (0.5, 0), (1.0, 20), (1.0, 256)])
def test_all_equal_logits(top_p, top_k):
    """Every logit ties: nucleus and top-k break ties by index; with top-k
    every group of a tile reaches the admission threshold, which sends the
    tiles down the exact fallback."""
    say("all-equal logits", top_p, top_k)
    B, k, V = 6, 3, 40001
    z = np.zeros((B, k + 1, V))
    rng = np.random.default_rng(1)
    inp = dict(target=z.astype(np.float32), draft=np.zeros((B, k, V), np.float32), dtype="f32",
               u=rng.random((B, k), dtype=np.float32), ur=rng.random(B, dtype=np.float32),
               draw_u=rng.random((B, k)), T=1.0, top_k=top_k, top_p=top_p)
    x = draw_drafts(inp)
    gpu = run_chain(inp, x, SV_MODE_SAMPLE)
    orc = oracle_chain(inp, x, SV_MODE_SAMPLE, list(range(B)))
    compare_chain(gpu, orc, range(B), f"equal logits top-p {top_p} top-k {top_k}")


def test_topk_ties_bf16():
    """bf16 logits on a coarse grid: many exact ties around each tile's
    top-k threshold (large candidate lists)."""
    say("top-k ties bf16")
    inp = wl.chain_inputs(3, seed=44, B=4, V=128256, k=3, dtype="bf16")
    rng = np.random.default_rng(44)
    t = np.round(rng.normal(0, 2, size=(4, 4, 128256)) * 2) / 2     # multiples of 0.5
    d = t[:, :3] + np.round(rng.normal(0, 1, size=(4, 3, 128256)) * 2) / 2
    inp["target"] = wl.bf16_from_f64(t)
    inp["draft"] = wl.bf16_from_f64(d)
    inp["top_k"] = 50
    x = draw_drafts(inp)
    gpu = run_chain(inp, x, SV_MODE_SAMPLE)
    orc = oracle_chain(inp, x, SV_MODE_SAMPLE, list(range(4)))
    compare_chain(gpu, orc, range(4), "top-k ties")


def test_tiny_vocab():
    say("tiny vocab")
    for V in (1, 2, 7, 8, 9):
        inp = wl.chain_inputs(1, seed=V, B=50, V=V, k=3, dtype="f32")
        x = draw_drafts(inp)
        gpu = run_chain(inp, x, SV_MODE_SAMPLE)
        orc = oracle_chain(inp, x, SV_MODE_SAMPLE, list(range(50)))
        compare_chain(gpu, orc, range(50), f"V={V}")


@pytest.mark.parametrize("top_k,top_p,max_batch", [(0, 1.0, None), (50, 1.0, None), (0, 0.9, None),
                                                   (0, 0.9, 4096)])
def test_deterministic_across_calls_and_addresses(top_k, top_p, max_batch):
    """Bit-identical outputs (resid_probs included) over repeated calls and
    shifted buffer addresses: plain, top-k and nucleus sampling, the last
    with a context that takes the nucleus residual through its queues."""
    say("determinism", top_k, top_p, max_batch)
    inp = wl.chain_inputs(2, seed=31, B=16, V=32000, k=5, dtype="bf16")
    inp["top_k"], inp["top_p"] = top_k, top_p
    x = draw_drafts(inp)
    a = run_chain(inp, x, SV_MODE_SAMPLE, max_batch=max_batch)
    b = run_chain(inp, x, SV_MODE_SAMPLE, max_batch=max_batch)
    pad = torch.empty(12345, dtype=torch.uint8, device="cuda")   # shift the next allocations
    c = run_chain(inp, x, SV_MODE_SAMPLE, max_batch=max_batch)
    del pad
    for key in ("accepted_len", "out_tokens", "seq_status", "resid_probs"):
        assert np.array_equal(a[key], b[key]) and np.array_equal(a[key], c[key]), key


@pytest.mark.parametrize("setting", [dict(T=1.0, top_k=0, top_p=1.0), dict(T=0.7, top_k=3, top_p=1.0),
                                     dict(T=1.0, top_k=0, top_p=0.7)])
def test_emitted_token_law_chisq(setting):
    """Many sequences with the same logits and fresh uniforms: the first
    emitted token follows p'_0 and the second (after acceptance) p'_1."""
    say("chi-square", setting)
    rng = np.random.default_rng(17)
    V, k, B = 8, 2, 40000
    t = rng.normal(0, 1.0, size=(k + 1, V))
    d = t[:k] + rng.normal(0, 1.0, size=(k, V))
    T, tk, tp = setting["T"], setting["top_k"], setting["top_p"]
    q = [ov.transform_row(d[j].astype(np.float32).astype(np.float64), T, tk, tp) for j in range(k)]
    p = [ov.transform_row(t[j].astype(np.float32).astype(np.float64), T, tk, tp) for j in range(k + 1)]
    x = np.array([[ov.draw_from(q[j], rng.random()) for j in range(k)] for _ in range(B)], np.int32)
    inp = dict(target=np.broadcast_to(t.astype(np.float32), (B, k + 1, V)).copy(),
               draft=np.broadcast_to(d.astype(np.float32), (B, k, V)).copy(), dtype="f32",
               u=rng.random((B, k), dtype=np.float32), ur=rng.random(B, dtype=np.float32),
               T=T, top_k=tk, top_p=tp)
    gpu = run_chain(inp, x, SV_MODE_SAMPLE, want_resid=False)
    first = np.bincount(gpu["out_tokens"][:, 0], minlength=V)
    acc1 = gpu["accepted_len"] >= 1
    second = np.bincount(gpu["out_tokens"][acc1, 1], minlength=V)
    for counts, probs in ((first, p[0]), (second, p[1])):
        sup = probs > 0
        assert counts[~sup].sum() == 0
        pval = scipy.stats.chisquare(counts[sup], probs[sup] * counts.sum()).pvalue
        say("  p-value", pval)
        assert pval > 1e-3
