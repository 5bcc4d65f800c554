"""Token-tree sampling verification on the GPU against the oracle
(oracle/tree_sample.py, readings R24-R27), through the C ABI.

Comparison rule as the chain's (reading R14): accepted length, emitted
tokens, path nodes and status equal on every tree the oracle does not flag;
the distribution of the last draw within 1e-5 absolute on every tree.
"""
import numpy as np
import pytest
import scipy.stats
import torch

import oracle.tree_sample as ts
import oracle.verify as ov
from draft_token_verification_softmax_amd import (SV_MODE_SAMPLE, SV_MODE_TREE_SAMPLE, SpecVerify)
from draft_token_verification_softmax_amd import workloads as wl
from gpu_common import RESID_TOL, dev, say

pytestmark = pytest.mark.gpu


def tree_tokens(inp, parents=None):
    """Node i's token drawn from the draft's adjusted row at its parent (the
    draft model's own draw, through the oracle's distribution)."""
    parents = inp["parents"] if parents is None else parents
    B, N = parents.shape
    d64 = wl.rows_f64(inp["draft"], inp["dtype"])
    tok = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        qs = {}
        for i in range(1, N):
            par = int(parents[b, i])
            if not (0 <= par < i):
                continue
            if par not in qs:
                qs[par] = ov.transform_row(d64[b, par], inp["T"], inp.get("top_k", 0), inp.get("top_p", 1.0))
            tok[b, i] = ov.draw_from(qs[par], inp["draw_u"][b, i])
    return tok


def run_gpu(inp, tok, parents=None, want_resid=True):
    parents = inp["parents"] if parents is None else parents
    B, N, V = inp["target"].shape
    sv = SpecVerify(mode=SV_MODE_TREE_SAMPLE, dtype=inp["dtype"], max_batch=B, k=N, vocab=V,
                    temperature=inp["T"], top_k=inp.get("top_k", 0), top_p=inp.get("top_p", 1.0))
    out = sv.run(dev(inp["target"], inp["dtype"]), dev(inp["draft"], inp["dtype"]), dev(tok.astype(np.int32)),
                 dev(inp["u"]), dev(inp["ur"]), parents=dev(parents.astype(np.int32)),
                 want_resid_probs=want_resid)
    torch.cuda.synchronize()
    res = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
    sv.close()
    return res


def run_oracle(inp, tok, which, parents=None):
    parents = inp["parents"] if parents is None else parents
    T64 = wl.rows_f64(inp["target"], inp["dtype"])
    D64 = wl.rows_f64(inp["draft"], inp["dtype"])
    acc, toks, nodes, st, flagged, resid = ts.run_tree_sample_batch(
        T64, D64, parents, tok, inp["u"], inp["ur"], inp["T"], inp.get("top_k", 0), inp.get("top_p", 1.0),
        want_resid=True, which=which)
    return dict(accepted_len=acc, out_tokens=toks, out_nodes=nodes, seq_status=st, flagged=flagged,
                resid=resid)


def compare(gpu, orc, which, label):
    mism, unflagged = [], []
    for b in which:
        same = (gpu["accepted_len"][b] == orc["accepted_len"][b]
                and np.array_equal(gpu["out_tokens"][b], orc["out_tokens"][b])
                and np.array_equal(gpu["out_nodes"][b], orc["out_nodes"][b])
                and gpu["seq_status"][b] == orc["seq_status"][b])
        if not same:
            mism.append(b)
            if not orc["flagged"][b]:
                unflagged.append((b, int(gpu["accepted_len"][b]), gpu["out_tokens"][b][:8].tolist(),
                                  gpu["out_nodes"][b][:8].tolist(), int(gpu["seq_status"][b]),
                                  int(orc["accepted_len"][b]), orc["out_tokens"][b][:8].tolist(),
                                  orc["out_nodes"][b][:8].tolist(), int(orc["seq_status"][b])))
    diff = np.abs(gpu["resid_probs"][which].astype(np.float64) - orc["resid"][which])
    rep = dict(checked=len(which), mismatches=len(mism), flagged=int(np.sum(orc["flagged"][which])),
               resid_max_abs=float(diff.max()) if diff.size else 0.0,
               mean_len=float(np.mean(gpu["accepted_len"][which])))
    say(label, rep)
    assert not unflagged, f"{label}: unflagged mismatches: {unflagged[:3]}"
    assert len(mism) <= 1e-4 * len(which), f"{label}: {len(mism)} flagged mismatches"
    assert rep["resid_max_abs"] <= RESID_TOL, rep
    return rep


@pytest.mark.parametrize("B,N,V,dtype,T,mc", [
    (16, 12, 3000, "bf16", 1.0, 4),
    (16, 12, 3000, "f32", 0.7, 4),
    (12, 30, 5003, "bf16", 1.0, 8),     # wide nodes: more rejections than the precomputed passes
    (8, 20, 4000, "f32", 1.0, 1),       # path-shaped trees
    (10, 2, 2048, "bf16", 1.0, 4),
    (10, 1, 2048, "f32", 1.0, 4),       # a root alone: the bonus draw
    # more nodes with children than one launch's workgroups take in one
    # batch each (a workgroup then runs several batches of its pass)
    (6, 80, 2048, "bf16", 1.0, 1),
    (6, 120, 2048, "f32", 1.0, 2),
    (2, 1024, 1024, "bf16", 1.0, 4),    # the largest tree the API takes
    (8, 30, 3000, "bf16", 0.05, 4),     # near one-hot rows
    (8, 30, 3000, "f32", 4.0, 4),       # flat rows: long accepted paths
])
def test_tree_sample_parity(B, N, V, dtype, T, mc):
    say("tree sample", B, N, V, dtype, T, mc)
    inp = wl.tree_sample_inputs(seed=31 + N + V, B=B, N=N, V=V, dtype=dtype, T=T, max_children=mc,
                                max_depth=N if mc == 1 else 6)
    tok = tree_tokens(inp)
    gpu = run_gpu(inp, tok)
    orc = run_oracle(inp, tok, range(B))
    compare(gpu, orc, list(range(B)), f"tree sample N={N} V={V} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tree_sample_close_draft(dtype):
    """Draft rows that track their targets closely (noise sd 0.05): after a
    rejected child the running residual holds a few percent of the mass, and
    every further test and the draw divide by it."""
    say("tree sample close draft", dtype)
    inp = wl.tree_sample_inputs(seed=808, B=24, N=30, V=32000, dtype=dtype, noise=0.05)
    tok = tree_tokens(inp)
    gpu = run_gpu(inp, tok)
    orc = run_oracle(inp, tok, range(24))
    compare(gpu, orc, list(range(24)), f"tree sample close draft {dtype}")


@pytest.mark.parametrize("B,N,V,dtype,T,top_k,top_p", [
    (16, 12, 3000, "bf16", 1.0, 20, 1.0),
    (16, 12, 3000, "f32", 0.7, 0, 0.8),
    (12, 30, 5003, "bf16", 1.0, 50, 0.9),     # ragged rows, top-k then nucleus
    (8, 30, 3000, "f32", 1.0, 1, 1.0),        # top-k 1: one token per row
    (8, 24, 4096, "bf16", 1.0, 256, 1.0),     # the largest top-k (block merge)
    (8, 60, 128256, "bf16", 1.0, 50, 1.0),    # the sampled-tree workload's shape, top-k 50
    (8, 60, 128256, "bf16", 1.0, 0, 0.9),     # the same, nucleus 0.9
    (32, 3, 8, "f32", 1.0, 3, 1.0),           # tiny rows: the filter pass's bound is -inf
    (16, 5, 20, "bf16", 1.0, 10, 0.9),
])
def test_tree_sample_filters(B, N, V, dtype, T, top_k, top_p):
    """Top-k and nucleus applied to every target and draft row of the tree
    before the tests (the adjusted distributions of the chain modes)."""
    say("tree sample filters", B, N, V, dtype, T, top_k, top_p)
    inp = wl.tree_sample_inputs(seed=57 + N + V + top_k, B=B, N=N, V=V, dtype=dtype, T=T)
    inp["top_k"], inp["top_p"] = top_k, top_p
    tok = tree_tokens(inp)
    gpu = run_gpu(inp, tok)
    orc = run_oracle(inp, tok, range(B))
    compare(gpu, orc, list(range(B)), f"tree sample N={N} V={V} {dtype} top-k {top_k} top-p {top_p}")


@pytest.mark.parametrize("top_k,top_p", [(0, 1.0), (3, 1.0), (0, 0.7)])
def test_tree_sample_emitted_token_law_chisq(top_k, top_p):
    """A root with two children drafted independently from q'_root (V = 8),
    the same logits in 40000 trees with fresh uniforms: the first emitted
    token follows p'_root."""
    say("tree chi-square", top_k, top_p)
    rng = np.random.default_rng(23 + top_k)
    V, N, B = 8, 3, 40000
    t = rng.normal(0, 1.0, size=(N, V))
    d = t + rng.normal(0, 1.0, size=(N, V))
    p0 = ov.transform_row(t[0].astype(np.float32).astype(np.float64), 1.0, top_k, top_p)
    q0 = ov.transform_row(d[0].astype(np.float32).astype(np.float64), 1.0, top_k, top_p)
    tok = np.zeros((B, N), np.int32)
    for b in range(B):
        tok[b, 1] = ov.draw_from(q0, rng.random())
        tok[b, 2] = ov.draw_from(q0, rng.random())
    inp = dict(target=np.broadcast_to(t.astype(np.float32), (B, N, V)).copy(),
               draft=np.broadcast_to(d.astype(np.float32), (B, N, V)).copy(), dtype="f32",
               parents=np.tile(np.array([-1, 0, 0], np.int32), (B, 1)),
               u=rng.random((B, N), dtype=np.float32), ur=rng.random(B, dtype=np.float32),
               T=1.0, top_k=top_k, top_p=top_p)
    gpu = run_gpu(inp, tok, want_resid=False)
    counts = np.bincount(gpu["out_tokens"][:, 0], minlength=V)
    sup = p0 > 0
    assert counts[~sup].sum() == 0
    pval = scipy.stats.chisquare(counts[sup], p0[sup] * counts.sum()).pvalue
    say("  p-value", pval, "mean accepted", float(gpu["accepted_len"].mean()))
    assert pval > 1e-3


def test_tree_sample_full_size():
    say("tree sample 8 x 60 nodes, V=128256 bf16")
    inp = wl.tree_sample_inputs()
    tok = tree_tokens(inp)
    gpu = run_gpu(inp, tok)
    orc = run_oracle(inp, tok, range(inp["B"]))
    rep = compare(gpu, orc, list(range(inp["B"])), "tree sample full size")
    assert rep["mean_len"] > 0.0


def test_tree_sample_path_equals_chain():
    """A path-shaped tree through the tree mode gives the chain mode's answer."""
    say("path tree vs chain")
    B, k, V = 16, 6, 3000
    inp = wl.tree_sample_inputs(seed=77, B=B, N=k + 1, V=V, dtype="bf16", max_children=1)
    tok = tree_tokens(inp)
    gpu_t = run_gpu(inp, tok)
    sv = SpecVerify(mode=SV_MODE_SAMPLE, dtype="bf16", max_batch=B, k=k, vocab=V, temperature=1.0)
    out = sv.run(dev(inp["target"], "bf16"), dev(np.ascontiguousarray(inp["draft"][:, :k]), "bf16"),
                 dev(np.ascontiguousarray(tok[:, 1:])), dev(np.ascontiguousarray(inp["u"][:, 1:])),
                 dev(inp["ur"]), want_resid_probs=True)
    torch.cuda.synchronize()
    acc_c = out["accepted_len"].cpu().numpy()
    tok_c = out["out_tokens"].cpu().numpy()
    rp_c = out["resid_probs"].cpu().numpy()
    sv.close()
    orc = run_oracle(inp, tok, range(B))
    for b in range(B):
        if orc["flagged"][b]:
            continue
        n = acc_c[b]
        assert gpu_t["accepted_len"][b] == n
        assert np.array_equal(gpu_t["out_tokens"][b][:n + 1], tok_c[b][:n + 1])
        assert np.abs(gpu_t["resid_probs"][b].astype(np.float64) - rp_c[b]).max() <= RESID_TOL


def test_tree_sample_identical_rows():
    """q = p: every first child is accepted (ratio 1), so the walk follows
    first children to a leaf and draws the bonus there."""
    say("tree sample q == p")
    inp = wl.tree_sample_inputs(seed=5, B=8, N=24, V=2048, dtype="bf16")
    inp["draft"] = inp["target"].copy()
    tok = tree_tokens(inp)
    gpu = run_gpu(inp, tok)
    orc = run_oracle(inp, tok, range(8))
    compare(gpu, orc, list(range(8)), "q == p")
    for b in range(8):
        node, n = 0, 0
        while True:
            kids = [i for i in range(1, 24) if inp["parents"][b, i] == node]
            if not kids:
                break
            node, n = kids[0], n + 1
        assert gpu["accepted_len"][b] == n


def test_tree_sample_bad_data():
    say("tree sample bad data")
    B, N, V = 8, 16, 2048
    inp = wl.tree_sample_inputs(seed=9, B=B, N=N, V=V, dtype="f32")
    parents = inp["parents"].copy()
    tok = tree_tokens(inp)
    t, d = inp["target"], inp["draft"]
    leaf = [i for i in range(1, N) if not (parents[1] == i).any()][0]
    t[0, 3, 11] = np.nan                    # a target row: the tree emits nothing
    d[1, leaf, 5] = np.nan                  # a leaf's draft row is never read
    inner = int(parents[2, N - 1])
    d[2, inner, 7] = np.inf                 # the draft row of a node with a child
    tok[3, 1] = V + 5                       # a token outside the vocabulary
    parents[4, N - 1] = N + 3               # a bad parent
    parents[5, 0] = 7                       # the root's parent is not -1
    tok = np.where(tok < 0, 0, tok)
    gpu = run_gpu(inp, tok, parents=parents)
    orc = run_oracle(inp, tok, range(B), parents=parents)
    compare(gpu, orc, list(range(B)), "bad data")
    assert list(gpu["seq_status"][:6]) == [4, 0, 4, orc["seq_status"][3], orc["seq_status"][4],
                                           orc["seq_status"][5]]
    assert gpu["seq_status"][3] & 1 and gpu["seq_status"][4] & 2 and gpu["seq_status"][5] & 2
    assert (gpu["out_tokens"][0] == -1).all() and gpu["accepted_len"][0] == 0


def test_tree_sample_without_resid_probs():
    inp = wl.tree_sample_inputs(seed=4, B=8, N=30, V=4096, dtype="bf16")
    tok = tree_tokens(inp)
    a = run_gpu(inp, tok, want_resid=True)
    b = run_gpu(inp, tok, want_resid=False)
    for key in ("accepted_len", "out_tokens", "out_nodes", "seq_status"):
        assert np.array_equal(a[key], b[key]), key


def test_tree_sample_deterministic():
    inp = wl.tree_sample_inputs(seed=3, B=8, N=30, V=4096, dtype="bf16")
    tok = tree_tokens(inp)
    a = run_gpu(inp, tok)
    b = run_gpu(inp, tok)
    for key in ("accepted_len", "out_tokens", "out_nodes", "seq_status", "resid_probs"):
        assert np.array_equal(a[key], b[key]), key
