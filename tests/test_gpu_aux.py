"""GPU parity of the steps around verification: acceptance statistics, tree
attention mask, commit map (C ABI through the binding) against oracle/aux.py.
Integer outputs and counts must match exactly; the float64 statistics to
1e-12 relative (the same formulas, rounding order aside)."""
import numpy as np
import pytest
import torch

import oracle.aux as ax
from draft_token_verification_softmax_amd import (SV_MODE_SAMPLE, SV_MODE_TREE_GREEDY,
                                                  SV_STATS_ACCEPTANCE, SV_STATS_ACCEPTED,
                                                  SV_STATS_ALPHA, SV_STATS_DRAFTED,
                                                  SV_STATS_EXPECTED_TOKENS, SV_STATS_GAMMA_BEST,
                                                  SV_STATS_MAL, SV_STATS_SEQUENCES,
                                                  SV_STATS_SPEEDUP_BEST, SV_STATS_SPEEDUP_GAMMA1,
                                                  SV_STATS_TESTED, SV_STATS_TOKENS_PER_STEP,
                                                  SpecVerify, accept_stats, tree_commit, tree_mask)
from draft_token_verification_softmax_amd import workloads as wl
from gpu_common import dev, draw_drafts, run_chain, say

pytestmark = pytest.mark.gpu

SLOTS = [("sequences", SV_STATS_SEQUENCES), ("accepted", SV_STATS_ACCEPTED),
         ("drafted", SV_STATS_DRAFTED), ("tested", SV_STATS_TESTED)]
RATES = [("acceptance", SV_STATS_ACCEPTANCE), ("mal", SV_STATS_MAL),
         ("tokens_per_step", SV_STATS_TOKENS_PER_STEP), ("alpha", SV_STATS_ALPHA),
         ("expected_tokens", SV_STATS_EXPECTED_TOKENS), ("speedup_best", SV_STATS_SPEEDUP_BEST)]


def check_stats(gpu, n, k, c, status, label):
    o = ax.accept_stats(n, k, c, status)
    for name, i in SLOTS:
        assert gpu[i] == o[name], (label, name, gpu[i], o[name])
    for name, i in RATES:
        assert abs(gpu[i] - o[name]) <= 1e-12 * max(1.0, abs(o[name])), (label, name, gpu[i], o[name])
    assert int(gpu[SV_STATS_GAMMA_BEST]) == o["gamma_best"], label
    sp = gpu[SV_STATS_SPEEDUP_GAMMA1:SV_STATS_SPEEDUP_GAMMA1 + 12]
    assert np.allclose(sp, o["speedups"], rtol=1e-12, atol=0), label


@pytest.mark.parametrize("B,k,c,with_status", [(1, 4, 0.1, False), (16, 5, 0.05, True), (5000, 8, 0.2, True),
                                                (300, 1, 0.0, False)])
def test_accept_stats_random(B, k, c, with_status):
    say("accept stats", B, k, c, with_status)
    rng = np.random.default_rng(B + k)
    n = rng.integers(0, k + 1, size=B).astype(np.int32)
    st = (rng.integers(0, 8, size=B) * (rng.random(B) < 0.2)).astype(np.int32) if with_status else None
    out = accept_stats(dev(n), k, c, dev(st) if st is not None else None)
    torch.cuda.synchronize()
    check_stats(out.cpu().numpy(), n, k, c, st, f"B={B}")


def test_accept_stats_empty_and_all_accepted():
    out = accept_stats(torch.empty(0, dtype=torch.int32, device="cuda"), 4, 0.1)
    torch.cuda.synchronize()
    check_stats(out.cpu().numpy(), np.zeros(0, np.int32), 4, 0.1, None, "empty")
    n = np.full(7, 3, np.int32)
    out = accept_stats(dev(n), 3, 0.0)
    torch.cuda.synchronize()
    check_stats(out.cpu().numpy(), n, 3, 0.0, None, "all accepted")


def test_accept_stats_of_a_verification_call():
    """The statistics of a real sampling call (workload 2 settings), with its
    own status output."""
    inp = wl.chain_inputs(2, seed=555, B=64, V=4000, k=5)
    x = draw_drafts(inp)
    res = run_chain(inp, x, SV_MODE_SAMPLE, want_resid=False)
    n, st = res["accepted_len"], res["seq_status"]
    out = accept_stats(dev(n), 5, 0.1, dev(st))
    torch.cuda.synchronize()
    check_stats(out.cpu().numpy(), n, 5, 0.1, st, "workload-2 call")


def _trees(rng, B, N, bad):
    par = np.zeros((B, N), np.int32)
    for b in range(B):
        par[b, 0] = -1
        for i in range(1, N):
            par[b, i] = rng.integers(0, i) if rng.random() < 0.6 or i < 2 else i - 1
        if bad and N > 3 and b % 2 == 1:
            par[b, rng.integers(2, N)] = rng.choice([N + 3, -2, rng.integers(0, N) + N])
    return par


@pytest.mark.parametrize("B,N,bad", [(1, 1, False), (4, 7, True), (8, 60, True), (3, 33, False),
                                     (2, 100, True), (2, 1024, True)])
def test_tree_mask(B, N, bad):
    say("tree mask", B, N, bad)
    rng = np.random.default_rng(N * 7 + B)
    par = _trees(rng, B, N, bad)
    if N == 1024:
        par[0, 1:] = np.arange(N - 1)          # a chain of 1024: depth 1023, 32 words per row
    mask, depth = tree_mask(dev(par))
    torch.cuda.synchronize()
    mask = mask.cpu().numpy().view(np.uint32)
    depth = depth.cpu().numpy()
    for b in range(B):
        m, d = ax.tree_attention_mask(par[b])
        assert np.array_equal(mask[b], m), (b, par[b])
        assert np.array_equal(depth[b], d), (b, par[b])


def test_tree_commit_after_verification():
    """Commit map from a real tree call (workload 4 shape at a small V), a
    bad-logits tree included."""
    tr = wl.tree_inputs(4, seed=9, B=6, N=60, V=3000)
    T64 = wl.rows_f64(tr["target"], "bf16")
    tokens = wl.tree_tokens(tr, np.argmax(T64, axis=-1))
    target = tr["target"].copy()
    target[5, 0, 11] = 0x7fc0                   # a NaN in the root row of tree 5: emits nothing
    t = SpecVerify(mode=SV_MODE_TREE_GREEDY, dtype="bf16", max_batch=6, k=60, vocab=3000)
    out = t.run(dev(target, "bf16"), draft_tokens=dev(tokens), parents=dev(tr["parents"]))
    pos = tree_commit(out["out_nodes"], out["accepted_len"])
    torch.cuda.synchronize()
    pos = pos.cpu().numpy()
    nodes, n = out["out_nodes"].cpu().numpy(), out["accepted_len"].cpu().numpy()
    assert (out["seq_status"].cpu().numpy()[5] & 4)
    for b in range(6):
        assert np.array_equal(pos[b], ax.tree_commit_map(nodes[b], n[b], 60)), b
    assert np.all(pos[5] == -1)
    t.close()


# ------------------------------------------------------------------ read floor

def test_read_floor_reads_every_byte():
    """The benchmark's read-floor kernel: data whose words XOR to the kernel's
    marker value make it store the marker (so the loads reach the data), any
    other data leave the sink alone; sizes of a partial last tile too."""
    import draft_token_verification_softmax_amd as svm
    marker = 0x9E3779B9
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for nbytes in (16, 16384 * 3 + 16, 1 << 20):
        t = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
        svm.read_floor(t, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) == 0, nbytes
        t[0] = np.array(marker, dtype=np.uint32).view(np.int32).item()   # one lane's four words XOR to the marker
        svm.read_floor(t, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) & 0xFFFFFFFF == marker, nbytes
        sink.zero_()
