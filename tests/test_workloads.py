"""Seeded workload generators (CPU only)."""
import numpy as np
import torch

from draft_token_verification_softmax_amd import workloads as wl


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    x = rng.normal(0, 5, size=200000).astype(np.float32)
    x[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0]  # exact ties
    ours = wl.bf16_from_f64(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_direct_rounding_avoids_double_rounding():
    # 1 + 2^-8 + 2^-30 is just above a bf16 tie; fp32 would round it onto the tie first
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30])
    assert wl.bf16_to_f32(wl.bf16_from_f64(x))[0] == np.float32(1.0 + 2.0 ** -7)


def test_chain_inputs_deterministic_and_shaped():
    a = wl.chain_inputs(2, seed=5, B=3, V=1000)
    b = wl.chain_inputs(2, seed=5, B=3, V=1000)
    assert a["target"].shape == (3, 6, 1000) and a["draft"].shape == (3, 5, 1000)
    assert a["target"].dtype == np.uint16 and a["u"].dtype == np.float32
    for key in ("target", "draft", "u", "ur", "draw_u"):
        assert np.array_equal(a[key], b[key])
    assert np.all((a["u"] >= 0) & (a["u"] < 1)) and np.all((a["ur"] >= 0) & (a["ur"] < 1))
    t = wl.rows_f64(a["target"], "bf16")
    # five boosted tokens per row: the top five sit well above the rest on average
    top = np.sort(t, axis=-1)[..., -5:]
    assert np.mean(top) > 8.0


def test_zipf_rows_are_permuted_log_rank_decay():
    a = wl.chain_inputs(3, seed=1, B=2, V=5000, k=2)
    t = wl.rows_f64(a["target"], "bf16")
    s = -np.sort(-t, axis=-1)
    # sorted values decay at least like -ln(rank) on top of a sorted Gaussian
    assert np.all(s[..., 0] - s[..., 999] > np.log(1000) - 0.5)
    # and the positions are scrambled (the maximum is not at index 0)
    assert not np.all(np.argmax(t, axis=-1) == 0)


def test_tree_shape_limits_and_planting():
    tr = wl.tree_inputs(4, seed=3, B=4, V=500)
    P = tr["parents"]
    assert P.shape == (4, 60) and np.all(P[:, 0] == -1)
    for b in range(4):
        depth = np.zeros(60, dtype=int)
        for i in range(1, 60):
            assert 0 <= P[b, i] < i
            depth[i] = depth[P[b, i]] + 1
        assert depth.max() <= 6
        assert np.bincount(P[b, 1:], minlength=60).max() <= 4
    g = np.random.default_rng(0).integers(0, 500, size=(4, 60))
    toks = wl.tree_tokens(tr, g)
    for b in range(4):
        for p in range(60):
            kids = [i for i in range(1, 60) if P[b, i] == p]
            vals = [toks[b, i] for i in kids]
            assert len(set(vals)) == len(vals)                   # distinct siblings
            planted = tr["plant"][b, p]
            for i in kids:
                assert (toks[b, i] == g[b, p]) == (i == planted)
