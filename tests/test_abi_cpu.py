"""The C-ABI library on the host: it loads, exports every function the header
declares, and rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes
import math
import os
import re

import numpy as np

import pytest

import draft_token_verification_softmax_amd as svm
from draft_token_verification_softmax_amd import (
    SV_DTYPE_BF16, SV_DTYPE_F32, SV_ERR_CAPACITY, SV_ERR_DTYPE, SV_ERR_MODE, SV_ERR_NULL,
    SV_ERR_PARAM, SV_ERR_SHAPE, SV_MODE_GREEDY, SV_MODE_SAMPLE, SV_MODE_TREE_GREEDY,
    SV_MODE_TREE_SAMPLE, SV_OK,
    make_config, specverify_check_args)

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "specverify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(specverify_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = svm.load()
    names = declared_functions()
    assert len(names) == 13
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(svm.EXPORTED) == names


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ("SV_MAX_K", "SV_MAX_TREE_NODES", "SV_MAX_TOP_K"):
        m = re.search(r"#define %s (\d+)" % name, text)
        assert int(m.group(1)) == getattr(svm, name)
    for name in ("SV_ERR_NULL", "SV_ERR_SHAPE", "SV_ERR_DTYPE", "SV_ERR_PARAM", "SV_ERR_CAPACITY",
                 "SV_ERR_HIP", "SV_ERR_MODE", "SV_ERR_SCRATCH"):
        m = re.search(r"%s = (-\d+)" % name, text)
        assert int(m.group(1)) == getattr(svm, name)


def test_static_scratch_limit_is_checked_on_the_host():
    """specverify_run_static: a call whose workspace (specverify_workspace_bytes
    with max_batch = batch) exceeds SV_STATIC_SCRATCH_BYTES is refused with
    SV_ERR_SCRATCH before any HIP call; argument errors as specverify_run."""
    text = open(HEADER).read()
    m = re.search(r"#define SV_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert int(m.group(1)) << int(m.group(2)) == svm.SV_STATIC_SCRATCH_BYTES
    lib = svm.load()
    fake = ctypes.c_void_p(16)   # never dereferenced: the call returns before any HIP call
    big = make_config(SV_MODE_SAMPLE, "bf16", 512, 8, 128256, 0.7, top_k=50)
    cfg_b = make_config(SV_MODE_SAMPLE, "bf16", 512, 8, 128256, 0.7, top_k=50)
    cfg_b.max_batch = 512
    assert svm.specverify_workspace_bytes(cfg_b) > svm.SV_STATIC_SCRATCH_BYTES
    # target, draft, tokens, parents, u, ur, accepted_len, out_tokens, out_nodes, resid_probs, status
    args = [fake, fake, fake, None, fake, fake, fake, fake, None, None, None]
    assert lib.specverify_run_static(ctypes.byref(big), 512, *args, None) == svm.SV_ERR_SCRATCH
    # batch 0 is a no-op, NULL config and missing pointers are argument errors
    assert lib.specverify_run_static(ctypes.byref(big), 0, *([None] * 11), None) == SV_OK
    assert lib.specverify_run_static(None, 1, *([None] * 11), None) == SV_ERR_NULL
    assert lib.specverify_run_static(ctypes.byref(big), 1, *([None] * 11), None) == SV_ERR_NULL
    assert lib.specverify_run_static(ctypes.byref(big), 513, *args, None) == svm.SV_ERR_CAPACITY


def _tiling(cfg, batch, grid, aligned):
    out = (ctypes.c_int32 * 6)()
    rc = svm.load().specverify_tiling(ctypes.byref(cfg), batch, grid, aligned, out)
    return rc, list(out)


def test_tiling_fits_the_workspace_over_a_sweep_of_shapes():
    """The streaming pass's tiling (the host code specverify_run runs before
    any launch) fits the workspace the context sized, for every mode, dtype,
    batch, k, vocabulary, top-k, nucleus, device size and alignment of a
    seeded sweep.  A mismatch between the two once made a top-k tiling
    write more candidate lists than the workspace held (a GPU memory fault on
    V = 3000 fp32, B = 8, top_k = 20); now it would be an SV_ERR_SHAPE
    refusal, and this sweep fails on it."""
    rng = np.random.default_rng(123)
    Vs = [1, 7, 8, 9, 100, 2047, 2048, 2049, 3000, 4099, 8192, 8193, 32000, 65536, 128256, 152064,
          262144, 524288, 1 << 20, 3_000_001, 1 << 24]
    checked = 0
    cases = [(SV_MODE_SAMPLE, "f32", 8, 5, 3000, 20, 1.0)]   # the shape of the fault
    for _ in range(6000):
        mode = int(rng.choice([SV_MODE_SAMPLE, SV_MODE_GREEDY, SV_MODE_TREE_GREEDY, SV_MODE_TREE_SAMPLE]))
        dtype = str(rng.choice(["f32", "bf16"]))
        tree = mode in (SV_MODE_TREE_GREEDY, SV_MODE_TREE_SAMPLE)
        k = int(rng.choice([1, 2, 60, 200, 1024])) if tree else int(rng.choice([1, 2, 4, 5, 8, 17, 64]))
        V = int(rng.choice(Vs))
        top_k = int(rng.choice([0, 0, 1, 7, 20, 50, 64, 65, 256])) if mode == SV_MODE_SAMPLE else 0
        top_p = float(rng.choice([1.0, 1.0, 0.9, 0.5])) if mode == SV_MODE_SAMPLE else 1.0
        B = int(rng.choice([1, 2, 3, 8, 16, 64, 256, 1000]))
        if B * k * V > 1 << 33:
            B = max(1, (1 << 33) // (k * V))
        cases.append((mode, dtype, B, k, V, top_k, top_p))
    for mode, dtype, B, k, V, top_k, top_p in cases:
        cfg = make_config(mode, dtype, B, k, V, 1.0, top_k, top_p)
        for grid in (256, 1024, 2048):
            for aligned in (0, 1):
                for batch in sorted({1, max(1, B // 3), B}):
                    rc, (tm, S, L, P, cap_tiles, cap_partials) = _tiling(cfg, batch, grid, aligned)
                    assert rc == SV_OK, (mode, dtype, B, k, V, top_k, top_p, grid, aligned, batch, rc)
                    assert L % 8 == 0 and L > 0 and S >= 1
                    assert S * L >= V > (S - 1) * L, (V, S, L)
                    assert S <= cap_tiles and P <= cap_partials, (S, cap_tiles, P, cap_partials)
                    checked += 1
    assert checked > 10000


def test_tiling_rejects_bad_arguments_on_the_host():
    cfg = make_config(SV_MODE_SAMPLE, "bf16", 4, 5, 32000, 1.0)
    assert svm.load().specverify_tiling(ctypes.byref(cfg), 1, 256, 1, None) == SV_ERR_NULL
    assert _tiling(cfg, 0, 256, 1)[0] == SV_ERR_SHAPE
    assert _tiling(cfg, 5, 256, 1)[0] == svm.SV_ERR_CAPACITY
    assert _tiling(cfg, 4, 0, 1)[0] == svm.SV_ERR_PARAM


def test_lazy_rows_option_rules():
    """SV_OPT_LAZY_ROWS: plain sampling only; unknown option bits are refused."""
    lib = svm.load()
    lazy = svm.SV_OPT_LAZY_ROWS

    def ws(cfg):
        return lib.specverify_workspace_bytes(ctypes.byref(cfg))
    assert svm.sv_config.options.offset == 20
    assert ws(make_config(SV_MODE_SAMPLE, "f32", 1, 4, 32000, 1.0, options=lazy)) > 0
    for bad in (make_config(SV_MODE_SAMPLE, "f32", 1, 4, 32000, 1.0, top_k=50, options=lazy),
                make_config(SV_MODE_SAMPLE, "f32", 1, 4, 32000, 1.0, top_p=0.9, options=lazy),
                make_config(SV_MODE_GREEDY, "f32", 1, 4, 32000, options=lazy),
                make_config(SV_MODE_TREE_SAMPLE, "f32", 1, 4, 32000, 1.0, options=lazy),
                make_config(SV_MODE_SAMPLE, "f32", 1, 4, 32000, 1.0, options=2)):
        assert ws(bad) == 0
        h = ctypes.c_void_p()
        assert lib.specverify_create(ctypes.byref(bad), 0, ctypes.byref(h)) == svm.SV_ERR_PARAM
    # top_k >= V is no filter, so the option stands
    assert ws(make_config(SV_MODE_SAMPLE, "f32", 1, 4, 100, 1.0, top_k=100, options=lazy)) > 0


def test_config_struct_layout():
    assert ctypes.sizeof(svm.sv_config) == 48
    assert svm.sv_config.temperature.offset == 24 and svm.sv_config.top_p.offset == 40
    cfg = make_config(SV_MODE_SAMPLE, "bf16", 16, 5, 32000, 1.0)
    assert svm.specverify_workspace_bytes(cfg) > 0
    bad = make_config(SV_MODE_SAMPLE, "bf16", 16, 5, 32000, -1.0)
    assert svm.specverify_workspace_bytes(bad) == 0


def test_workspace_keeps_residual_weights_up_to_32_mib():
    """Small sampling contexts keep the float64 residual weights of every
    2048-logit segment for the draw; past 32 MiB of them the draw recomputes
    its segment instead, and the workspace drops by that much."""
    def ws(max_batch):
        return svm.specverify_workspace_bytes(make_config(SV_MODE_SAMPLE, "bf16", max_batch, 5, 32000, 1.0))
    per_seq = math.ceil(32000 / 2048) * 2048 * 8      # kept weights of one sequence
    assert 128 * per_seq == 32 << 20
    w127, w128, w129 = ws(127), ws(128), ws(129)
    assert w128 - w127 > per_seq                      # one more sequence, weights included
    assert w128 - w129 > 127 * per_seq                # 128 sequences' weights gone at 129
    greedy = [svm.specverify_workspace_bytes(make_config(SV_MODE_GREEDY, "bf16", b, 5, 32000, 1.0))
              for b in (1, 64, 128, 129, 4096)]
    assert all(x < y for x, y in zip(greedy, greedy[1:]))


def test_workspace_holds_a_nucleus_candidate_buffer_per_row():
    """Chain sampling with top-p alone: a context's workspace holds one 192 KB
    candidate buffer per row (the residual kernel reads the target rows' kept
    entries there), plus a record per row, wave and 4096-logit round; so it
    grows by at least a row's buffer per row of max_batch."""
    buf = 24576 * 8
    def ws(max_batch, top_p=0.9):
        return svm.specverify_workspace_bytes(make_config(SV_MODE_SAMPLE, "f32", max_batch, 4, 152064, 0.8,
                                                          top_p=top_p))
    rows_per_seq = 4 + 5
    w1, w2, w256 = ws(1), ws(2), ws(256)
    assert w2 - w1 >= rows_per_seq * buf
    assert w256 >= 256 * rows_per_seq * buf              # workload 5: 453 MB of buffers
    rounds = math.ceil(152064 / 4096)
    assert w2 - w1 >= rows_per_seq * (buf + 4 * rounds * 8)
    assert ws(256, top_p=1.0) < 256 * rows_per_seq * buf  # no nucleus, no buffers


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert svm.specverify_status_string(st).startswith("SV_")
    assert svm.specverify_status_string(-99) == "unknown status"


P = 0x1000  # any non-NULL address: check_args never dereferences


def sample_args(**over):
    a = dict(target=P, draft=P, draft_tokens=P, parents=None, uniforms=P, resid_uniforms=P,
             accepted_len=P, out_tokens=P, out_nodes=None)
    a.update(over)
    return a


def check(cfg, batch=4, **args):
    a = sample_args(**args)
    return specverify_check_args(cfg, batch, a["target"], a["draft"], a["draft_tokens"], a["parents"],
                                 a["uniforms"], a["resid_uniforms"], a["accepted_len"],
                                 a["out_tokens"], a["out_nodes"])


@pytest.mark.parametrize("over,want", [
    (dict(), SV_OK),
    (dict(mode=7), SV_ERR_MODE),
    (dict(dtype=5), SV_ERR_DTYPE),
    (dict(max_batch=0), SV_ERR_SHAPE),
    (dict(vocab=0), SV_ERR_SHAPE),
    (dict(vocab=(1 << 24) + 1), SV_ERR_SHAPE),
    (dict(k=0), SV_ERR_SHAPE),
    (dict(k=65), SV_ERR_SHAPE),
    (dict(temperature=0.0), SV_ERR_PARAM),
    (dict(temperature=-0.5), SV_ERR_PARAM),
    (dict(temperature=math.nan), SV_ERR_PARAM),
    (dict(temperature=math.inf), SV_ERR_PARAM),
    (dict(top_k=-1), SV_ERR_PARAM),
    (dict(top_k=257), SV_ERR_PARAM),
    (dict(top_k=32000), SV_OK),            # >= V acts as off
    (dict(top_k=256), SV_OK),
    (dict(top_p=0.0), SV_ERR_PARAM),
    (dict(top_p=1.5), SV_ERR_PARAM),
    (dict(top_p=math.nan), SV_ERR_PARAM),
    (dict(top_p=1.0), SV_OK),
    (dict(top_p=0.9, top_k=50), SV_OK),
])
def test_sample_config_validation(over, want):
    base = dict(mode=SV_MODE_SAMPLE, dtype=SV_DTYPE_BF16, max_batch=8, k=5, vocab=32000,
                temperature=1.0, top_k=0, top_p=1.0)
    base.update(over)
    cfg = make_config(**base)
    assert check(cfg) == want


def test_greedy_modes_ignore_sampling_settings():
    cfg = make_config(SV_MODE_GREEDY, SV_DTYPE_F32, 2, 4, 100, temperature=-1.0, top_k=-3, top_p=7.0)
    assert check(cfg, batch=2, draft=None, uniforms=None, resid_uniforms=None) == SV_OK
    tree = make_config(SV_MODE_TREE_GREEDY, SV_DTYPE_BF16, 2, 1024, 100, temperature=0.0)
    assert check(tree, batch=2, draft=None, uniforms=None, resid_uniforms=None, parents=P) == SV_OK
    tree = make_config(SV_MODE_TREE_GREEDY, SV_DTYPE_BF16, 2, 1025, 100)
    assert check(tree, batch=2, draft=None, uniforms=None, resid_uniforms=None, parents=P) == SV_ERR_SHAPE


def test_batch_and_pointer_rules():
    cfg = make_config(SV_MODE_SAMPLE, "f32", 8, 4, 1000)
    assert check(cfg, batch=0) == SV_OK
    assert check(cfg, batch=0, target=None, draft=None, draft_tokens=None, uniforms=None,
                 resid_uniforms=None, accepted_len=None, out_tokens=None) == SV_OK
    assert check(cfg, batch=8) == SV_OK
    assert check(cfg, batch=9) == SV_ERR_CAPACITY
    assert check(cfg, batch=-1) == SV_ERR_SHAPE
    for name in ("target", "draft", "draft_tokens", "uniforms", "resid_uniforms", "accepted_len", "out_tokens"):
        assert check(cfg, **{name: None}) == SV_ERR_NULL, name
    assert check(cfg, parents=P) == SV_ERR_MODE
    assert check(cfg, out_nodes=P) == SV_ERR_MODE
    g = make_config(SV_MODE_GREEDY, "f32", 8, 4, 1000)
    ok = dict(draft=None, uniforms=None, resid_uniforms=None)
    assert check(g, **ok) == SV_OK
    for name in ("draft", "uniforms", "resid_uniforms", "parents", "out_nodes"):
        kw = dict(ok)
        kw[name] = P
        assert check(g, **kw) == SV_ERR_MODE, name
    t = make_config(SV_MODE_TREE_GREEDY, "bf16", 8, 60, 1000)
    assert check(t, parents=None, **ok) == SV_ERR_NULL
    assert check(t, parents=P, out_nodes=P, **ok) == SV_OK
    assert check(t, parents=P, draft=P, uniforms=None, resid_uniforms=None) == SV_ERR_MODE


def test_tree_sample_rules():
    t = make_config(SV_MODE_TREE_SAMPLE, "bf16", 8, 60, 1000, temperature=0.8)
    assert check(t, parents=P) == SV_OK
    assert check(t, parents=P, out_nodes=P) == SV_OK
    for name in ("parents", "draft", "uniforms", "resid_uniforms", "target", "draft_tokens"):
        kw = dict(parents=P)
        kw[name] = None
        assert check(t, **kw) == SV_ERR_NULL, name
    assert check(make_config(SV_MODE_TREE_SAMPLE, "bf16", 8, 1024, 1000), parents=P) == SV_OK
    assert check(make_config(SV_MODE_TREE_SAMPLE, "bf16", 8, 1025, 1000), parents=P) == SV_ERR_SHAPE
    # top-k and top-p as in chain sampling; top_k >= V means off
    assert check(make_config(SV_MODE_TREE_SAMPLE, "bf16", 8, 60, 1000, top_k=50), parents=P) == SV_OK
    assert check(make_config(SV_MODE_TREE_SAMPLE, "bf16", 8, 60, 1000, top_p=0.9), parents=P) == SV_OK
    assert check(make_config(SV_MODE_TREE_SAMPLE, "bf16", 8, 60, 1000, top_k=257), parents=P) == SV_ERR_PARAM
    assert check(make_config(SV_MODE_TREE_SAMPLE, "bf16", 8, 60, 1000, top_p=1.5), parents=P) == SV_ERR_PARAM
    assert check(make_config(SV_MODE_TREE_SAMPLE, "bf16", 8, 60, 1000, top_k=1000), parents=P) == SV_OK
    for f in (dict(top_k=50), dict(top_p=0.9), dict(top_k=20, top_p=0.8)):
        assert svm.load().specverify_workspace_bytes(
            ctypes.byref(make_config(SV_MODE_TREE_SAMPLE, "bf16", 8, 60, 128256, **f))) > 0
    assert check(make_config(SV_MODE_TREE_SAMPLE, "bf16", 8, 60, 1000, temperature=0.0), parents=P) == SV_ERR_PARAM
    assert svm.load().specverify_workspace_bytes(ctypes.byref(t)) > 0


def test_null_config_and_bad_create_make_no_hip_call():
    lib = svm.load()
    assert lib.specverify_check_args(None, 1, *([None] * 9)) == SV_ERR_NULL
    h = ctypes.c_void_p()
    bad = make_config(SV_MODE_SAMPLE, "bf16", 1, 5, 100, temperature=0.0)
    assert lib.specverify_create(ctypes.byref(bad), 0, ctypes.byref(h)) == SV_ERR_PARAM
    assert h.value is None
    assert lib.specverify_create(ctypes.byref(bad), 0, None) == SV_ERR_NULL
    lib.specverify_destroy(None)   # NULL-safe


def test_run_rejects_null_context():
    lib = svm.load()
    assert lib.specverify_run(None, 1, *([None] * 11), None) == SV_ERR_NULL
    assert lib.specverify_profile_events(None, None, None, None) == SV_ERR_NULL


def test_read_floor_checks_arguments_on_the_host():
    """Argument errors come back before any HIP call (no GPU needed)."""
    lib = svm.load()
    assert lib.specverify_read_floor(None, 0, None, None) == SV_OK          # nothing to read
    assert lib.specverify_read_floor(None, 64, None, None) == SV_ERR_NULL
    assert lib.specverify_read_floor(None, -16, None, None) == SV_ERR_SHAPE
    assert lib.specverify_read_floor(16, 24, 64, None) == SV_ERR_SHAPE        # bytes not a multiple of 16
    assert lib.specverify_read_floor(8, 32, 64, None) == SV_ERR_SHAPE         # src not 16-byte aligned


def test_stats_layout_matches_header():
    text = open(HEADER).read()
    for name in ("SV_STATS_SEQUENCES", "SV_STATS_ACCEPTED", "SV_STATS_DRAFTED", "SV_STATS_TESTED",
                 "SV_STATS_ACCEPTANCE", "SV_STATS_MAL", "SV_STATS_TOKENS_PER_STEP", "SV_STATS_ALPHA",
                 "SV_STATS_EXPECTED_TOKENS", "SV_STATS_GAMMA_BEST", "SV_STATS_SPEEDUP_BEST",
                 "SV_STATS_SPEEDUP_GAMMA1", "SV_STATS_LEN"):
        m = re.search(r"%s = (\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(svm, name), name


def test_aux_entry_points_reject_bad_arguments_on_the_host():
    """Argument errors come back before any HIP call (so no GPU is needed)."""
    lib = svm.load()
    stats, mask, commit = lib.specverify_accept_stats, lib.specverify_tree_mask, lib.specverify_tree_commit
    assert stats(P, None, 4, 4, 0.1, None, None) == SV_ERR_NULL           # no output
    assert stats(None, None, 4, 4, 0.1, P, None) == SV_ERR_NULL           # no input with batch > 0
    assert stats(P, None, -1, 4, 0.1, P, None) == SV_ERR_SHAPE
    assert stats(P, None, 4, 0, 0.1, P, None) == SV_ERR_SHAPE             # k >= 1
    assert stats(P, None, 4, 4, -0.5, P, None) == SV_ERR_PARAM
    assert stats(P, None, 4, 4, float("nan"), P, None) == SV_ERR_PARAM
    assert stats(P, None, 4, 4, float("inf"), P, None) == SV_ERR_PARAM
    assert mask(P, 2, 0, P, None, None) == SV_ERR_SHAPE
    assert mask(P, 2, 1025, P, None, None) == SV_ERR_SHAPE
    assert mask(P, -1, 10, P, None, None) == SV_ERR_SHAPE
    assert mask(None, 2, 10, P, None, None) == SV_ERR_NULL
    assert mask(P, 2, 10, None, None, None) == SV_ERR_NULL
    assert mask(None, 0, 10, None, None, None) == SV_OK                  # empty batch: nothing to do
    assert commit(P, P, 2, 0, P, None) == SV_ERR_SHAPE
    assert commit(None, P, 2, 10, P, None) == SV_ERR_NULL
    assert commit(P, None, 2, 10, P, None) == SV_ERR_NULL
    assert commit(P, P, 2, 10, None, None) == SV_ERR_NULL
    assert commit(None, None, 0, 10, None, None) == SV_OK
