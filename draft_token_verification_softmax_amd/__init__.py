"""Python binding of libspecverify (the MI355X verification step of
speculative decoding).

The functions below carry the C ABI's names (include/specverify.h) and only
marshal arguments: torch tensors become device pointers, the current HIP
stream is passed along, status codes become exceptions.  Every step of the
computation runs in the library's HIP kernels; there is no other code path.
If the shared library is missing, ``load()`` raises instead of falling back.

    from draft_token_verification_softmax_amd import SpecVerify, SV_MODE_SAMPLE
    sv = SpecVerify(mode=SV_MODE_SAMPLE, dtype="bf16", max_batch=16, k=5, vocab=32000,
                    temperature=1.0)
    out = sv.run(target, draft, draft_tokens, uniforms, resid_uniforms)
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecverify.so")

SV_MODE_SAMPLE, SV_MODE_GREEDY, SV_MODE_TREE_GREEDY, SV_MODE_TREE_SAMPLE = 0, 1, 2, 3
SV_DTYPE_F32, SV_DTYPE_BF16 = 0, 1
SV_OK, SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_DTYPE, SV_ERR_PARAM = 0, -1, -2, -3, -4
SV_ERR_CAPACITY, SV_ERR_HIP, SV_ERR_MODE, SV_ERR_SCRATCH = -5, -6, -7, -8
SV_STATIC_SCRATCH_BYTES = 64 << 20
SV_STATUS_BAD_TOKEN, SV_STATUS_BAD_PARENT, SV_STATUS_BAD_LOGITS = 1, 2, 4
SV_OPT_LAZY_ROWS = 1
SV_MAX_K, SV_MAX_TREE_NODES, SV_MAX_TOP_K, SV_MAX_VOCAB = 64, 1024, 256, 1 << 24

EXPORTED = ("specverify_create", "specverify_check_args", "specverify_run", "specverify_run_static",
            "specverify_tiling",
            "specverify_destroy", "specverify_profile_events", "specverify_status_string",
            "specverify_workspace_bytes", "specverify_accept_stats", "specverify_tree_mask",
            "specverify_tree_commit", "specverify_read_floor")

# Slots of specverify_accept_stats' output (SV_STATS_* of the header).
SV_STATS_SEQUENCES, SV_STATS_ACCEPTED, SV_STATS_DRAFTED, SV_STATS_TESTED = 0, 1, 2, 3
SV_STATS_ACCEPTANCE, SV_STATS_MAL, SV_STATS_TOKENS_PER_STEP, SV_STATS_ALPHA = 4, 5, 6, 7
SV_STATS_EXPECTED_TOKENS, SV_STATS_GAMMA_BEST, SV_STATS_SPEEDUP_BEST = 8, 9, 10
SV_STATS_SPEEDUP_GAMMA1, SV_STATS_LEN = 11, 23


class sv_config(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("max_batch", ctypes.c_int32), ("k", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("options", ctypes.c_int32), ("temperature", ctypes.c_double),
                ("top_k", ctypes.c_int32), ("top_p", ctypes.c_double)]


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {specverify_status_string(status)}" if what else
                         specverify_status_string(status))


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the shared library once.  Raises OSError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is not built; run python -m draft_token_verification_softmax_amd.build")
    # torch carries its own HIP runtime under the same soname; loading torch
    # first makes this library bind to that one, so the process has a single
    # runtime (two would each claim the device)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, P = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER
    lib.specverify_create.argtypes = [P(sv_config), ctypes.c_int, P(vp)]
    lib.specverify_create.restype = ctypes.c_int
    lib.specverify_check_args.argtypes = [P(sv_config), i32] + [vp] * 9
    lib.specverify_check_args.restype = ctypes.c_int
    lib.specverify_run.argtypes = [vp, i32] + [vp] * 11 + [vp]
    lib.specverify_run.restype = ctypes.c_int
    lib.specverify_run_static.argtypes = [P(sv_config), i32] + [vp] * 11 + [vp]
    lib.specverify_run_static.restype = ctypes.c_int
    lib.specverify_tiling.argtypes = [P(sv_config), i32, i32, i32, P(i32)]
    lib.specverify_tiling.restype = ctypes.c_int
    lib.specverify_destroy.argtypes = [vp]
    lib.specverify_destroy.restype = None
    lib.specverify_profile_events.argtypes = [vp, vp, vp, vp]
    lib.specverify_profile_events.restype = ctypes.c_int
    lib.specverify_status_string.argtypes = [ctypes.c_int]
    lib.specverify_status_string.restype = ctypes.c_char_p
    lib.specverify_workspace_bytes.argtypes = [P(sv_config)]
    lib.specverify_workspace_bytes.restype = ctypes.c_size_t
    lib.specverify_accept_stats.argtypes = [vp, vp, i32, i32, ctypes.c_double, vp, vp]
    lib.specverify_accept_stats.restype = ctypes.c_int
    lib.specverify_tree_mask.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.specverify_tree_mask.restype = ctypes.c_int
    lib.specverify_tree_commit.argtypes = [vp, vp, i32, i32, vp, vp]
    lib.specverify_tree_commit.restype = ctypes.c_int
    lib.specverify_read_floor.argtypes = [vp, ctypes.c_int64, vp, vp]
    lib.specverify_read_floor.restype = ctypes.c_int
    _lib = lib
    return lib


def make_config(mode, dtype, max_batch, k, vocab, temperature=1.0, top_k=0, top_p=1.0,
                options=0) -> sv_config:
    if isinstance(dtype, str):
        dtype = {"f32": SV_DTYPE_F32, "float32": SV_DTYPE_F32, "bf16": SV_DTYPE_BF16,
                 "bfloat16": SV_DTYPE_BF16}[dtype]
    return sv_config(int(mode), int(dtype), int(max_batch), int(k), int(vocab), int(options),
                     float(temperature), int(top_k), float(top_p))


def _ptr(x):
    """Device pointer of a tensor (or an int address, or None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


# ------------------------------------------------------------------ C ABI names

def specverify_status_string(status: int) -> str:
    return load().specverify_status_string(int(status)).decode()


def specverify_workspace_bytes(cfg: sv_config) -> int:
    return int(load().specverify_workspace_bytes(ctypes.byref(cfg)))


def specverify_check_args(cfg: sv_config, batch, target, draft, draft_tokens, parents,
                          uniforms, resid_uniforms, accepted_len, out_tokens, out_nodes) -> int:
    return int(load().specverify_check_args(
        ctypes.byref(cfg), int(batch), _ptr(target), _ptr(draft), _ptr(draft_tokens),
        _ptr(parents), _ptr(uniforms), _ptr(resid_uniforms), _ptr(accepted_len),
        _ptr(out_tokens), _ptr(out_nodes)))


def specverify_create(cfg: sv_config, device: int = 0) -> int:
    h = ctypes.c_void_p()
    st = load().specverify_create(ctypes.byref(cfg), int(device), ctypes.byref(h))
    if st != SV_OK:
        raise SpecVerifyError(st, "specverify_create")
    return h.value


def specverify_run(ctx: int, batch, target, draft, draft_tokens, parents, uniforms,
                   resid_uniforms, accepted_len, out_tokens, out_nodes=None,
                   resid_probs=None, seq_status=None, stream=None) -> None:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    st = load().specverify_run(
        ctypes.c_void_p(ctx), int(batch), _ptr(target), _ptr(draft), _ptr(draft_tokens),
        _ptr(parents), _ptr(uniforms), _ptr(resid_uniforms), _ptr(accepted_len),
        _ptr(out_tokens), _ptr(out_nodes), _ptr(resid_probs), _ptr(seq_status),
        ctypes.c_void_p(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "specverify_run")


def specverify_run_static(cfg: sv_config, batch, target, draft, draft_tokens, parents, uniforms,
                          resid_uniforms, accepted_len, out_tokens, out_nodes=None,
                          resid_probs=None, seq_status=None, stream=None) -> None:
    """The allocation-free variant: no context, workspace in the library's
    fixed device array (at most SV_STATIC_SCRATCH_BYTES); cfg is an
    sv_config (see make_config)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    st = load().specverify_run_static(
        ctypes.byref(cfg), int(batch), _ptr(target), _ptr(draft), _ptr(draft_tokens),
        _ptr(parents), _ptr(uniforms), _ptr(resid_uniforms), _ptr(accepted_len),
        _ptr(out_tokens), _ptr(out_nodes), _ptr(resid_probs), _ptr(seq_status),
        ctypes.c_void_p(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "specverify_run_static")


def specverify_profile_events(ctx: int, ev_begin, ev_stream_end, ev_call_end=None) -> None:
    """Raw hipEvent_t handles (ints) or None; all None to stop."""
    st = load().specverify_profile_events(ctypes.c_void_p(ctx), ev_begin, ev_stream_end, ev_call_end)
    if st != SV_OK:
        raise SpecVerifyError(st, "specverify_profile_events")


def read_floor(t, sink, stream=None) -> None:
    """Read every byte of the device tensor t once (specverify_read_floor):
    the HBM read floor of its bytes, for timing beside a call.  sink: a
    device tensor of at least one int32."""
    import torch
    st = stream if stream is not None else torch.cuda.current_stream()
    rc = load().specverify_read_floor(ctypes.c_void_p(t.data_ptr()), t.numel() * t.element_size(),
                                      ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st.cuda_stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "specverify_read_floor")


def specverify_destroy(ctx) -> None:
    if ctx:
        load().specverify_destroy(ctypes.c_void_p(ctx))


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def specverify_accept_stats(accepted_len, seq_status, batch, k, draft_cost, out, stream=None) -> None:
    """out: SV_STATS_LEN float64 on the device (written)."""
    st = load().specverify_accept_stats(_ptr(accepted_len), _ptr(seq_status), int(batch), int(k),
                                        float(draft_cost), _ptr(out),
                                        ctypes.c_void_p(_stream_handle(stream)))
    if st != SV_OK:
        raise SpecVerifyError(st, "specverify_accept_stats")


def specverify_tree_mask(parents, batch, nodes, mask, depth=None, stream=None) -> None:
    """mask: [B, N, ceil(N/32)] uint32-sized (int32 tensor) written; depth: [B, N] int32 or None."""
    st = load().specverify_tree_mask(_ptr(parents), int(batch), int(nodes), _ptr(mask), _ptr(depth),
                                     ctypes.c_void_p(_stream_handle(stream)))
    if st != SV_OK:
        raise SpecVerifyError(st, "specverify_tree_mask")


def specverify_tree_commit(path_nodes, accepted_len, batch, nodes, commit_pos, stream=None) -> None:
    st = load().specverify_tree_commit(_ptr(path_nodes), _ptr(accepted_len), int(batch), int(nodes),
                                       _ptr(commit_pos), ctypes.c_void_p(_stream_handle(stream)))
    if st != SV_OK:
        raise SpecVerifyError(st, "specverify_tree_commit")


def accept_stats(accepted_len, k, draft_cost=0.0, seq_status=None, stream=None):
    """Allocates the output and queues specverify_accept_stats; returns the
    float64 tensor of SV_STATS_LEN values."""
    import torch
    out = torch.empty(SV_STATS_LEN, dtype=torch.float64, device=accepted_len.device)
    specverify_accept_stats(accepted_len, seq_status, accepted_len.numel(), k, draft_cost, out, stream)
    return out


def tree_mask(parents, want_depth=True, stream=None):
    """parents [B, N] int32 -> (mask [B, N, ceil(N/32)] int32 holding the uint32 words, depth [B, N])."""
    import torch
    B, N = parents.shape
    mask = torch.empty(B, N, (N + 31) // 32, dtype=torch.int32, device=parents.device)
    depth = torch.empty(B, N, dtype=torch.int32, device=parents.device) if want_depth else None
    specverify_tree_mask(parents, B, N, mask, depth, stream)
    return mask, depth


def tree_commit(path_nodes, accepted_len, stream=None):
    """out_nodes [B, N] and accepted_len [B] of a tree call -> commit_pos [B, N]."""
    import torch
    B, N = path_nodes.shape
    pos = torch.empty(B, N, dtype=torch.int32, device=path_nodes.device)
    specverify_tree_commit(path_nodes, accepted_len, B, N, pos, stream)
    return pos


# ------------------------------------------------------------------ convenience wrapper

class SpecVerify:
    """Owns one context; checks tensors and allocates the outputs of a call."""

    def __init__(self, mode=SV_MODE_SAMPLE, dtype="bf16", max_batch=1, k=1, vocab=2,
                 temperature=1.0, top_k=0, top_p=1.0, device=None, options=0):
        import torch
        self.cfg = make_config(mode, dtype, max_batch, k, vocab, temperature, top_k, top_p, options)
        self.device = torch.cuda.current_device() if device is None else int(device)
        self.ctx = specverify_create(self.cfg, self.device)

    def close(self):
        if getattr(self, "ctx", None):
            specverify_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, name, t, shape, dtypes):
        import torch
        if t is None:
            return
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if t.device.type != "cuda" or t.device.index != self.device:
            raise ValueError(f"{name} must live on cuda:{self.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype not in dtypes:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtypes}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")

    def run(self, target, draft=None, draft_tokens=None, uniforms=None, resid_uniforms=None,
            parents=None, want_resid_probs=False, stream=None):
        """Queue one call; returns a dict of output tensors (valid after the stream syncs)."""
        import torch
        c = self.cfg
        B = int(target.shape[0])
        V, k = c.vocab, c.k
        ldt = (torch.bfloat16, torch.int16, torch.uint16) if c.dtype == SV_DTYPE_BF16 else (torch.float32,)
        tree = c.mode in (SV_MODE_TREE_GREEDY, SV_MODE_TREE_SAMPLE)
        rows_t = k if tree else k + 1
        self._check("target", target, (B, rows_t, V), ldt)
        if c.mode in (SV_MODE_SAMPLE, SV_MODE_TREE_SAMPLE):
            self._check("draft", draft, (B, k, V), ldt)
            self._check("uniforms", uniforms, (B, k), (torch.float32,))
            self._check("resid_uniforms", resid_uniforms, (B,), (torch.float32,))
        self._check("draft_tokens", draft_tokens, (B, k), (torch.int32,))
        if tree:
            self._check("parents", parents, (B, k), (torch.int32,))
        dev = target.device
        out_w = k if tree else k + 1
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        toks = torch.empty(B, out_w, dtype=torch.int32, device=dev)
        nodes = torch.empty(B, out_w, dtype=torch.int32, device=dev) if tree else None
        status = torch.empty(B, dtype=torch.int32, device=dev)
        rp = torch.empty(B, V, dtype=torch.float32, device=dev) if want_resid_probs else None
        specverify_run(self.ctx, B, target, draft, draft_tokens, parents, uniforms,
                       resid_uniforms, acc, toks, nodes, rp, status, stream)
        return {"accepted_len": acc, "out_tokens": toks, "out_nodes": nodes,
                "seq_status": status, "resid_probs": rp}
