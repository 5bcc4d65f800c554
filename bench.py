#!/usr/bin/env python3
"""Benchmark of the verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C] [--no-cpu]

One step = one specverify_run over one batch of the workload (every logit
read once by the streaming kernel, then acceptance, residual / bonus draw and
outputs).  Inputs are seeded synthetic logits with the workloads' shapes,
already resident in HBM; calls rotate over identical copies at distinct
addresses totalling >= 1 GB so that every call reads cold HBM rather than the
256 MB Infinity Cache.  Prints one JSON line.

Metric: verified logit rows per second (target rows: B*(k+1) per chain call,
B*N per tree call) and, in "roofline", the streaming kernel's achieved HBM
bandwidth = algorithmic bytes per launch / its average duration, timed with
HIP events recorded around that kernel on its own stream.

The draft tokens of a workload are the draft model's own draws from its
adjusted distribution; here they are synthesised on the device with plain
torch ops before timing (workload synthesis, not part of the verified path).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "verified logit rows/sec + achieved HBM GB/s (fraction of peak), 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ workload synthesis

def draft_tokens_torch(draft, T, top_k, top_p, draw_u):
    """The draft model draws x_j ~ q'_j (its logits adjusted by T, top-k,
    top-p) by inverse CDF with its own uniforms.  fp32 torch on the device."""
    import torch
    z = draft.float() / T
    if top_k:
        thr = z.topk(top_k, dim=-1).values[..., -1:]
        z = torch.where(z >= thr, z, torch.full_like(z, -math.inf))
    p = torch.softmax(z, dim=-1)
    if top_p < 1.0:
        ps, order = p.sort(dim=-1, descending=True, stable=True)
        before = ps.cumsum(-1) - ps
        keep_sorted = before < top_p
        keep = torch.zeros_like(keep_sorted).scatter(-1, order, keep_sorted)
        p = torch.where(keep, p, torch.zeros_like(p))
    c = p.cumsum(-1)
    t = torch.as_tensor(draw_u, device=p.device, dtype=torch.float32).unsqueeze(-1) * c[..., -1:]
    x = torch.searchsorted(c.contiguous(), t.contiguous(), right=True).squeeze(-1)
    return x.clamp_(max=p.shape[-1] - 1).to(torch.int32).contiguous()


def logits_to_device(arr, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(arr).cuda()


# ------------------------------------------------------------------ HIP events via ctypes

class HipEvents:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e.value)
        return evs

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


# ------------------------------------------------------------------ measured HBM traffic

# the kernels and the host code that picks their tiling (both decide the
# streaming kernel's memory traffic)
KERNEL_SOURCES = [os.path.join(ROOT, "draft_token_verification_softmax_amd", "csrc", f)
                  for f in ("sv_kernels.hip", "sv_internal.h", "sv_api.cpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_stream_traffic.md")


def source_code(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed: what the
    compiler sees, so a comment edit does not count as a kernel change."""
    import re
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                               # string / char literal
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def kernel_digest():
    """sha256 of the kernel sources' code (comments and whitespace removed);
    the traffic counters are only valid for it."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            h.update(source_code(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(config):
    """HBM bytes per launch of the streaming kernel for a workload, from the
    committed FETCH_SIZE / WRITE_SIZE summary, if it was taken on the current
    kernel sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    digest = kernel_digest()
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if not line.startswith("traffic:"):
                continue
            kv = dict(tok.split("=", 1) for tok in line.split()[1:])
            if kv.get("workload") == str(config) and kv.get("sources") == digest:
                return int(kv["bytes_per_launch"])
    return None


# ------------------------------------------------------------------ CPU baseline (oracle)

def cpu_baseline(config, budget_s=12.0):
    """The float64 oracle, untuned, on a bounded sample of the same workload,
    single process (NumPy elementwise work runs on one core)."""
    import oracle.verify as ov
    from draft_token_verification_softmax_amd import workloads as wl
    cfg = wl.CONFIGS[config]
    t0 = time.perf_counter()
    rows = 0
    seqs = 0
    if cfg["kind"] == "tree_sample":
        import oracle.tree_sample as ts
        ti = wl.tree_sample_inputs(wl.DEFAULT_SEED[config], B=cfg["B"], N=cfg["N"], V=cfg["V"],
                                   dtype=cfg["dtype"], T=cfg["T"], sd=cfg["sd"], noise=cfg["noise"],
                                   max_depth=cfg["max_depth"], max_children=cfg["max_children"])
        T64 = wl.rows_f64(ti["target"], ti["dtype"])
        D64 = wl.rows_f64(ti["draft"], ti["dtype"])
        B, N = ti["B"], ti["N"]
        tokens = np.zeros((B, N), np.int32)
        for b in range(B):
            for i in range(1, N):
                q = ov.transform_row(D64[b, ti["parents"][b, i]], ti["T"])
                tokens[b, i] = ov.draw_from(q, ti["draw_u"][b, i])
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            b = seqs % B
            ts.tree_sample(T64[b], D64[b], ti["parents"][b], tokens[b], ti["u"][b], ti["ur"][b], ti["T"])
            rows += N
            seqs += 1
        el = time.perf_counter() - t0
        nbytes = rows * 2 * ti["V"] * (2 if ti["dtype"] == "bf16" else 4)
    elif cfg["kind"] == "tree":
        tr = wl.tree_inputs(config)
        T64 = wl.rows_f64(tr["target"], tr["dtype"])
        tokens = wl.tree_tokens(tr, np.argmax(T64, axis=-1))
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            b = seqs % tr["B"]
            ov.tree_greedy(T64[b], tr["parents"][b], tokens[b])
            rows += tr["N"]
            seqs += 1
        el = time.perf_counter() - t0
        nbytes = rows * tr["V"] * (2 if tr["dtype"] == "bf16" else 4)
    else:
        B = min(cfg["B"], 16)
        inp = wl.chain_inputs(config, B=B)
        T64 = wl.rows_f64(inp["target"], inp["dtype"])
        D64 = wl.rows_f64(inp["draft"], inp["dtype"])
        k = inp["k"]
        x = np.array([[ov.draw_from(ov.transform_row(D64[b, j], inp["T"], inp["top_k"], inp["top_p"]),
                                    inp["draw_u"][b, j]) for j in range(k)] for b in range(B)], np.int32)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            b = seqs % B
            ov.sample_chain(T64[b], D64[b], x[b], inp["u"][b], inp["ur"][b],
                            inp["T"], inp["top_k"], inp["top_p"])
            rows += k + 1
            seqs += 1
        el = time.perf_counter() - t0
        nbytes = seqs * (2 * k + 1) * inp["V"] * (2 if inp["dtype"] == "bf16" else 4)
    return {"value": rows / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{seqs} sequences of workload {config} ({rows} target rows, "
                      f"{nbytes / el / 1e9:.4f} GB/s of logits) in {el:.1f} s, one process",
            "host_cpus": os.cpu_count()}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device three times (scale reference for "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--digest", action="store_true", help="print the kernel-source digest and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the verification step shards by batch with no exchange, see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    import draft_token_verification_softmax_amd as svm
    from draft_token_verification_softmax_amd import workloads as wl

    if args.digest:
        print(kernel_digest())
        return
    if args.copy_calibrate:
        n = args.copy_calibrate * (1 << 20) // 4
        src = torch.ones(n, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_call": n * 4, "calls": 3}), flush=True)
        return

    svm.load()
    cfg = wl.CONFIGS[args.config]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    log(f"workload {args.config}: generating inputs")
    if cfg["kind"] == "tree_sample":
        ti = wl.tree_sample_inputs(wl.DEFAULT_SEED[args.config], B=cfg["B"], N=cfg["N"], V=cfg["V"], dtype=cfg["dtype"],
                                   T=cfg["T"], sd=cfg["sd"], noise=cfg["noise"],
                                   max_depth=cfg["max_depth"], max_children=cfg["max_children"])
        B, N, V, dtype, T = ti["B"], ti["N"], ti["V"], ti["dtype"], ti["T"]
        tgt = logits_to_device(ti["target"], dtype)
        dft = logits_to_device(ti["draft"], dtype)
        parents = torch.from_numpy(ti["parents"]).to(dev)
        par = parents.clamp(min=0).long()
        rows = dft[torch.arange(B, device=dev).unsqueeze(1), par]       # draft row of each node's parent
        tokens = draft_tokens_torch(rows, T, 0, 1.0, ti["draw_u"])
        tokens[:, 0] = 0
        inputs = dict(target=tgt, draft=dft, tokens=tokens, parents=parents,
                      u=torch.from_numpy(ti["u"]).to(dev), ur=torch.from_numpy(ti["ur"]).to(dev))
        mode, k, rows_t, rows_d = svm.SV_MODE_TREE_SAMPLE, N, N, N
        top_k, top_p = 0, 1.0
        workload = f"tree sampling verification, B={B}, N={N} nodes, V={V}, {dtype} logits, T={T}"
        extra = dict(B=B, N=N, V=V, logits_dtype=dtype, T=T, depth_max=cfg["max_depth"],
                     children_max=cfg["max_children"])
    elif cfg["kind"] == "tree":
        tr = wl.tree_inputs(args.config)
        B, N, V, dtype = tr["B"], tr["N"], tr["V"], tr["dtype"]
        tgt = logits_to_device(tr["target"], dtype)
        g = tgt.float().argmax(dim=-1).cpu().numpy()
        tokens = torch.from_numpy(wl.tree_tokens(tr, g)).to(dev)
        parents = torch.from_numpy(tr["parents"]).to(dev)
        inputs = dict(target=tgt, tokens=tokens, parents=parents)
        mode, k, rows_t, rows_d = svm.SV_MODE_TREE_GREEDY, N, N, 0
        T, top_k, top_p = 1.0, 0, 1.0
        workload = f"tree greedy verification, B={B}, N={N} nodes, V={V}, {dtype} logits"
        extra = dict(B=B, N=N, V=V, logits_dtype=dtype, depth_max=cfg["max_depth"], children_max=cfg["max_children"])
    else:
        inp = wl.chain_inputs(args.config)
        B, k, V, dtype = inp["B"], inp["k"], inp["V"], inp["dtype"]
        T, top_k, top_p = inp["T"], inp["top_k"], inp["top_p"]
        tgt = logits_to_device(inp["target"], dtype)
        dft = logits_to_device(inp["draft"], dtype)
        x = draft_tokens_torch(dft, T, top_k, top_p, inp["draw_u"])
        inputs = dict(target=tgt, draft=dft, tokens=x,
                      u=torch.from_numpy(inp["u"]).to(dev), ur=torch.from_numpy(inp["ur"]).to(dev))
        mode, rows_t, rows_d = svm.SV_MODE_SAMPLE, k + 1, k
        filt = f"top-k {top_k}" if top_k else (f"top-p {top_p}" if top_p < 1 else "no filter")
        workload = f"chain sampling verification, B={B}, k={k}, V={V}, {dtype} logits, T={T}, {filt}"
        extra = dict(B=B, k=k, V=V, logits_dtype=dtype, T=T, top_k=top_k, top_p=top_p)

    es = 2 if dtype == "bf16" else 4
    logit_bytes = B * (rows_t + rows_d) * V * es
    small_bytes = sum(t.numel() * t.element_size() for n, t in inputs.items() if n not in ("target", "draft"))
    tree = cfg["kind"] in ("tree", "tree_sample")
    out_bytes = B * 4 * (2 + (k + 1 if not tree else 2 * N))
    alg_bytes = logit_bytes + small_bytes + out_bytes
    ncopies = max(1, math.ceil(1e9 / logit_bytes))
    ncopies = min(ncopies, max(1, int(48e9 // logit_bytes)))
    log(f"{ncopies} input copies x {logit_bytes / 1e6:.3f} MB of logits")
    copies = [inputs] + [{n: t.clone() for n, t in inputs.items()} for _ in range(ncopies - 1)]

    sv = svm.SpecVerify(mode=mode, dtype=dtype, max_batch=B, k=k, vocab=V,
                        temperature=T, top_k=top_k, top_p=top_p)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    out_w = N if tree else k + 1
    out_tok = torch.empty(B, out_w, dtype=torch.int32, device=dev)
    out_nodes = torch.empty(B, out_w, dtype=torch.int32, device=dev) if tree else None
    status = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def step(i):
        c = copies[i % ncopies]
        svm.specverify_run(sv.ctx, B, c["target"], c.get("draft"), c["tokens"], c.get("parents"),
                           c.get("u"), c.get("ur"), acc, out_tok, out_nodes, None, status, stream)

    hip = HipEvents()
    hip.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region 1 (the metric): K plain calls, nothing else on the stream
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # timed region 2 (the roofline): the same K calls with HIP events recorded
    # on the call's stream around the streaming kernel (by the library) and
    # around the whole call
    evs = hip.create(4 * args.steps)
    torch.cuda.synchronize()
    for i in range(args.steps):
        e = evs[4 * i: 4 * i + 4]
        svm.specverify_profile_events(sv.ctx, e[1], e[2])
        hip.hip.hipEventRecord(ctypes.c_void_p(e[0]), ctypes.c_void_p(stream))
        step(i)
        hip.hip.hipEventRecord(ctypes.c_void_p(e[3]), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    svm.specverify_profile_events(sv.ctx, None, None)
    kms = np.array([hip.elapsed_ms(evs[4 * i + 1], evs[4 * i + 2]) for i in range(args.steps)])
    cms = np.array([hip.elapsed_ms(evs[4 * i], evs[4 * i + 3]) for i in range(args.steps)])
    hip.destroy(evs)
    kern_ms = float(np.mean(kms))
    call_ms = float(np.mean(cms))
    ms_per_step = wall * 1e3 / args.steps
    rows_per_call = B * rows_t
    value = rows_per_call * args.steps / wall
    achieved = logit_bytes / (kern_ms * 1e-3) / 1e9
    log(f"step {ms_per_step * 1e3:.2f} us (wall), call {call_ms * 1e3:.2f} us (events), streaming kernel "
        f"{kern_ms * 1e3:.2f} us (p10 {np.percentile(kms, 10) * 1e3:.2f}, p90 {np.percentile(kms, 90) * 1e3:.2f}), "
        f"{achieved:.1f} GB/s")
    result = {
        "metric": METRIC, "value": value, "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": dict(workload=workload, rows_per_call=rows_per_call,
                       logit_bytes_per_call=logit_bytes, input_copies=ncopies, **extra),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(args.config),
                     "kernel": "k_stream (the pass that reads every logit)", "kernel_us": kern_ms * 1e3,
                     "call_us_events": call_ms * 1e3,
                     "call_bytes_algorithmic": alg_bytes,
                     "call_GBps": alg_bytes / (call_ms * 1e-3) / 1e9},
    }
    # the kernels around the step, on this workload's outputs: acceptance
    # statistics (every mode); tree attention mask and commit map (tree)
    extras = {}

    def time_launches(fn, reps=100):
        e = hip.create(2)
        fn()
        torch.cuda.synchronize()
        hip.hip.hipEventRecord(ctypes.c_void_p(e[0]), ctypes.c_void_p(stream))
        for _ in range(reps):
            fn()
        hip.hip.hipEventRecord(ctypes.c_void_p(e[1]), ctypes.c_void_p(stream))
        torch.cuda.synchronize()
        us = hip.elapsed_ms(e[0], e[1]) * 1e3 / reps
        hip.destroy(e)
        return us

    kk = k if not tree else cfg["max_depth"]
    stats_out = torch.empty(svm.SV_STATS_LEN, dtype=torch.float64, device=dev)
    extras["accept_stats_us"] = time_launches(
        lambda: svm.specverify_accept_stats(acc, status, B, kk, 0.1, stats_out, stream))
    st = stats_out.cpu().numpy()
    extras["acceptance"] = float(st[svm.SV_STATS_ACCEPTANCE])
    extras["mal"] = float(st[svm.SV_STATS_MAL])
    extras["alpha"] = float(st[svm.SV_STATS_ALPHA])
    if tree:
        mask = torch.empty(B, N, (N + 31) // 32, dtype=torch.int32, device=dev)
        depth = torch.empty(B, N, dtype=torch.int32, device=dev)
        pos = torch.empty(B, N, dtype=torch.int32, device=dev)
        extras["tree_mask_us"] = time_launches(
            lambda: svm.specverify_tree_mask(inputs["parents"], B, N, mask, depth, stream))
        extras["tree_commit_us"] = time_launches(
            lambda: svm.specverify_tree_commit(out_nodes, acc, B, N, pos, stream))
    extras["note"] = ("mean per launch by HIP events over 100 back-to-back launches on the call's "
                      "stream; acceptance statistics of the last timed call (draft cost c = 0.1)")
    result["extras"] = extras
    sv.close()
    if not args.no_cpu:
        log("CPU baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(args.config)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
