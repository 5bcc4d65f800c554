#!/usr/bin/env python3
"""Benchmark of the verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C] [--also 2,3,4] [--no-cpu]

One step = one specverify_run over one batch of the workload: every logit
read once by the streaming kernel, then the acceptance step, the residual or
bonus draw and the outputs.  Inputs are seeded synthetic logits with the
workloads' shapes, already resident in HBM; calls rotate over identical
copies at distinct addresses totalling >= 1 GB, so every call reads cold HBM
rather than the 256 MB Infinity Cache.  Prints one JSON line.

The default workload is the largest one: 256 sequences, k = 4, V = 152064
float32 logits, temperature 0.8, nucleus 0.9 (1.40 GB of logits per call).

Metric: verified logit rows per second (target rows: B*(k+1) per chain
call, B*N per tree call).  "roofline": algorithmic bytes of one call (every
logit the mode reads, once, plus tokens, uniforms and outputs) / the call's
time from its first kernel's start to its last kernel's end, both recorded
by HIP events in the dispatch packets of those kernels on the call's stream;
the streaming kernel alone is reported beside it.  "traffic" is the HBM
bytes of every kernel of one call from the committed FETCH_SIZE / WRITE_SIZE
counters (profiles/traffic.md), while those were taken on the current kernel
sources.

The draft tokens of a workload are the draft model's own draws from its
adjusted distribution; here they are synthesised on the device with plain
torch ops before timing (workload synthesis, not part of the verified path).

Helpers for the committed profiles (no GPU needed):
    python bench.py --trace-summary <rocprofv3 kernel_trace.csv>
    python bench.py --pmc-summary <FETCH_SIZE counter_collection.csv> <WRITE_SIZE counter_collection.csv>
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
# kernels launched around a call by the bench itself (not part of the step)
AUX_KERNELS = ("k_accept_stats", "k_tree_mask", "k_tree_commit", "k_read_floor")


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
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e.value)
        return evs

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


# ------------------------------------------------------------------ measured HBM traffic

# the kernels and the host code that picks their tiling and launches (all of
# them decide a call's memory traffic)
KERNEL_SOURCES = [os.path.join(ROOT, "draft_token_verification_softmax_amd", "csrc", f)
                  for f in ("sv_kernels.hip", "sv_internal.h", "sv_api.cpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.md")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "workload5_nuc_counters.md")


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
    """HBM bytes of one call (every kernel of it) for a workload, from the
    committed FETCH_SIZE / WRITE_SIZE summary, if it was taken on the current
    kernel sources; else None.  Returns (call_bytes, stream_bytes)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, None
    digest = kernel_digest()
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if not line.startswith("traffic:"):
                continue
            kv = dict(tok.split("=", 1) for tok in line.split()[1:])
            if kv.get("workload") == str(config) and kv.get("sources") == digest:
                return int(kv["call_bytes"]), int(kv["stream_bytes"])
    return None, None


def measured_valu_busy():
    """The nucleus kernel's share of cycles in which its SIMDs issue vector
    instructions, and its vector instructions per logit, from the committed
    hardware-counter summary of workload 5 if it was taken on the current
    kernel sources; else None."""
    import re
    if not os.path.exists(COUNTERS_FILE):
        return None
    text = open(COUNTERS_FILE).read()
    dm = re.search(r"digest `([0-9a-f]+)`", text)
    bm = re.search(r"issued vector work in\s+(\d+)% of the launch's cycles", text)
    im = re.search(r"([0-9.]+) per logit", text)
    if not (dm and bm and im) or dm.group(1) != kernel_digest():
        return None
    return {"valu_busy_frac": int(bm.group(1)) / 100.0, "valu_instructions_per_logit": float(im.group(1)),
            "source": "rocprofv3 --pmc SQ_INSTS_VALU, GRBM_GUI_ACTIVE (profiles/workload5_nuc_counters.md)"}


# ------------------------------------------------------------------ rocprofv3 summaries

def _read_csv(path):
    import csv
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _short(name):
    """Kernel name without the return type and the parameter list."""
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def _reads_rows(name):
    """The kernel that reads every logit of a call: the streaming pass, or the
    one-read nucleus kernel of chain sampling with top-p."""
    return "k_stream" in name or "k_nuc_rows" in name


def _calls(rows, key_start, key_end):
    """Group library dispatches (in dispatch order) into calls: a call starts
    at a streaming-kernel dispatch (other than the second one of a lazy call,
    which follows its gate kernel) and holds the library kernels up to the
    next call; the bench's own kernels around the step are left out."""
    rows = [r for r in rows if r["Kernel_Name"].startswith(("k_", "void sv::k_", "sv::k_"))
            and not any(a in r["Kernel_Name"] for a in AUX_KERNELS)]
    rows.sort(key=lambda r: int(r.get("Dispatch_Id", r.get("Correlation_Id", 0))))
    calls, cur = [], None
    for r in rows:
        # a lazy call streams twice: the second streaming launch follows its gate
        if _reads_rows(r["Kernel_Name"]) and not (cur and "k_lazy_gate" in cur[-1]["Kernel_Name"]):
            cur = []
            calls.append(cur)
        if cur is not None:
            cur.append(r)
    return calls


def trace_summary(path):
    """Per-kernel durations and per-call spans (first kernel start to last
    kernel end) from a rocprofv3 --kernel-trace CSV, as markdown."""
    rows = _read_csv(path)
    calls = _calls(rows, "Start_Timestamp", "End_Timestamp")
    per = {}
    for c in calls:
        for r in c:
            per.setdefault(_short(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    spans = np.array([(max(int(r["End_Timestamp"]) for r in c) - min(int(r["Start_Timestamp"]) for r in c)) / 1e3
                      for c in calls if c])
    busy = np.array([sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in c) / 1e3
                     for c in calls if c])
    out = ["| kernel | dispatches | avg us | median us | min us | max us |", "|---|---|---|---|---|---|"]
    for name, d in sorted(per.items(), key=lambda kv: -np.mean(kv[1])):
        d = np.array(d)
        out.append(f"| `{name}` | {len(d)} | {d.mean():.2f} | {np.median(d):.2f} | {d.min():.2f} | {d.max():.2f} |")
    out.append("")
    out.append(f"calls: {len(spans)}; call span (first kernel start to last kernel end): mean {spans.mean():.2f} us, "
               f"median {np.median(spans):.2f} us, p10 {np.percentile(spans, 10):.2f}, p90 {np.percentile(spans, 90):.2f}; "
               f"sum of the call's kernel durations: mean {busy.mean():.2f} us")
    print("\n".join(out))


def pmc_summary(fetch_csv, write_csv, fetch_scale=2.0, write_scale=1.0):
    """Per-kernel FETCH_SIZE / WRITE_SIZE (KiB per dispatch, medians) and the
    HBM bytes of one call (sum over its kernels), from two rocprofv3 --pmc
    runs; bytes = fetch_scale * FETCH_SIZE + write_scale * WRITE_SIZE (the
    factors a copy of known size gives)."""
    res = {}
    for path, cname in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        rows = [r for r in _read_csv(path) if r.get("Counter_Name", cname) == cname]
        calls = _calls(rows, "Start_Timestamp", "End_Timestamp")
        per = {}
        tot = []
        for c in calls:
            s = 0.0
            for r in c:
                v = float(r["Counter_Value"])
                per.setdefault(_short(r["Kernel_Name"]), []).append(v)
                s += v
            tot.append(s)
        res[cname] = ({k: float(np.median(v)) for k, v in per.items()}, float(np.median(tot)) if tot else 0.0,
                      len(calls))
    f_per, f_tot, nf = res["FETCH_SIZE"]
    w_per, w_tot, nw = res["WRITE_SIZE"]
    out = ["| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per dispatch |", "|---|---|---|---|"]
    stream_bytes = 0
    for name in sorted(set(f_per) | set(w_per), key=lambda n: -f_per.get(n, 0.0)):
        b = int(round(1024 * (fetch_scale * f_per.get(name, 0.0) + write_scale * w_per.get(name, 0.0))))
        if _reads_rows(name):
            stream_bytes = b
        out.append(f"| `{name}` | {f_per.get(name, 0.0):.0f} | {w_per.get(name, 0.0):.0f} | {b} |")
    call_bytes = int(round(1024 * (fetch_scale * f_tot + write_scale * w_tot)))
    out.append("")
    out.append(f"calls: {nf} (FETCH_SIZE run), {nw} (WRITE_SIZE run); one call, median over calls: "
               f"FETCH_SIZE {f_tot:.0f} KiB, WRITE_SIZE {w_tot:.0f} KiB, HBM bytes {call_bytes}")
    out.append(f"call_bytes={call_bytes} stream_bytes={stream_bytes}")
    print("\n".join(out))


def counter_summary(csv_path):
    """Mean per dispatch of every counter of one rocprofv3 --pmc run, per
    library kernel, with the kernel's mean duration in that run."""
    per, dur = {}, {}
    for r in _read_csv(csv_path):
        name = _short(r["Kernel_Name"])
        if not name.startswith("sv::"):
            continue
        per.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        key = (name, r["Dispatch_Id"])
        dur[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
    counters = sorted({c for d in per.values() for c in d})
    out = ["| kernel | dispatches | mean us | " + " | ".join(counters) + " |",
           "|---|---|---|" + "---|" * len(counters)]
    for name in sorted(per, key=lambda n: -max(per[n].get(counters[0], [0.0]))):
        d = [v for (n, _), v in dur.items() if n == name]
        cells = [f"{float(np.mean(per[name][c])):.4g}" if c in per[name] else "" for c in counters]
        out.append(f"| `{name}` | {len(d)} | {float(np.mean(d)):.1f} | " + " | ".join(cells) + " |")
    print("\n".join(out))


def copy_summary(fetch_csv, write_csv, nbytes):
    """Scale factors of FETCH_SIZE and WRITE_SIZE from the copy kernel of
    ``bench.py --copy-calibrate``: bytes moved / counter bytes."""
    out = []
    for path, cname, moved in ((fetch_csv, "FETCH_SIZE", nbytes), (write_csv, "WRITE_SIZE", nbytes)):
        rows = [r for r in _read_csv(path) if r.get("Counter_Name", cname) == cname
                and not r["Kernel_Name"].startswith(("k_", "void sv::"))]
        big = [float(r["Counter_Value"]) for r in rows if float(r["Counter_Value"]) * 1024 > moved / 8]
        v = float(np.median(big))
        out.append(f"{cname}: {v:.0f} KiB per copy of {moved} bytes: factor {moved / (v * 1024):.3f}")
    print("\n".join(out))


# ------------------------------------------------------------------ CPU baseline (oracle)

def cpu_model():
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(config, budget_s=12.0):
    """The float64 oracle, untuned, on a bounded sample of the same workload,
    single process (NumPy elementwise work runs on one core)."""
    import oracle.verify as ov
    from draft_token_verification_softmax_amd import workloads as wl
    cfg = wl.CONFIGS[config]
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
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


# ------------------------------------------------------------------ one workload on the GPU

def measure(config, steps, warmup, hip, with_extras=True, lazy=False):
    """Time `steps` calls of workload `config` (after `warmup`): wall time
    of plain back-to-back calls (the metric), then the same calls with the
    library's call and streaming-kernel events.  Returns a dict."""
    import torch
    import draft_token_verification_softmax_amd as svm
    from draft_token_verification_softmax_amd import workloads as wl

    cfg = wl.CONFIGS[config]
    dev = torch.device("cuda:0")
    log(f"workload {config}: generating inputs")
    if cfg["kind"] == "tree_sample":
        ti = wl.tree_sample_inputs(wl.DEFAULT_SEED[config], B=cfg["B"], N=cfg["N"], V=cfg["V"], dtype=cfg["dtype"],
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
        arith = "f64"
    elif cfg["kind"] == "tree":
        tr = wl.tree_inputs(config)
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
        arith = "f32"
    else:
        inp = wl.chain_inputs(config)
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
        if lazy:
            workload += ", lazy row reads (rows after position 0 only where x_0 is accepted)"
        extra = dict(B=B, k=k, V=V, logits_dtype=dtype, T=T, top_k=top_k, top_p=top_p)
        arith = "f64"

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
                        temperature=T, top_k=top_k, top_p=top_p,
                        options=svm.SV_OPT_LAZY_ROWS if lazy else 0)
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

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region 1 (the metric): K plain calls, nothing else on the stream
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # timed region 2 (the roofline): the same K calls, the library recording
    # per call the streaming kernel's start and end and the last kernel's end
    evs = hip.create(3 * steps)
    torch.cuda.synchronize()
    for i in range(steps):
        e = evs[3 * i: 3 * i + 3]
        svm.specverify_profile_events(sv.ctx, e[0], e[1], e[2])
        step(i)
    torch.cuda.synchronize()
    svm.specverify_profile_events(sv.ctx, None, None, None)
    kms = np.array([hip.elapsed_ms(evs[3 * i], evs[3 * i + 1]) for i in range(steps)])
    cms = np.array([hip.elapsed_ms(evs[3 * i], evs[3 * i + 2]) for i in range(steps)])
    hip.destroy(evs)
    kern_us = float(np.mean(kms)) * 1e3
    call_us = float(np.mean(cms)) * 1e3
    step_us = wall * 1e6 / steps
    achieved = alg_bytes / (call_us * 1e-6) / 1e9
    stream_ach = logit_bytes / (kern_us * 1e-6) / 1e9
    call_traffic, stream_traffic = measured_traffic(config)
    log(f"workload {config}: step {step_us:.2f} us (wall), call {call_us:.2f} us (first kernel start to last "
        f"kernel end; p10 {np.percentile(cms, 10) * 1e3:.2f}, p90 {np.percentile(cms, 90) * 1e3:.2f}), "
        f"{achieved:.1f} GB/s = {achieved / PEAK_HBM_GBS:.3f} of peak; streaming kernel {kern_us:.2f} us, "
        f"{stream_ach:.1f} GB/s")
    # floors for the same call: a bare read of the same logits (the library's
    # read-floor kernel over each logit tensor of the same rotating copies:
    # every byte read once, in the streaming pass's tile shape), and one tiny
    # kernel per launch, back to back
    small = torch.zeros(1, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def reads(i):
        c = copies[i % ncopies]
        svm.read_floor(c["target"], sink)
        if c.get("draft") is not None:
            svm.read_floor(c["draft"], sink)

    # each floor's launches are captured in a HIP graph and timed by replay,
    # so the GPU runs them back to back whatever the host's launch rate (a
    # loop of small launches from Python would time the host)
    for i in range(warmup):
        reads(i)
        small.add_(1.0)
    torch.cuda.synchronize()
    g_read, g_tiny = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_read):
        for i in range(steps):
            reads(i)
    with torch.cuda.graph(g_tiny):
        for i in range(steps):
            small.add_(1.0)
    g_read.replay()
    g_tiny.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    fe = hip.create(3)
    hip.record(fe[0], stream)
    g_read.replay()
    hip.record(fe[1], stream)
    g_tiny.replay()
    hip.record(fe[2], stream)
    torch.cuda.synchronize()
    read_us = hip.elapsed_ms(fe[0], fe[1]) * 1e3 / steps
    tiny_us = hip.elapsed_ms(fe[1], fe[2]) * 1e3 / steps
    hip.destroy(fe)
    del g_read, g_tiny
    # the kernel that reads every logit: chain sampling with top-p alone takes
    # the one-read nucleus kernel, every other call the streaming pass
    one_read = cfg["kind"] == "chain" and top_p < 1.0 and not top_k
    res = dict(config=config, workload=workload, extra=extra, arith=arith, B=B, rows_per_call=B * rows_t,
               stream_name="k_nuc_rows" if one_read else "k_stream",
               logit_bytes=logit_bytes, alg_bytes=alg_bytes, ncopies=ncopies, wall=wall, step_us=step_us,
               call_us=call_us, call_us_p10=float(np.percentile(cms, 10)) * 1e3,
               call_us_p90=float(np.percentile(cms, 90)) * 1e3, kern_us=kern_us, achieved=achieved,
               stream_achieved=stream_ach, call_traffic=call_traffic, stream_traffic=stream_traffic,
               read_us=read_us, tiny_us=tiny_us)

    if with_extras:
        # the kernels around the step, on this workload's outputs: acceptance
        # statistics (every mode); tree attention mask and commit map (tree)
        extras = {}

        def time_launches(fn, reps=100):
            e = hip.create(2)
            fn()
            torch.cuda.synchronize()
            hip.record(e[0], stream)
            for _ in range(reps):
                fn()
            hip.record(e[1], stream)
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
        res["extras"] = extras
    sv.close()
    del copies, inputs
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--also", default="2,3,4",
                    help="other workloads whose call-level roofline goes into extras (comma list, '' for none)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--lazy", action="store_true",
                    help="plain sampling with lazy row reads (SV_OPT_LAZY_ROWS, the rejection fast path)")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device three times (scale reference for "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--digest", action="store_true", help="print the kernel-source digest and exit")
    ap.add_argument("--trace-summary", metavar="CSV", help="summarise a rocprofv3 kernel trace and exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 counter runs of the bench and exit")
    ap.add_argument("--counter-summary", metavar="CSV",
                    help="mean per dispatch of each counter of a rocprofv3 --pmc run, per kernel, and exit")
    ap.add_argument("--copy-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "BYTES"),
                    help="counter scale factors from two --copy-calibrate counter runs and exit")
    args = ap.parse_args()
    if args.digest:
        print(kernel_digest())
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.copy_summary:
        copy_summary(args.copy_summary[0], args.copy_summary[1], int(args.copy_summary[2]))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the verification "
              f"step shards by batch with no exchange, so N GPUs each run this one-GPU call on B/N "
              f"sequences", file=sys.stderr)
        sys.exit(2)

    import torch
    import draft_token_verification_softmax_amd as svm

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
    torch.cuda.set_device(0)
    hip = HipEvents()
    m = measure(args.config, args.steps, args.warmup, hip, lazy=args.lazy)
    value = m["rows_per_call"] * args.steps / m["wall"]
    result = {
        "metric": METRIC, "value": value, "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": m["step_us"] / 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": m["arith"], "data": "synthetic",
        "config": dict(workload=m["workload"], rows_per_call=m["rows_per_call"],
                       logit_bytes_per_call=m["logit_bytes"], input_copies=m["ncopies"], **m["extra"]),
        "roofline": {
            "bound": "hbm", "achieved": m["achieved"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": m["achieved"] / PEAK_HBM_GBS, "traffic": m["call_traffic"],
            "time": "one call, first kernel start to last kernel end (HIP events in the dispatch packets "
                    "of the call's first and last kernels), mean over the timed calls",
            "call_us": m["call_us"], "call_us_p10": m["call_us_p10"], "call_us_p90": m["call_us_p90"],
            "bytes_algorithmic": m["alg_bytes"],
            "stream_kernel": {"name": m["stream_name"] + " (the pass that reads every logit)", "us": m["kern_us"],
                              "achieved": m["stream_achieved"], "frac": m["stream_achieved"] / PEAK_HBM_GBS,
                              "traffic": m["stream_traffic"], "bytes_algorithmic": m["logit_bytes"],
                              "limiter": (dict(kind="vector ALU (float64 row-sum terms, candidate staging)",
                                               **measured_valu_busy())
                                          if args.config == 5 and "nuc_rows" in m["stream_name"]
                                          and measured_valu_busy() else None)},
            "floor": {"bare_read_us": m["read_us"], "bare_read_frac": m["logit_bytes"] / (m["read_us"] * 1e-6) / 1e9
                      / PEAK_HBM_GBS, "tiny_kernel_us": m["tiny_us"],
                      "note": "bare read: specverify_read_floor over each logit tensor of the same rotating "
                              "copies (16-byte non-temporal loads, 16 KB per workgroup), K calls captured in a "
                              "HIP graph, HIP events around its replay, mean per call; tiny kernel: a "
                              "one-element add per launch, K of them in a graph the same way"},
        },
    }
    extras = m.get("extras", {})
    others = []
    for c in [int(t) for t in args.also.split(",") if t.strip()]:
        if c == args.config:
            continue
        o = measure(c, min(args.steps, 100), args.warmup, hip, with_extras=False)
        others.append({"workload": o["workload"], "step_us": o["step_us"], "call_us": o["call_us"],
                       "bytes_algorithmic": o["alg_bytes"], "achieved_GBps": o["achieved"],
                       "frac": o["achieved"] / PEAK_HBM_GBS, "stream_us": o["kern_us"],
                       "stream_frac": o["stream_achieved"] / PEAK_HBM_GBS, "traffic": o["call_traffic"],
                       "bare_read_us": o["read_us"], "tiny_kernel_us": o["tiny_us"]})
    if others:
        extras["other_workloads"] = others
    result["extras"] = extras
    if not args.no_cpu:
        log("CPU baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(args.config)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
