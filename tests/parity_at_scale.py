"""Parity of the library against the oracle over many sequences (GPU).

    python tests/parity_at_scale.py --config 3 --sequences 10000 [--threads 16] [--out FILE]
    python tests/parity_at_scale.py --config 2 --sequences 10000 --noise 0.05   # draft close to its target
    python tests/parity_at_scale.py --config 1 --sequences 1000 --batch 1 --seed-base 20000   # one sequence per call

Not a pytest module (pytest collects test_*.py only): a full run takes
minutes of host time for the oracle.  Each batch has its own seed
(seed base, 9000 by default, + 100 * config + batch index), so these sequences are not the ones the
benchmark or the unit tests use.  Inputs come from the workload generators;
the drafted tokens are drawn on the device from the draft's adjusted rows
(fp32 torch, the caller's side), which is enough for parity: the library and
the oracle see the same tokens.  Rule (reading R14): accepted length, tokens
and status equal on every unflagged sequence; flagged mismatches strictly
below 0.01% of the sequences; resid_probs within 1e-5.  Prints one JSON line and, with
--out, appends a markdown row.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402  (loads the HIP runtime before the library)

import oracle.tree_sample as ts  # noqa: E402
import oracle.verify as ov  # noqa: E402
from draft_token_verification_softmax_amd import (SV_MODE_GREEDY, SV_MODE_SAMPLE,  # noqa: E402
                                                  SV_MODE_TREE_GREEDY, SV_MODE_TREE_SAMPLE, SpecVerify)
from draft_token_verification_softmax_amd import workloads as wl  # noqa: E402

RESID_TOL = 1e-5


def to_dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def draw_device(draft_dev, dtype, T, top_k, top_p, draw_u):
    """x ~ q' on the device (fp32): the draft model's own draw."""
    z = (draft_dev.view(torch.bfloat16).float() if dtype == "bf16" else draft_dev.float()) / T
    if top_k:
        thr = z.topk(top_k, dim=-1).values[..., -1:]
        z = torch.where(z >= thr, z, torch.full_like(z, -math.inf))
    p = torch.softmax(z, dim=-1)
    if top_p < 1.0:
        ps, order = p.sort(dim=-1, descending=True, stable=True)
        keep_sorted = (ps.cumsum(-1) - ps) < top_p
        keep = torch.zeros_like(keep_sorted).scatter(-1, order, keep_sorted)
        p = torch.where(keep, p, torch.zeros_like(p))
    c = p.cumsum(-1)
    t = torch.as_tensor(draw_u, device=p.device, dtype=torch.float32).unsqueeze(-1) * c[..., -1:]
    x = torch.searchsorted(c.contiguous(), t.contiguous(), right=True).squeeze(-1)
    return x.clamp_(max=p.shape[-1] - 1).to(torch.int32).contiguous()


def run_chain_batch(cfg_id, inp, mode, pool, sv):
    dtype, T, top_k, top_p = inp["dtype"], inp["T"], inp["top_k"], inp["top_p"]
    B, k = inp["u"].shape
    tgt = to_dev(inp["target"], dtype)
    if mode == SV_MODE_SAMPLE:
        dft = to_dev(inp["draft"], dtype)
        x_dev = draw_device(dft, dtype, T, top_k, top_p, inp["draw_u"])
        out = sv.run(tgt, dft, x_dev, to_dev(inp["u"], None), to_dev(inp["ur"], None), want_resid_probs=True)
    else:
        z = tgt.view(torch.bfloat16).float() if dtype == "bf16" else tgt.float()
        g = z.argmax(dim=-1)[:, :k].to(torch.int32)
        rnd = torch.from_numpy(np.random.default_rng(inp["seed_greedy"]).integers(0, z.shape[-1], size=(B, k))
                               .astype(np.int32)).cuda()
        keep = torch.from_numpy(np.random.default_rng(inp["seed_greedy"] + 1).random((B, k)) < 0.8).cuda()
        x_dev = torch.where(keep, g, rnd).contiguous()
        out = sv.run(tgt, draft_tokens=x_dev)
    torch.cuda.synchronize()
    x = x_dev.cpu().numpy()
    gpu = {key: (v.cpu().numpy() if v is not None else None) for key, v in out.items()}
    T64 = wl.rows_f64(inp["target"], dtype)
    D64 = wl.rows_f64(inp["draft"], dtype) if mode == SV_MODE_SAMPLE else None

    def one(b):
        if mode == SV_MODE_SAMPLE:
            o = ov.sample_chain(T64[b], D64[b], x[b], inp["u"][b], inp["ur"][b], T, top_k, top_p)
            return o["n"], o["tokens"], o["status"], o["flagged"], o["resid"]
        n, t, s = ov.greedy_chain(T64[b], x[b])
        return n, t, s, False, None

    res = list(pool.map(one, range(B)))
    return gpu, res


def run_tree_batch(tr, B, pool, sv):
    T64 = tr["T64"]
    tokens = wl.tree_tokens(tr, np.argmax(T64, axis=-1))
    out = sv.run(to_dev(tr["target"], tr["dtype"]), draft_tokens=torch.from_numpy(tokens).cuda(),
                 parents=torch.from_numpy(tr["parents"]).cuda())
    torch.cuda.synchronize()
    gpu = {key: (v.cpu().numpy() if v is not None else None) for key, v in out.items()}

    def one(b):
        n, t, nodes, s = ov.tree_greedy(T64[b], tr["parents"][b], tokens[b])
        return n, t, s, False, None, nodes

    return gpu, list(pool.map(one, range(B)))


def run_tree_sample_batch(ti, B, pool, sv):
    dtype, T = ti["dtype"], ti["T"]
    tgt = to_dev(ti["target"], dtype)
    dft = to_dev(ti["draft"], dtype)
    parents = torch.from_numpy(ti["parents"]).cuda()
    par = parents.clamp(min=0).long()
    rows = dft[torch.arange(B, device="cuda").unsqueeze(1), par]   # each node's parent's draft row
    tok_dev = draw_device(rows, dtype, T, 0, 1.0, ti["draw_u"])
    tok_dev[:, 0] = 0
    out = sv.run(tgt, dft, tok_dev.contiguous(), to_dev(ti["u"], None), to_dev(ti["ur"], None),
                 parents=parents, want_resid_probs=True)
    torch.cuda.synchronize()
    tokens = tok_dev.cpu().numpy()
    gpu = {key: (v.cpu().numpy() if v is not None else None) for key, v in out.items()}
    T64, D64 = ti["T64"], ti["D64"]

    def one(b):
        o = ts.tree_sample(T64[b], D64[b], ti["parents"][b], tokens[b], ti["u"][b], ti["ur"][b], T)
        return o["n"], o["tokens"], o["status"], o["flagged"], o["resid"], o["nodes"]

    return gpu, list(pool.map(one, range(B)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, required=True)
    ap.add_argument("--sequences", type=int, default=10000)
    ap.add_argument("--batch", type=int, default=0)
    ap.add_argument("--threads", type=int, default=16)
    ap.add_argument("--gen-threads", type=int, default=4)
    ap.add_argument("--mode", choices=["sample", "greedy"], default="sample")
    ap.add_argument("--out", default="")
    ap.add_argument("--noise", type=float, default=None, help="draft noise sd (chain and sampled-tree workloads)")
    ap.add_argument("--seed-base", type=int, default=9000)
    args = ap.parse_args()
    c = args.config
    cfg = wl.CONFIGS[c]
    tsample = cfg["kind"] == "tree_sample"
    tree = cfg["kind"] == "tree" or tsample
    mode = (SV_MODE_TREE_SAMPLE if tsample else SV_MODE_TREE_GREEDY) if tree else \
        (SV_MODE_SAMPLE if args.mode == "sample" else SV_MODE_GREEDY)
    B = args.batch or (cfg["B"] if cfg["B"] > 1 else 64)
    nb = (args.sequences + B - 1) // B
    if tsample:
        sv = SpecVerify(mode=mode, dtype=cfg["dtype"], max_batch=B, k=cfg["N"], vocab=cfg["V"],
                        temperature=cfg["T"])
    elif tree:
        sv = SpecVerify(mode=mode, dtype=cfg["dtype"], max_batch=B, k=cfg["N"], vocab=cfg["V"])
    else:
        sv = SpecVerify(mode=mode, dtype=cfg["dtype"], max_batch=B, k=cfg["k"], vocab=cfg["V"],
                        temperature=cfg["T"], top_k=cfg["top_k"], top_p=cfg["top_p"])
    stats = dict(sequences=0, flagged=0, mismatches=0, flagged_mismatches=0, resid_max_abs=0.0,
                 accepted=0)
    bad = []
    t0 = time.perf_counter()
    with ThreadPoolExecutor(args.threads) as pool, ThreadPoolExecutor(args.gen_threads) as gen:
        def make(i):
            seed = args.seed_base + 100 * c + i
            if tsample:
                noise = cfg["noise"] if args.noise is None else args.noise
                ti = wl.tree_sample_inputs(seed, B=B, N=cfg["N"], V=cfg["V"], dtype=cfg["dtype"], T=cfg["T"],
                                           sd=cfg["sd"], noise=noise, max_depth=cfg["max_depth"],
                                           max_children=cfg["max_children"])
                ti["T64"] = wl.rows_f64(ti["target"], ti["dtype"])
                ti["D64"] = wl.rows_f64(ti["draft"], ti["dtype"])
                return ti
            if tree:
                tr = wl.tree_inputs(4, seed=seed, B=B)
                tr["T64"] = wl.rows_f64(tr["target"], tr["dtype"])
                return tr
            inp = wl.chain_inputs(c, seed=seed, B=B, noise=args.noise)
            inp["seed_greedy"] = seed + 50000
            return inp
        ahead = [gen.submit(make, j) for j in range(min(args.gen_threads, nb))]
        for i in range(nb):
            cur = ahead.pop(0).result()
            if i + len(ahead) + 1 < nb:
                ahead.append(gen.submit(make, i + len(ahead) + 1))
            if tsample:
                gpu, res = run_tree_sample_batch(cur, B, pool, sv)
            elif tree:
                gpu, res = run_tree_batch(cur, B, pool, sv)
            else:
                gpu, res = run_chain_batch(c, cur, mode, pool, sv)
            for b, r in enumerate(res):
                n, toks, st, flagged = r[0], r[1], r[2], r[3]
                want = np.full(gpu["out_tokens"].shape[1], -1, np.int32)
                want[:len(toks)] = toks
                same = (gpu["accepted_len"][b] == n and np.array_equal(gpu["out_tokens"][b], want)
                        and gpu["seq_status"][b] == st)
                if tree:
                    wn = np.full(gpu["out_nodes"].shape[1], -1, np.int32)
                    wn[:len(r[5])] = r[5]
                    same = same and np.array_equal(gpu["out_nodes"][b], wn)
                stats["sequences"] += 1
                stats["flagged"] += int(flagged)
                stats["accepted"] += int(n)
                if not same:
                    stats["mismatches"] += 1
                    stats["flagged_mismatches"] += int(flagged)
                    if not flagged and len(bad) < 5:
                        bad.append(dict(batch=i, b=b, gpu_n=int(gpu["accepted_len"][b]), orc_n=int(n)))
                if r[4] is not None and gpu.get("resid_probs") is not None:
                    d = float(np.abs(gpu["resid_probs"][b].astype(np.float64) - r[4]).max())
                    stats["resid_max_abs"] = max(stats["resid_max_abs"], d)
            print(f"batch {i + 1}/{nb}: {stats['sequences']} sequences, {stats['mismatches']} mismatches, "
                  f"{stats['flagged']} flagged, {time.perf_counter() - t0:.0f} s", flush=True)
    sv.close()
    unflagged = stats["mismatches"] - stats["flagged_mismatches"]
    ok = unflagged == 0 and stats["flagged_mismatches"] < 1e-4 * stats["sequences"] and \
        stats["resid_max_abs"] <= RESID_TOL
    label = ("tree sampling" if tsample else "tree greedy" if tree else args.mode)
    if args.noise is not None:
        label += f", draft noise sd {args.noise:g}"
    if B == 1:
        label += ", one sequence per call"
    stats.update(config=c, mode=label,
                 batch=B, ok=bool(ok),
                 unflagged_mismatches=unflagged, examples=bad,
                 mean_accepted=stats["accepted"] / max(1, stats["sequences"]),
                 seconds=round(time.perf_counter() - t0, 1))
    print(json.dumps(stats), flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(f"| {c} | {stats['mode']} | {stats['sequences']} | {stats['mean_accepted']:.3f} | "
                    f"{stats['flagged']} | {stats['mismatches']} | {unflagged} | "
                    f"{stats['resid_max_abs']:.2e} | {'pass' if ok else 'FAIL'} |\n")
    sys.exit(0 if ok else 1)


if __name__ == "__main__":
    main()
