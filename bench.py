"""Benchmark of the shared-prefix attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

One step = one pass of the whole path over one batch of synthetic input: build the
tile map from the per-token labels (label scan -> interval ends -> classification ->
CSR/CSC), the forward (O, LSE), then the backward (dQ together with the preparation
of D and LSE in log2 units, then dK/dV).  Inputs and
outputs stay resident in HBM; nothing is skipped inside the timed region.

The default workload is the 8-group rollout batch (P = 512, G = 8 completions of
R = 256 each, T = 20480, 32 q heads / 8 kv heads, head_dim 128, bf16, dO ~ N(0,1)).
Prints one JSON line: effective TFLOP/s over unmasked 128x128 tiles (fwd 4*d and
bwd 10*d FLOPs per pair per q head), its share of the bf16 MFMA peak, tokens/s, a
roofline entry for the dominant kernel (timed live with HIP events on the stream the
kernels run on) and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s (unmasked tiles) fwd+bwd, % bf16 MFMA peak; tokens/s"
PEAK_TFLOPS = {"bf16": 2516.6, "fp32": 157.3, "fp8": 5033.2}  # MI355X dense MFMA
# e4m3 forward: S = Q K^T on the fp8 MFMA, P V on the bf16 one (2d FLOPs each per
# kept pair): the peak of that mix is 4d over the time both halves take at their peaks
PEAK_FP8_FWD = 4.0 / (2.0 / PEAK_TFLOPS["fp8"] + 2.0 / PEAK_TFLOPS["bf16"])
HBM_PEAK_GBS = 8000.0
TILE = 128
KERNEL_SOURCES = ["attn_common.h", "attn_fwd.hip", "attn_bwd.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "shared_prefix_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kept_pairs(lay) -> int:
    """Exact number of kept (q, kv) pairs of a packed layout (per q head)."""
    if lay.kind == "draft":  # per kept block: its document's context before the anchor
        import numpy as np  # and its own block (all of it, or causally)
        x = lay.extra
        bs, doc, total = x["block_size"], x["ctx_doc"], 0
        pos = np.arange(len(doc))
        for a, dd, kp in zip(x["anchors"], x["anchor_doc"], x["keep"]):
            if kp:
                total += bs * int(((pos < a) & (doc == dd)).sum())
                total += bs * (bs + 1) // 2 if x["causal"] else bs * bs
        return total
    if lay.kind == "tokens":
        return sum(p * (p + 1) // 2 + sum(r * p + r * (r + 1) // 2 for r in rs)
                   for p, rs in lay.specs)
    anc = {}
    for path in lay.sample_paths:
        acc = 0
        for n in path:
            anc[n] = acc
            acc += lay.node_lengths[n]
    return sum(ln * (ln + 1) // 2 + ln * anc[n] for n, ln in enumerate(lay.node_lengths))


def describe(cfg, lay, layout_mode="packed", form="auto") -> str:
    if lay.kind == "draft":
        x = lay.extra
        n_docs = len(set(int(d) for d in x["ctx_doc"]))
        return (f"draft blocks over packed documents fwd+bwd: {n_docs} documents, context "
                f"{x['ctx_len']}, {len(x['anchors'])} blocks of {x['block_size']} "
                f"({'causal' if x['causal'] else 'bidirectional'}), T={lay.T}, "
                f"hq={cfg.hq}/hkv={cfg.hkv}, d={cfg.d}, {cfg.dtype}")
    if lay.kind == "tokens":
        ps = sorted({p for p, _ in lay.specs})
        layout = (f"{len(lay.specs)} groups, P={ps[0]}" if len(ps) == 1
                  else f"{len(lay.specs)} groups, P in [{ps[0]},{ps[-1]}]")
        rs = sorted({r for _, r_ in lay.specs for r in r_})
        g = {len(r_) for _, r_ in lay.specs}
        layout += f", G={'/'.join(map(str, sorted(g)))}, R=" + (
            str(rs[0]) if len(rs) == 1 else f"[{rs[0]},{rs[-1]}]")
    else:
        layout = "8 trees: root 1024 -> 4 x 256 -> 4 x 384 leaves"
    if layout_mode == "chunked":
        layout += " (completions interleaved in turns of 64 tokens)"
    elif layout_mode == "bfs":
        layout += " (nodes in breadth-first order)"
    if form == "nodes":
        layout += ", node-form map"
    return (f"shared-prefix attention fwd+bwd: {layout}, T={lay.T}, "
            f"hq={cfg.hq}/hkv={cfg.hkv}, d={cfg.d}, {cfg.dtype}")


def cpu_baseline(cfg, lay, min_seconds=10.0):
    """Time the float64 oracle on whole groups (trees) of the workload, all heads, one
    after another until at least min_seconds of CPU work (or the whole workload) is
    done; scale to the workload's effective FLOPs by the sample's share of the kept
    pairs.  Groups never see each other, so a group is a self-contained slice."""
    from threadpoolctl import threadpool_info

    from oracle import attention as oa
    from oracle.mask import meta_from_layout
    from shared_prefix_block_amd import workloads as wl

    if lay.kind == "tokens":
        parts = [wl.tokens_layout([spec]) for spec in lay.specs]
        unit = "group"
    else:
        per = 21  # root, 4 branches, 16 leaves
        parts = []
        for t in range(len(lay.node_lengths) // per):
            nodes = set(range(per * t, per * t + per))
            paths = [[n - per * t for n in pth] for pth in lay.sample_paths if pth[0] in nodes]
            parts.append(wl.tree_layout(lay.node_lengths[per * t:per * t + per], paths))
        unit = "tree"
    done, pairs, dt = 0, 0, 0.0
    for sub in parts:
        q, k, v, do = wl.make_tensors(sub.T, cfg.hq, cfg.hkv, cfg.d, cfg.dtype, cfg.sigma,
                                      cfg.idx)
        meta = meta_from_layout(sub)
        t0 = time.perf_counter()
        if cfg.passes == "fwd":
            oa.forward(meta, q, k, v)
        else:
            oa.backward(meta, q, k, v, do)
        dt += time.perf_counter() - t0
        done += 1
        pairs += kept_pairs(sub)
        if dt >= min_seconds:
            break
    frac = pairs / kept_pairs(lay)
    what = f"{done} of {len(parts)} {unit}s (first {done}), all {cfg.hq} q heads"
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    return {"sample": what, "frac": frac, "seconds": dt, "cores": int(threads)}


KERNEL_STAGE = {"fwd_kernel": "fwd", "dkdv_kernel": "bwd_dkdv", "dq_kernel": "bwd_dq"}
TRAFFIC_PASSES = ("FETCH_SIZE", "WRITE_SIZE")


def traffic_from_pmc(pmc_dir: str, calib_mb: int, dtype_tag: str = "bf16") -> dict:
    """Per attention stage: the kernel's FETCH_SIZE and WRITE_SIZE (KiB per dispatch,
    averaged over its dispatches) from the counter CSVs under pmc_dir, each with the
    factor that makes the reference negation over calib_mb MiB read and write exactly
    calib_mb MiB.  Only kernels instantiated for dtype_tag ("bf16" or "fp8") count."""
    import csv
    import glob

    def per_dispatch(counter):
        vals = {}
        for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] != counter:
                        continue
                    key = (r["Kernel_Name"], r["Dispatch_Id"])
                    vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        by_kernel = {}
        for (name, _), v in vals.items():
            by_kernel.setdefault(name, []).append(v)
        return {k: sum(v) / len(v) for k, v in by_kernel.items()}

    out = {}
    ref_kib = calib_mb * 1024.0
    for counter in TRAFFIC_PASSES:
        avg = per_dispatch(counter)
        calib = [v for k, v in avg.items() if "elementwise_kernel" in k and v > 0.25 * ref_kib]
        if not calib:
            raise SystemExit(f"no reference negation kernel found for {counter} in {pmc_dir}")
        factor = ref_kib / max(calib)
        for name, kib in avg.items():
            for sym, stage in KERNEL_STAGE.items():
                if sym in name and f"{dtype_tag}_t" in name:
                    short = name.replace("void ", "").replace("(anonymous namespace)::", "")
                    short = short.replace("psa::", "").rsplit("(", 1)[0]
                    e = out.setdefault(stage, {"kernel": short})
                    e[counter + "_KiB"] = kib
                    e[counter + "_scale"] = factor
    for e in out.values():
        if all(c + "_KiB" in e for c in TRAFFIC_PASSES):
            e["bytes_per_launch"] = int(sum(e[c + "_KiB"] * e[c + "_scale"] * 1024
                                            for c in TRAFFIC_PASSES))
    return out


def traffic_summary(pmc_dir: str, workload: str, calib_mb: int, command: str,
                    nograd: str = "") -> None:
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, each
    with --calib-mb) into profiles/traffic_<stage>[_nograd_<dtype>]_<workload>.json, one
    per attention kernel (traffic_from_pmc)."""
    out = traffic_from_pmc(pmc_dir, calib_mb, "fp8" if nograd == "fp8" else "bf16")
    variant = f"_nograd_{nograd}" if nograd else ""
    src_hash = kernel_source_hash()
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for stage, e in out.items():
        if "bytes_per_launch" not in e:
            continue
        e["kernel_source_hash"] = src_hash
        e["command"] = command
        path = os.path.join(ROOT, "profiles", f"traffic_{stage}{variant}_{workload}.json")
        with open(path, "w") as fh:
            json.dump(e, fh, indent=1)
        print(path, e["bytes_per_launch"])


def fold_bench(cfg, lay, steps: int, warmup: int) -> dict:
    """Fold of the workload's rollout groups (random token ids) and the unfold of a
    folded [T, hq, d] tensor back to the samples, timed with HIP events on the launch
    stream; both are pure data movement, measured against the HBM roofline on their
    algorithmic bytes (fold: the real tokens read once, six [T] outputs written; unfold:
    every unfolded row read once and written once)."""
    import numpy as np
    import torch

    from shared_prefix_block_amd import psa

    dev = torch.device("cuda:0")
    r = psa.Rollouts([p for p, _ in lay.specs], [rs for _, rs in lay.specs])
    gen = torch.Generator("cpu").manual_seed(cfg.idx)
    n_prompt = int(r.prompt_len.sum())
    pt = torch.randint(0, 150000, (n_prompt,), generator=gen, dtype=torch.int32).to(dev)
    ct = torch.randint(0, 150000, (r.fold_len - n_prompt,), generator=gen,
                       dtype=torch.int32).to(dev)
    src = torch.randn(lay.T, cfg.hq, cfg.d, generator=gen).to(torch.bfloat16).to(dev)
    ws = psa.fold_workspace(r, dev)
    dst = torch.empty((r.unfold_len, cfg.hq, cfg.d), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        ts = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    ms_fold = timed(lambda: psa.fold_rollouts(r, pt, ct, lay.T, workspace=ws))
    ms_unfold = timed(lambda: psa.unfold_rows(r, src, out=dst, workspace=ws))
    fold_bytes = 4 * r.fold_len + 21 * lay.T
    unfold_bytes = 2 * r.unfold_len * cfg.hq * cfg.d * 2
    gbs = unfold_bytes / (ms_unfold * 1e-3) / 1e9
    return {"metric": "fold / unfold throughput (HBM GB/s)", "value": round(gbs, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "higher_is_better": True, "dtype": "int32 / bf16 rows", "data": "synthetic",
            "config": {"workload": describe(cfg, lay), "T": lay.T, "T_real": lay.T_real,
                       "unfolded_rows": r.unfold_len, "row_bytes": cfg.hq * cfg.d * 2},
            "fold_ms": round(ms_fold, 4),
            "fold_gbs": round(fold_bytes / (ms_fold * 1e-3) / 1e9, 1),
            "unfold_ms": round(ms_unfold, 4),
            "roofline": {"kernel": "k_unfold", "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": None, "algorithmic_bytes_per_launch": unfold_bytes}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--grad-dtype", default="fp32", choices=["fp32", "bf16"])
    ap.add_argument("--split", action="store_true",
                    help="backward with P and dS as hi + lo bf16 pairs (PSA_BWD_SPLIT_PDS)")
    ap.add_argument("--calib-mb", type=int, default=0,
                    help="before warm-up, run one elementwise negation over this many MiB of "
                         "fp32 (reads and writes that many bytes): the reference kernel the "
                         "HBM byte counters are scaled by")
    ap.add_argument("--traffic-summary", metavar="PMC_DIR",
                    help="no timing: write the profiles/traffic_*.json files from the two "
                         "rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE) under PMC_DIR")
    ap.add_argument("--fold", action="store_true",
                    help="time the fold of the workload's rollout groups and the unfold of a "
                         "folded [T, hq, d] tensor instead of the attention step (token-form "
                         "workloads)")
    ap.add_argument("--form", default="auto", choices=["auto", "nodes"],
                    help="tile-map encoding: auto (the interval form for packed layouts) or "
                         "the node form forced (the general encoding, on the same tiles)")
    ap.add_argument("--layout", default="packed", choices=["packed", "chunked", "bfs"],
                    help="packed (as the workload states); chunked: each group's completions "
                         "interleaved in turns of 64 tokens after its prompt (token-form "
                         "workloads); bfs: tree nodes in breadth-first order (tree workloads). "
                         "Both keep the kept pairs; the map takes the node form")
    ap.add_argument("--nograd", default=None, choices=["bf16", "fp8"],
                    help="time the no-grad forward (no LSE stored) in this input dtype "
                         "instead of the workload's passes: map build + forward")
    ap.add_argument("--traffic-command", default="",
                    help="with --traffic-summary: the command line the passes ran, recorded")
    args = ap.parse_args()
    if args.traffic_summary:
        from shared_prefix_block_amd import workloads as wl
        traffic_summary(args.traffic_summary, wl.WORKLOADS[args.workload].name,
                        args.calib_mb or 512, args.traffic_command, args.nograd or "")
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures the single-GPU hot path only: the shared-prefix attention "
              "path has no cross-GPU step here (groups and heads shard with no communication); "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from shared_prefix_block_amd import psa
    from shared_prefix_block_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    psa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = wl.WORKLOADS[args.workload]
    lay = wl.layout_for(cfg)
    if args.layout == "chunked":
        if lay.kind != "tokens":
            sys.exit("--layout chunked needs a token-form workload")
        import numpy as np
        lay = wl.shuffled_tokens_layout(lay.specs, np.random.default_rng(cfg.idx),
                                        prompt_first=True, relabel=False, chunk=64,
                                        n_pad=lay.T - lay.T_real)
    elif args.layout == "bfs":
        if lay.kind != "tree":
            sys.exit("--layout bfs needs a tree workload")
        nl, paths = wl.reorder_tree(lay.node_lengths, lay.sample_paths)
        lay = wl.tree_layout(nl, paths, extra_pad=lay.T - lay.T_real)
    if args.layout != "packed" or lay.kind == "draft":
        args.no_cpu_baseline = True  # the oracle's sample slices packed groups
    if args.fold:
        if lay.kind != "tokens":
            sys.exit("--fold needs a token-form workload (rollout groups)")
        print(json.dumps(fold_bench(cfg, lay, args.steps, args.warmup)), flush=True)
        return
    if args.nograd:
        args.no_cpu_baseline = True
        q, k, v, do = wl.make_tensors(lay.T, cfg.hq, cfg.hkv, cfg.d, args.nograd, cfg.sigma,
                                      cfg.idx, with_grad_out=False)
        passes = f"fwd, no grad (no LSE), {args.nograd} inputs"
    else:
        q, k, v, do = wl.workload_tensors(cfg, lay)
        passes = cfg.passes
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    backward = cfg.passes != "fwd" and not args.nograd
    dtype_name = args.nograd or cfg.dtype
    do = do.to(dev) if backward else None
    if lay.kind == "tokens":
        labels = (torch.as_tensor(lay.group).to(dev), torch.as_tensor(lay.suffix).to(dev),
                  torch.as_tensor(lay.is_prefix).to(dev))
    tdt = q.dtype
    gdt = torch.float32 if args.grad_dtype == "fp32" else tdt
    o = torch.empty(q.shape, device=dev,
                    dtype=torch.bfloat16 if tdt == torch.float8_e4m3fn else tdt)
    lse = None if args.nograd else torch.empty(cfg.hq, lay.T, device=dev, dtype=torch.float32)
    grads = (torch.empty(q.shape, dtype=gdt, device=dev), torch.empty(k.shape, dtype=gdt, device=dev),
             torch.empty(v.shape, dtype=gdt, device=dev))
    stream = torch.cuda.current_stream(dev)

    def build_map():
        if lay.kind == "draft":
            return psa.layout_tile_map(lay, dev, block_m=TILE, block_n=TILE, dtype=tdt, d=cfg.d)
        if lay.kind == "tokens":
            return psa.build_tile_map_tokens(*labels, TILE, TILE, form=args.form)
        return psa.build_tile_map_tree(lay.node_lengths, lay.sample_paths, lay.T, dev, TILE, TILE,
                                       form=args.form)

    m0 = build_map()
    ws = torch.empty(max(psa.bwd_workspace_size(m0, q, k) if backward else 0, 1),
                     dtype=torch.uint8, device=dev)
    info = dict(m0.info)
    del m0

    # the backward as psa_bwd runs it: dQ with the preparation of its rows, then dK/dV
    names = ["map", "fwd"] + (["bwd_dq", "bwd_dkdv"] if backward else [])
    stage_of = {"bwd_dq": psa.STAGE_PREPARE | psa.STAGE_DQ, "bwd_dkdv": psa.STAGE_DKDV}

    def step(events=None):
        ev = (lambda i: events[i].record(stream)) if events else (lambda i: None)
        ev(0)
        m = build_map()
        ev(1)
        psa.fwd(m, q, k, v, out=o, lse=lse, with_lse=lse is not None)
        ev(2)
        if backward:
            for i, nm in enumerate(names[2:]):
                psa.bwd(m, q, k, v, o, lse, do, workspace=ws, grad_dtype=gdt,
                        stages=stage_of[nm], out=grads, split=args.split)
                ev(3 + i)
        return m

    if args.calib_mb:
        src = torch.ones(args.calib_mb * (1 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize(dev)
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)

    # timed region: K full steps, wall clock between two device synchronisations
    all_events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
                  for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    maps = []
    for s in range(args.steps):
        maps.append(step(all_events[s]))
        if len(maps) > 2:
            maps.pop(0)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    del maps

    per = {nm: [] for nm in names}
    for evs in all_events:
        for i, nm in enumerate(names):
            per[nm].append(evs[i].elapsed_time(evs[i + 1]))
    avg = {nm: sum(x) / len(x) for nm, x in per.items()}

    kept = kept_pairs(lay)
    tiles = info["n_full"] + info["n_partial"]
    d, hq = cfg.d, cfg.hq
    f_fwd, f_bwd = 4 * d, 10 * d
    tile_flops = tiles * TILE * TILE * hq * (f_fwd + (f_bwd if backward else 0))
    kept_flops = kept * hq * (f_fwd + (f_bwd if backward else 0))
    ms_step = wall * 1e3 / args.steps
    value = tile_flops / (ms_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype_name]
    dom_peak = PEAK_FP8_FWD if dtype_name == "fp8" else peak

    # dominant kernel: algorithmic FLOPs per launch (fwd 4d; dK/dV 8d = S, dP, dV, dK;
    # dQ 2d: its S and dP are recomputations) per kept pair per q head
    algo = {"fwd": 4 * d, "bwd_dkdv": 8 * d, "bwd_dq": 2 * d}
    cand = {k_: avg[k_] for k_ in algo if k_ in avg}
    dom = max(cand, key=cand.get)
    achieved = kept * hq * algo[dom] / (avg[dom] * 1e-3) / 1e12
    traffic = None
    variant = f"_nograd_{args.nograd}" if args.nograd else ""
    tpath = os.path.join(ROOT, "profiles", f"traffic_{dom}{variant}_{cfg.name}.json")
    if os.path.exists(tpath):
        with open(tpath) as fh:
            t = json.load(fh)
        if t.get("kernel_source_hash") == kernel_source_hash():
            traffic = t.get("bytes_per_launch")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name,
        "data": "synthetic (seeded N(0, sigma) Q/K/V/dO; layout as the workload states)",
        "config": {"workload": describe(cfg, lay, args.layout, args.form), "T": lay.T,
                   "T_real": lay.T_real, "map_form": ["interval", "nodes"][info["form"]],
                   "hq": cfg.hq, "hkv": cfg.hkv, "head_dim": d,
                   "passes": passes, "grad_dtype": args.grad_dtype if backward else None,
                   "bwd_p_ds": (("hi+lo bf16" if args.split else "bf16, hi+lo where large")
                                if backward else None),
                   "tiles_128": {"full": info["n_full"], "partial": info["n_partial"]},
                   "kept_pairs_per_head": kept},
        f"pct_{dtype_name}_peak": round(100 * value / peak, 2),
        "kept_pair_tflops": round(kept_flops / (ms_step * 1e-3) / 1e12, 2),
        "tokens_per_s": round(lay.T_real / (ms_step * 1e-3), 1),
        "stage_ms": {nm: round(avg[nm], 4) for nm in names},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": round(dom_peak, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / dom_peak, 4),
                     "traffic": traffic,
                     "algorithmic_flops_per_launch": kept * hq * algo[dom],
                     "avg_launch_ms": round(avg[dom], 4)},
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(cfg, lay)
        work_tile_flops = tile_flops * cb["frac"]
        out["cpu_baseline"] = {"value": round(work_tile_flops / cb["seconds"] / 1e12, 6),
                               "unit": "TFLOP/s", "cores": cb["cores"], "kind": "oracle",
                               "sample": f"{cb['sample']}: {cb['seconds']:.2f} s of float64 "
                                         f"dense-mask oracle "
                                         f"({'fwd' if not backward else 'fwd+bwd'}), "
                                         f"scaled by its share {cb['frac']:.4f} of the "
                                         f"workload's kept pairs"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
