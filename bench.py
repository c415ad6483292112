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
KERNEL_SOURCES = ["attn_common.h", "attn_fwd.hip", "attn_bwd.h", "attn_bwd.hip", "attn_bwd_dkdv.hip"]


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


def _parts(lay):
    """The self-contained slices of a packed layout: its groups (token form) or trees."""
    from shared_prefix_block_amd import workloads as wl

    if lay.kind == "tokens":
        return [("group", spec) for spec in lay.specs]
    per = 21  # root, 4 branches, 16 leaves
    out = []
    for t in range(len(lay.node_lengths) // per):
        nodes = set(range(per * t, per * t + per))
        paths = [[n - per * t for n in pth] for pth in lay.sample_paths if pth[0] in nodes]
        out.append(("tree", (lay.node_lengths[per * t:per * t + per], paths)))
    return out


def _part_layout(kind, spec):
    from shared_prefix_block_amd import workloads as wl

    if kind == "group":
        return wl.tokens_layout([spec])
    return wl.tree_layout(*spec)


def oracle_dense_flops(lay, hq: int, d: int, backward: bool) -> float:
    """The float64 oracle's own work: per group (tree) and q head, dense products over
    the group's columns; S and P V forward (4 d per pair of the group), plus dP, dQ,
    dK and dV backward (8 d more)."""
    sizes = []
    for kind, spec in _parts(lay):
        sizes.append(spec[0] + sum(spec[1]) if kind == "group" else sum(spec[0]))
    per_pair = (12 if backward else 4) * d
    return float(sum(n * n for n in sizes)) * hq * per_pair


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, lay, budget_flop: float = 1.2e12) -> dict:
    """The float64 oracle, unchanged, timed on a bounded sample of the workload: its
    first group (tree), on as many q heads as keep the oracle's dense work of the
    sample under budget_flop (then its completions cut too, if one head is still over),
    forward alone and forward + backward.  The oracle's time follows its dense work
    (oracle_dense_flops), so each time is scaled to the whole workload by the ratio of
    that work; tokens/s = real tokens / scaled time."""
    from threadpoolctl import threadpool_info

    from oracle import attention as oa
    from oracle.mask import meta_from_layout
    from shared_prefix_block_amd import workloads as wl

    backward = cfg.passes != "fwd"
    kind, spec = _parts(lay)[0]
    rep = cfg.hq // cfg.hkv
    hkv_s = cfg.hkv
    sub = _part_layout(kind, spec)
    while hkv_s > 1 and oracle_dense_flops(sub, hkv_s * rep, cfg.d, backward) > budget_flop:
        hkv_s = (hkv_s + 1) // 2
    hq_s = hkv_s * rep
    cut = ""
    if kind == "group":
        p, rs = spec
        while len(rs) > 1 and oracle_dense_flops(sub, hq_s, cfg.d, backward) > budget_flop:
            rs = rs[: max(1, len(rs) * 3 // 4)]
            sub = _part_layout(kind, (p, rs))
        if len(rs) < len(spec[1]):
            cut = f" with {len(rs)} of its {len(spec[1])} completions"
    q, k, v, do = wl.make_tensors(sub.T, hq_s, hkv_s, cfg.d, cfg.dtype, cfg.sigma, cfg.idx)
    meta = meta_from_layout(sub)
    t0 = time.perf_counter()
    oa.forward(meta, q, k, v)
    t_fwd = time.perf_counter() - t0
    t_fb = None
    if backward:
        t0 = time.perf_counter()
        oa.backward(meta, q, k, v, do)
        t_fb = time.perf_counter() - t0
    scale_f = oracle_dense_flops(lay, cfg.hq, cfg.d, False) / oracle_dense_flops(
        sub, hq_s, cfg.d, False)
    scale_b = oracle_dense_flops(lay, cfg.hq, cfg.d, True) / oracle_dense_flops(
        sub, hq_s, cfg.d, True)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    est_fwd = t_fwd * scale_f
    est_fb = t_fb * scale_b if backward else None
    sample = (f"{'group' if kind == 'group' else 'tree'} 0 of {len(_parts(lay))}{cut}, "
              f"{hq_s} of {cfg.hq} q heads ({hkv_s} kv heads): fwd {t_fwd:.2f} s"
              + (f", fwd+bwd {t_fb:.2f} s" if backward else "")
              + " of the float64 dense-mask oracle, scaled by the oracle's dense work")
    sig = lambda x: None if x is None else float(f"{x:.4g}")  # noqa: E731
    return {"sample": sample, "sample_fwd_s": sig(t_fwd), "sample_fwd_bwd_s": sig(t_fb),
            "est_fwd_s": sig(est_fwd), "est_fwd_bwd_s": sig(est_fb),
            "tokens_per_s": sig(lay.T_real / (est_fb if backward else est_fwd)),
            "oracle_dense_gflop": sig(oracle_dense_flops(lay, cfg.hq, cfg.d, backward) / 1e9),
            "blas_threads": int(threads)}


KERNEL_STAGE = {"fwd_kernel": "fwd", "dkdv_kernel": "bwd_dkdv", "dq_kernel": "bwd_dq"}
TRAFFIC_PASSES = ("FETCH_SIZE", "WRITE_SIZE")
BUSY_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE", "GRBM_COUNT")
N_CU, N_XCD = 256, 8


def _per_dispatch(pmc_dir: str, counter: str) -> dict:
    """Kernel name -> the counter per dispatch (summed over its rows, averaged over the
    kernel's dispatches) from the rocprofv3 counter CSVs under pmc_dir."""
    import csv
    import glob

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


def _stage_kernels(avg: dict, dtype_tag: str):
    """(stage, short kernel name, value) of the attention kernels for one input dtype."""
    for name, val in avg.items():
        for sym, stage in KERNEL_STAGE.items():
            if sym in name and f"{dtype_tag}_t" in name:
                short = name.replace("void ", "").replace("(anonymous namespace)::", "")
                yield stage, short.replace("psa::", "").rsplit("(", 1)[0], val


def traffic_from_pmc(pmc_dir: str, calib_mb: int, dtype_tag: str = "bf16") -> dict:
    """Per attention stage: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged over
    each kernel's dispatches, summed over the kernels of the stage: at d = 256 a stage
    is several launches) from the counter CSVs under pmc_dir, each with the factor that
    makes the reference negation over calib_mb MiB read and write exactly calib_mb MiB.
    Only kernels instantiated for dtype_tag ("bf16" or "fp8") count."""
    out = {}
    ref_kib = calib_mb * 1024.0
    for counter in TRAFFIC_PASSES:
        avg = _per_dispatch(pmc_dir, counter)
        calib = [v for k, v in avg.items() if "elementwise_kernel" in k and v > 0.25 * ref_kib]
        if not calib:
            raise SystemExit(f"no reference negation kernel found for {counter} in {pmc_dir}")
        factor = ref_kib / max(calib)
        for stage, short, kib in _stage_kernels(avg, dtype_tag):
            e = out.setdefault(stage, {"kernels": []})
            if short not in e["kernels"]:
                e["kernels"].append(short)
            e[counter + "_KiB"] = e.get(counter + "_KiB", 0.0) + kib
            e[counter + "_scale"] = factor
    for e in out.values():
        e["kernel"] = " + ".join(e["kernels"])
        if all(c + "_KiB" in e for c in TRAFFIC_PASSES):
            e["bytes_per_launch"] = int(sum(e[c + "_KiB"] * e[c + "_scale"] * 1024
                                            for c in TRAFFIC_PASSES))
    return out


def busy_from_pmc(pmc_dir: str, dtype_tag: str = "bf16") -> dict:
    """Per attention stage, from one rocprofv3 --pmc pass of BUSY_COUNTERS: MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 256 CUs x 4 SIMDs), CU busy =
    SQ_BUSY_CU_CYCLES / (GRBM_GUI_ACTIVE / 8 x 256), and the clock GRBM_GUI_ACTIVE /
    GRBM_COUNT x 100 MHz is not taken here (its reference clock is not documented);
    cycles are summed over the kernels of a stage."""
    tot = {}
    for counter in BUSY_COUNTERS:
        for stage, short, val in _stage_kernels(_per_dispatch(pmc_dir, counter), dtype_tag):
            e = tot.setdefault(stage, {"kernels": []})
            if short not in e["kernels"]:
                e["kernels"].append(short)
            e[counter] = e.get(counter, 0.0) + val
    out = {}
    for stage, e in tot.items():
        if not all(c in e for c in BUSY_COUNTERS[:3]) or e["GRBM_GUI_ACTIVE"] <= 0:
            continue
        xcd_clk = e["GRBM_GUI_ACTIVE"] / N_XCD
        out[stage] = {"kernel": " + ".join(e["kernels"]),
                      "mfma_busy": round(e["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd_clk * N_CU * 4), 4),
                      "cu_busy": round(e["SQ_BUSY_CU_CYCLES"] / (xcd_clk * N_CU), 4),
                      **{c: e[c] for c in BUSY_COUNTERS if c in e}}
    return out


def busy_summary(pmc_dir: str, workload: str, command: str) -> None:
    """profiles/busy_<workload>.json from one rocprofv3 --pmc pass of BUSY_COUNTERS."""
    out = {"kernel_source_hash": kernel_source_hash(), "command": command,
           "stages": busy_from_pmc(pmc_dir)}
    path = os.path.join(ROOT, "profiles", f"busy_{workload}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(path, {k: v["mfma_busy"] for k, v in out["stages"].items()})


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


def _stats(xs) -> dict:
    import numpy as np

    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "min": round(float(a.min()), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "mean": round(float(a.mean()), 4)}


def _profile_json(prefix: str, workload: str):
    """A committed counter summary of this workload, if its kernel sources are the
    current ones (else None: the counters were taken on other code)."""
    path = os.path.join(ROOT, "profiles", f"{prefix}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t


def run_config(idx: int, args, cold_iters: int = 5) -> dict:
    """Time one workload: K steps of (map build, forward, backward as psa_bwd runs it:
    dQ with the preparation of its rows, then dK/dV) after W warm-up steps; HIP events
    on the launch stream around every stage of every step, and the wall clock between
    two device synchronisations around the K steps.  Then cold_iters steps, each after
    a 512 MiB write that evicts the 256 MB last-level cache (outside the timed stages)."""
    import numpy as np
    import torch

    from shared_prefix_block_amd import psa
    from shared_prefix_block_amd import workloads as wl

    dev = torch.device("cuda:0")
    cfg = wl.WORKLOADS[idx]
    lay = wl.layout_for(cfg)
    if args.layout == "chunked":
        if lay.kind != "tokens":
            sys.exit("--layout chunked needs a token-form workload")
        lay = wl.shuffled_tokens_layout(lay.specs, np.random.default_rng(cfg.idx),
                                        prompt_first=True, relabel=False, chunk=64,
                                        n_pad=lay.T - lay.T_real)
    elif args.layout == "bfs":
        if lay.kind != "tree":
            sys.exit("--layout bfs needs a tree workload")
        nl, paths = wl.reorder_tree(lay.node_lengths, lay.sample_paths)
        lay = wl.tree_layout(nl, paths, extra_pad=lay.T - lay.T_real)
    if args.fold:
        if lay.kind != "tokens":
            sys.exit("--fold needs a token-form workload (rollout groups)")
        return {"fold": fold_bench(cfg, lay, args.steps, args.warmup)}
    if args.nograd:
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
    grads = None
    if backward:
        grads = (torch.empty(q.shape, dtype=gdt, device=dev),
                 torch.empty(k.shape, dtype=gdt, device=dev),
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

    def new_events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]

    # timed region: K full steps, wall clock between two device synchronisations
    all_events = [new_events() for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    maps = []
    for s_ in range(args.steps):
        maps.append(step(all_events[s_]))
        if len(maps) > 2:
            maps.pop(0)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    del maps

    def stage_times(events_list):
        per = {nm: [] for nm in names}
        for evs in events_list:
            for i, nm in enumerate(names):
                per[nm].append(evs[i].elapsed_time(evs[i + 1]))
        return per

    per = stage_times(all_events)
    cold = []
    if cold_iters and not args.no_cold:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for i in range(cold_iters):
            scratch.fill_(i + 1)  # 512 MiB written: the last-level cache holds none of the inputs
            torch.cuda.synchronize(dev)
            evs = new_events()
            m = step(evs)
            torch.cuda.synchronize(dev)
            cold.append(evs)
            del m
        del scratch
    cper = stage_times(cold) if cold else None

    kept = kept_pairs(lay)
    tiles = info["n_full"] + info["n_partial"]
    d, hq = cfg.d, cfg.hq
    f_fwd, f_bwd = 4 * d, 10 * d
    tile_flops = tiles * TILE * TILE * hq * (f_fwd + (f_bwd if backward else 0))
    kept_flops = kept * hq * (f_fwd + (f_bwd if backward else 0))
    ms_step = wall * 1e3 / args.steps
    peak = PEAK_TFLOPS[dtype_name]
    fwd_peak = PEAK_FP8_FWD if dtype_name == "fp8" else peak
    med = {nm: float(np.median(per[nm])) for nm in names}
    mean = {nm: sum(per[nm]) / len(per[nm]) for nm in names}
    t_fwd = med["fwd"]
    t_bwd = med["bwd_dq"] + med["bwd_dkdv"] if backward else 0.0
    res = {
        "workload": describe(cfg, lay, args.layout, args.form), "name": cfg.name,
        "T": lay.T, "T_real": lay.T_real, "map_form": ["interval", "nodes"][info["form"]],
        "hq": cfg.hq, "hkv": cfg.hkv, "head_dim": d, "dtype": dtype_name, "passes": passes,
        "sigma": cfg.sigma,
        "grad_dtype": args.grad_dtype if backward else None,
        "bwd_p_ds": (("hi+lo bf16" if args.split else "bf16, hi+lo where large")
                     if backward and dtype_name == "bf16" else None),
        "tiles_128": {"full": info["n_full"], "partial": info["n_partial"]},
        "kept_pairs_per_head": kept,
        "ms_per_step": round(ms_step, 4),
        "tflops_unmasked_tiles": round(tile_flops / (ms_step * 1e-3) / 1e12, 2),
        "tflops_kept_pairs": round(kept_flops / (ms_step * 1e-3) / 1e12, 2),
        f"pct_{dtype_name}_peak": round(100 * tile_flops / (ms_step * 1e-3) / 1e12 / peak, 2),
        "fwd_pct_peak": round(100 * kept * hq * f_fwd / (t_fwd * 1e-3) / 1e12 / fwd_peak, 2),
        "bwd_pct_peak": (round(100 * kept * hq * f_bwd / (t_bwd * 1e-3) / 1e12 / peak, 2)
                         if backward else None),
        "tokens_per_s": round(lay.T_real / ((t_fwd + t_bwd) * 1e-3), 1),
        "stage_ms": {nm: _stats(per[nm]) for nm in names},
        "cold_stage_ms": ({nm: _stats(cper[nm]) for nm in names} if cper else None),
    }
    # MFMA busy and HBM rate of the attention kernels: committed rocprofv3 counter
    # summaries of this workload, when they were taken on the current kernel sources
    variant = f"_nograd_{args.nograd}" if args.nograd else ""
    if args.layout == "packed" and args.form == "auto" and not args.split:
        busy = _profile_json("busy" + variant, cfg.name)
        if busy:
            res["mfma_busy"] = {st: e["mfma_busy"] for st, e in busy["stages"].items()
                                if st in med}
        hbm = {}
        for st in names[1:]:
            t = _profile_json(f"traffic_{st}{variant}", cfg.name)
            if t and t.get("bytes_per_launch"):
                hbm[st] = {"bytes_per_launch": t["bytes_per_launch"],
                           "gb_per_s": round(t["bytes_per_launch"] / (med[st] * 1e-3) / 1e9, 1)}
        if hbm:
            res["hbm"] = hbm
    # the dominant kernel: algorithmic FLOPs per launch (fwd 4d; dK/dV 8d = S, dP, dV,
    # dK; dQ 2d: its S and dP are recomputations) per kept pair per q head, over its
    # event-timed average launch
    algo = {"fwd": 4 * d, "bwd_dkdv": 8 * d, "bwd_dq": 2 * d}
    cand = {k_: mean[k_] for k_ in algo if k_ in mean}
    dom = max(cand, key=cand.get)
    dom_peak = fwd_peak if dom == "fwd" else peak
    achieved = kept * hq * algo[dom] / (mean[dom] * 1e-3) / 1e12
    traffic = None
    t = _profile_json(f"traffic_{dom}{variant}", cfg.name)
    if t and args.layout == "packed" and args.form == "auto":
        traffic = t.get("bytes_per_launch")
    res["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                       "peak": round(dom_peak, 1), "unit": "TFLOP/s",
                       "frac": round(achieved / dom_peak, 4), "traffic": traffic,
                       "algorithmic_flops_per_launch": kept * hq * algo[dom],
                       "avg_launch_ms": round(mean[dom], 4)}
    res["_tile_flops"] = tile_flops
    if not args.no_cpu_baseline and args.layout == "packed" and lay.kind != "draft" \
            and not args.nograd:
        del q, k, v, do, o, lse, grads, ws
        torch.cuda.empty_cache()
        res["cpu_oracle"] = cpu_baseline(cfg, lay)
    return res


HEADLINE = 4  # the largest single-GPU workload: 19.5 TFLOP of kept-pair work per step


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=None,
                    help="time this workload alone (default: the long-prompt workload 4 as "
                         "the headline, and every workload 1-5 in the same line)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache steps")
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
    ap.add_argument("--busy-summary", metavar="PMC_DIR",
                    help="no timing: write profiles/busy_<workload>.json from one rocprofv3 "
                         "counter pass of " + " ".join(BUSY_COUNTERS) + " under PMC_DIR")
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
                    help="with --traffic-summary / --busy-summary: the command line the "
                         "counter passes ran, recorded")
    args = ap.parse_args()
    if args.traffic_summary or args.busy_summary:
        from shared_prefix_block_amd import workloads as wl
        name = wl.WORKLOADS[args.workload or HEADLINE].name
        if args.traffic_summary:
            traffic_summary(args.traffic_summary, name, args.calib_mb or 512,
                            args.traffic_command, args.nograd or "")
        if args.busy_summary:
            busy_summary(args.busy_summary, name, args.traffic_command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures the single-GPU hot path only: the shared-prefix attention "
              "path has no cross-GPU step here (groups and heads shard with no communication); "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from shared_prefix_block_amd import psa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    psa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    head = args.workload or HEADLINE
    special = (args.fold or args.nograd or args.layout != "packed" or args.form != "auto"
               or args.split or args.grad_dtype != "fp32")
    order = [head] if (args.workload or special) else [head] + [i for i in (1, 2, 3, 5)]
    results = {}
    for idx in order:
        print(f"# workload {idx}", file=sys.stderr, flush=True)
        results[idx] = run_config(idx, args)
        torch.cuda.empty_cache()
        if "fold" in results[idx]:
            print(json.dumps(results[idx]["fold"]), flush=True)
            return
    h = results[head]
    tile_flops = h.pop("_tile_flops")
    for r in results.values():
        r.pop("_tile_flops", None)
    value = tile_flops / (h["ms_per_step"] * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": h["dtype"],
        "data": "synthetic (seeded N(0, sigma) Q/K/V, N(0,1) dO; layouts as the workloads state)",
        "config": {"workload": h["workload"], "T": h["T"], "T_real": h["T_real"],
                   "map_form": h["map_form"], "hq": h["hq"], "hkv": h["hkv"],
                   "head_dim": h["head_dim"], "passes": h["passes"],
                   "grad_dtype": h["grad_dtype"], "bwd_p_ds": h["bwd_p_ds"],
                   "tiles_128": h["tiles_128"], "kept_pairs_per_head": h["kept_pairs_per_head"]},
        f"pct_{h['dtype']}_peak": h[f"pct_{h['dtype']}_peak"],
        "kept_pair_tflops": h["tflops_kept_pairs"],
        "fwd_pct_peak": h["fwd_pct_peak"],
        "bwd_pct_peak": h["bwd_pct_peak"],
        "tokens_per_s": h["tokens_per_s"],
        "stage_ms": h["stage_ms"],
        "roofline": h["roofline"],
    }
    if "cpu_oracle" in h:
        c = h["cpu_oracle"]
        est = c["est_fwd_bwd_s"] or c["est_fwd_s"]
        out["cpu_baseline"] = {"value": round(tile_flops / est / 1e12, 6), "unit": "TFLOP/s",
                               "cores": c["blas_threads"], "kind": "oracle",
                               "sample": c["sample"],
                               "affinity_cores": len(os.sched_getaffinity(0)),
                               "cpu_model": cpu_model()}
    out["configs"] = {str(i): r for i, r in results.items()}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
