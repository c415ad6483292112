"""Seeded synthetic inputs for shared-prefix / prefix-tree attention.

This module only draws inputs: rollout layouts (prompt and completion lengths, or a
prefix tree), the per-token metadata arrays that describe them, and the Q/K/V/dO
tensors.  It holds none of the attention arithmetic, so both the HIP path and the
CPU oracle may use it.

Layouts follow the shared-prefix fold described on the unsloth
``prefix_grouper_kernel.py`` page (module docstring and
``build_seg_info_multigroup``): each group is packed flat as
``[prefix | s_0 | s_1 | ...]`` and groups follow one another.  Per-token metadata
is ``group`` (int32, negative for a pad token), ``suffix`` (int32, -1 on prefix
tokens, globally increasing over the suffixes) and ``is_prefix`` (uint8).  Pad
tokens are appended at the end up to the requested multiple.

Draft layouts (``draft_layout``) are the second mask workload: a block-diffusion
drafter's context of packed documents followed by blocks of draft tokens anchored in
it (Automodel PR #3023 page, PR description).

Prefix trees follow the Automodel PR #2564 page ("Changelog": ``node_lengths`` and
``sample_paths`` carried on the batch): nodes are listed in depth-first pre-order,
node ``n`` owns the n-th contiguous run of ``node_lengths`` tokens, and each sample
path lists node indices from a root down to a leaf.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

PAD_GROUP = -1

GroupSpecs = List[Tuple[int, List[int]]]


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: layout, head counts, head dim, dtype, passes."""

    idx: int
    name: str
    kind: str  # "tokens", "tree" or "draft"
    hq: int
    hkv: int
    d: int
    dtype: str  # "fp32" or "bf16"
    sigma: float
    passes: str  # "fwd" or "fwd+bwd"
    pad_multiple: int = 1
    note: str = ""


WORKLOADS = {
    1: Workload(1, "1grp_P64_G4_R32", "tokens", 2, 2, 64, "fp32", 1.0, "fwd",
              note="1 group, P=64, G=4 x R=32 (T=192), fp32, forward only"),
    2: Workload(2, "8grp_P512_G8_R256", "tokens", 32, 8, 128, "bf16", 1.0, "fwd+bwd",
              note="8 groups, P=512, G=8 x R=256 (T=20480), GQA 32/8, d=128, bf16"),
    3: Workload(3, "16grp_varlen", "tokens", 16, 4, 128, "bf16", 1.0, "fwd+bwd",
              pad_multiple=128,
              note="16 groups, P~U[128,2048], G=16, R~U[64,1024], padded to x128, GQA 16/4"),
    4: Workload(4, "2grp_P16384_G64_R512", "tokens", 8, 8, 128, "bf16", 0.5, "fwd+bwd",
              note="2 groups, P=16384, G=64 x R=512 (T=98304), 8/8 heads, N(0, 0.5)"),
    5: Workload(5, "8trees_1024_4x256_4x384", "tree", 16, 8, 256, "bf16", 1.0, "fwd+bwd",
              note="8 trees: root 1024 -> 4 x 256 -> 4 x 384 leaves (T=65536), GQA 16/8, d=256"),
    # the second mask workload: a block-diffusion drafter's packed-document batch
    6: Workload(6, "draft_4doc_4096_bs16", "draft", 16, 4, 128, "bf16", 1.0, "fwd+bwd",
              note="draft blocks: 4 packed documents of 4096 context tokens, 512 blocks of "
                   "16 per document (T=49152), bidirectional blocks, GQA 16/4, d=128"),
}


# ----------------------------------------------------------------------------
# layouts
# ----------------------------------------------------------------------------
def group_specs(cfg: Workload, seed: Optional[int] = None) -> GroupSpecs:
    """(P_g, [R_g0, R_g1, ...]) for every group of a token-form workload."""
    if cfg.idx == 1:
        return [(64, [32] * 4)]
    if cfg.idx == 2:
        return [(512, [256] * 8) for _ in range(8)]
    if cfg.idx == 3:
        gen = torch.Generator("cpu").manual_seed(cfg.idx if seed is None else seed)
        specs = []
        for _ in range(16):
            p = int(torch.randint(128, 2049, (1,), generator=gen))
            rs = [int(torch.randint(64, 1025, (1,), generator=gen)) for _ in range(16)]
            specs.append((p, rs))
        return specs
    if cfg.idx == 4:
        return [(16384, [512] * 64) for _ in range(2)]
    raise ValueError(f"workload {cfg.idx} is not token-form")


def tree_spec(n_trees: int = 8, root: int = 1024, n_branch: int = 4, branch: int = 256,
              n_leaf: int = 4, leaf: int = 384) -> Tuple[List[int], List[List[int]]]:
    """node_lengths and sample_paths of ``n_trees`` identical 3-level trees, DFS pre-order."""
    node_lengths: List[int] = []
    paths: List[List[int]] = []
    for _ in range(n_trees):
        r = len(node_lengths)
        node_lengths.append(root)
        for _b in range(n_branch):
            b = len(node_lengths)
            node_lengths.append(branch)
            for _l in range(n_leaf):
                lf = len(node_lengths)
                node_lengths.append(leaf)
                paths.append([r, b, lf])
    return node_lengths, paths


def token_labels(specs: GroupSpecs, pad_multiple: int = 1, extra_pad: int = 0,
                 first_suffix_id: int = 0):
    """Per-token (group, suffix, is_prefix) arrays of groups packed flat.

    Returns (group int32 [T], suffix int32 [T], is_prefix uint8 [T], T_real).
    Pad tokens (group = PAD_GROUP, suffix = PAD_GROUP, is_prefix = 0) are appended
    so that T is a multiple of ``pad_multiple``, plus ``extra_pad`` more.
    """
    group: List[int] = []
    suffix: List[int] = []
    is_prefix: List[int] = []
    sid = first_suffix_id
    for gid, (p, rs) in enumerate(specs):
        group += [gid] * p
        suffix += [-1] * p
        is_prefix += [1] * p
        for r in rs:
            group += [gid] * r
            suffix += [sid] * r
            is_prefix += [0] * r
            sid += 1
    t_real = len(group)
    t = -(-t_real // pad_multiple) * pad_multiple if pad_multiple > 1 else t_real
    t += extra_pad
    n_pad = t - t_real
    group += [PAD_GROUP] * n_pad
    suffix += [PAD_GROUP] * n_pad
    is_prefix += [0] * n_pad
    return (np.asarray(group, np.int32), np.asarray(suffix, np.int32),
            np.asarray(is_prefix, np.uint8), t_real)


@dataclass
class Layout:
    """The metadata of one workload, in the form the library and the oracle take."""

    kind: str
    T: int
    T_real: int
    group: Optional[np.ndarray] = None
    suffix: Optional[np.ndarray] = None
    is_prefix: Optional[np.ndarray] = None
    specs: Optional[GroupSpecs] = None
    node_lengths: Optional[List[int]] = None
    sample_paths: Optional[List[List[int]]] = None
    extra: dict = field(default_factory=dict)


def layout_for(cfg: Workload, seed: Optional[int] = None) -> Layout:
    if cfg.kind == "draft":
        rng = np.random.default_rng(cfg.idx if seed is None else seed)
        return draft_layout([4096] * 4, 16, 512, rng)
    if cfg.kind == "tree":
        nl, sp = tree_spec()
        t = int(sum(nl))
        return Layout("tree", t, t, node_lengths=nl, sample_paths=sp)
    specs = group_specs(cfg, seed)
    g, s, p, t_real = token_labels(specs, cfg.pad_multiple)
    return Layout("tokens", int(g.shape[0]), t_real, group=g, suffix=s, is_prefix=p,
                  specs=specs)


def tokens_layout(specs: GroupSpecs, pad_multiple: int = 1, extra_pad: int = 0) -> Layout:
    g, s, p, t_real = token_labels(specs, pad_multiple, extra_pad)
    return Layout("tokens", int(g.shape[0]), t_real, group=g, suffix=s, is_prefix=p,
                  specs=specs)


def tree_layout(node_lengths: Sequence[int], sample_paths: Sequence[Sequence[int]],
                extra_pad: int = 0) -> Layout:
    t_real = int(sum(node_lengths))
    return Layout("tree", t_real + extra_pad, t_real, node_lengths=list(node_lengths),
                  sample_paths=[list(p) for p in sample_paths])


# ----------------------------------------------------------------------------
# random tiny layouts (fuzz)
# ----------------------------------------------------------------------------
def random_group_specs(rng: np.random.Generator, max_groups: int = 3, max_p: int = 40,
                       max_g: int = 4, max_r: int = 40) -> GroupSpecs:
    n = int(rng.integers(1, max_groups + 1))
    return [(int(rng.integers(0, max_p + 1)),
             [int(rng.integers(0, max_r + 1)) for _ in range(int(rng.integers(0, max_g + 1)))])
            for _ in range(n)]


def random_tree(rng: np.random.Generator, max_nodes: int = 8, max_len: int = 40,
                max_trees: int = 2) -> Tuple[List[int], List[List[int]]]:
    """A random forest in DFS pre-order with one sample path per leaf."""
    node_lengths: List[int] = []
    parent: List[int] = []
    for _ in range(int(rng.integers(1, max_trees + 1))):
        budget = int(rng.integers(1, max_nodes + 1))
        stack: List[int] = []
        for k in range(budget):
            n = len(node_lengths)
            if k == 0:
                parent.append(-1)
                stack = [n]
            else:
                depth = int(rng.integers(1, len(stack) + 1))
                stack = stack[:depth]
                parent.append(stack[-1])
                stack.append(n)
            node_lengths.append(int(rng.integers(0, max_len + 1)))
    children = {i: [] for i in range(len(node_lengths))}
    for c, p in enumerate(parent):
        if p >= 0:
            children[p].append(c)
    paths = []
    for n in range(len(node_lengths)):
        if not children[n]:
            path = [n]
            while parent[path[-1]] >= 0:
                path.append(parent[path[-1]])
            paths.append(path[::-1])
    return node_lengths, paths


# ----------------------------------------------------------------------------
# layouts that are not packed (interleaved runs, ids out of order, other node orders)
# ----------------------------------------------------------------------------
def shuffled_tokens_layout(specs: GroupSpecs, rng: np.random.Generator,
                           prompt_first: bool = True, n_pad: int = 0,
                           relabel: bool = True, chunk: int = 1) -> Layout:
    """The groups of ``specs`` with their tokens interleaved at random.

    Every prompt and every completion keeps its own token order, but the runs are
    merged ``chunk`` tokens at a time (the last piece of a run may be shorter) in a
    random order of runs (as completions generated side by side and appended in
    turns would be): with ``prompt_first`` a completion's
    tokens start only after its group's whole prompt (each unfolded sample keeps its
    flat order), without it prompt tokens may follow completion tokens.  ``n_pad``
    pad tokens go to random places; with ``relabel`` group and completion ids are
    replaced by random distinct values in no particular order.  ``extra["pos"]``
    gives, for every token of the packed layout, its position in this one.
    """
    g0, s0, p0, t_real = token_labels(specs)
    streams = []  # (group index, is prompt, packed token indices)
    t = 0
    for gi, (p, rs) in enumerate(specs):
        streams.append((gi, True, list(range(t, t + p))))
        t += p
        for r in rs:
            streams.append((gi, False, list(range(t, t + r))))
            t += r
    prompt_left = {gi: p for gi, (p, _) in enumerate(specs)}
    heads = [0] * len(streams)
    order: List[int] = []
    while len(order) < t_real:
        ready = [k for k, (gi, isp, toks) in enumerate(streams)
                 if heads[k] < len(toks) and (isp or not prompt_first or prompt_left[gi] == 0)]
        k = ready[int(rng.integers(0, len(ready)))]
        gi, isp, toks = streams[k]
        take = min(chunk, len(toks) - heads[k])
        order += toks[heads[k]:heads[k] + take]
        heads[k] += take
        if isp:
            prompt_left[gi] -= take
    T = t_real + n_pad
    slots = np.sort(rng.choice(T, size=t_real, replace=False)) if T else np.zeros(0, np.int64)
    pos = np.zeros(t_real, np.int64)
    pos[np.asarray(order, np.int64)] = slots
    group = np.full(T, PAD_GROUP, np.int32)
    suffix = np.full(T, PAD_GROUP, np.int32)
    is_prefix = np.zeros(T, np.uint8)
    gmap = np.arange(len(specs))
    smap_from = np.unique(s0[s0 >= 0]) if t_real else np.zeros(0, np.int32)
    smap_to = smap_from
    if relabel:
        gmap = rng.choice(10**6, size=len(specs), replace=False)
        smap_to = rng.choice(10**6, size=len(smap_from), replace=False) - 1000
    group[pos] = gmap[g0[:t_real]]
    sfx = s0[:t_real].copy()
    for a, b_ in zip(smap_from, smap_to):
        sfx[s0[:t_real] == a] = b_
    suffix[pos] = sfx
    is_prefix[pos] = p0[:t_real]
    return Layout("tokens", T, t_real, group=group, suffix=suffix, is_prefix=is_prefix,
                  specs=specs, extra={"pos": pos})


def reorder_tree(node_lengths: Sequence[int], sample_paths: Sequence[Sequence[int]],
                 rng: Optional[np.random.Generator] = None):
    """The same forest with its nodes renumbered: breadth-first when ``rng`` is None,
    else in a random order that still puts every parent before its children.  Node n
    keeps its tokens (they move with it).  Returns (node_lengths, sample_paths)."""
    n = len(node_lengths)
    parent = [-1] * n
    for path in sample_paths:
        for a, b_ in zip(path[:-1], path[1:]):
            parent[b_] = a
    placed: List[int] = []
    done = [False] * n
    if rng is None:
        depth = [0] * n
        for v in range(n):  # packed order: parents come first
            depth[v] = depth[parent[v]] + 1 if parent[v] >= 0 else 0
        placed = sorted(range(n), key=lambda v: (depth[v], v))
    else:
        while len(placed) < n:
            ready = [v for v in range(n) if not done[v] and (parent[v] < 0 or done[parent[v]])]
            v = ready[int(rng.integers(0, len(ready)))]
            done[v] = True
            placed.append(v)
    new_index = {v: i for i, v in enumerate(placed)}
    nl = [int(node_lengths[v]) for v in placed]
    paths = [[new_index[v] for v in path] for path in sample_paths]
    return nl, paths


# ----------------------------------------------------------------------------
# draft blocks of a block-diffusion drafter over packed documents
# ----------------------------------------------------------------------------
def draft_layout(doc_lens: Sequence[int], block_size: int, blocks_per_doc,
                 rng: np.random.Generator, causal: bool = False, keep_frac: float = 1.0,
                 extra_pad: int = 0, doc_ids: Optional[Sequence[int]] = None) -> Layout:
    """Context = the documents packed in order; per document, ``blocks_per_doc`` anchors
    drawn uniformly where a whole block stays inside the document (anchor + block_size
    - 1 within it, as the Automodel PR #3023 page samples them; a shorter document gets
    none), sorted; blocks follow the context in that order.  ``keep_frac`` of the blocks
    are kept (the rest masked out).  ``extra`` holds the draft-mask arguments."""
    n_docs = len(doc_lens)
    per = ([int(blocks_per_doc)] * n_docs if np.isscalar(blocks_per_doc)
           else [int(x) for x in blocks_per_doc])
    ids = list(range(n_docs)) if doc_ids is None else [int(x) for x in doc_ids]
    ctx_doc = np.concatenate([np.full(n, i, np.int32) for i, n in zip(ids, doc_lens)] +
                             [np.zeros(0, np.int32)])
    anchors, adoc = [], []
    start = 0
    for i, n, k in zip(ids, doc_lens, per):
        hi = n - (block_size - 1)  # anchors 0 .. n - block_size: the block ends in the document
        if hi > 0 and k > 0:
            anchors += sorted(start + int(a) for a in rng.integers(0, hi, size=k))
            adoc += [i] * k
        start += n
    S = int(sum(doc_lens))
    N = len(anchors)
    keep = (rng.random(N) < keep_frac).astype(np.uint8) if keep_frac < 1.0 else \
        np.ones(N, np.uint8)
    t_real = S + N * block_size
    return Layout("draft", t_real + extra_pad, t_real,
                  extra={"ctx_len": S, "block_size": int(block_size),
                         "anchors": np.asarray(anchors, np.int32), "keep": keep,
                         "ctx_doc": ctx_doc, "anchor_doc": np.asarray(adoc, np.int32),
                         "causal": bool(causal)})


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------
TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


def make_tensors(T: int, hq: int, hkv: int, d: int, dtype: str, sigma: float = 1.0,
                 seed: int = 0, with_grad_out: bool = True):
    """Q [T,hq,d], K/V [T,hkv,d] and dO [T,hq,d]: fp32 N(0, sigma^2) draws (dO: N(0,1))
    from a seeded CPU generator, then rounded to ``dtype`` (nearest even)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = TORCH_DTYPE[dtype]
    q = (torch.randn(T, hq, d, generator=gen) * sigma).to(dt)
    k = (torch.randn(T, hkv, d, generator=gen) * sigma).to(dt)
    v = (torch.randn(T, hkv, d, generator=gen) * sigma).to(dt)
    do = torch.randn(T, hq, d, generator=gen).to(dt) if with_grad_out else None
    return q, k, v, do


def workload_tensors(cfg: Workload, layout: Layout, seed: Optional[int] = None):
    return make_tensors(layout.T, cfg.hq, cfg.hkv, cfg.d, cfg.dtype, cfg.sigma,
                        cfg.idx if seed is None else seed,
                        with_grad_out=(cfg.passes != "fwd"))
