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
class Config:
    """One synthetic workload: layout, head counts, head dim, dtype, passes."""

    idx: int
    name: str
    kind: str  # "tokens" or "tree"
    hq: int
    hkv: int
    d: int
    dtype: str  # "fp32" or "bf16"
    sigma: float
    passes: str  # "fwd" or "fwd+bwd"
    pad_multiple: int = 1
    note: str = ""


CONFIGS = {
    1: Config(1, "1grp_P64_G4_R32", "tokens", 2, 2, 64, "fp32", 1.0, "fwd",
              note="1 group, P=64, G=4 x R=32 (T=192), fp32, forward only"),
    2: Config(2, "8grp_P512_G8_R256", "tokens", 32, 8, 128, "bf16", 1.0, "fwd+bwd",
              note="8 groups, P=512, G=8 x R=256 (T=20480), GQA 32/8, d=128, bf16"),
    3: Config(3, "16grp_varlen", "tokens", 16, 4, 128, "bf16", 1.0, "fwd+bwd",
              pad_multiple=128,
              note="16 groups, P~U[128,2048], G=16, R~U[64,1024], padded to x128, GQA 16/4"),
    4: Config(4, "2grp_P16384_G64_R512", "tokens", 8, 8, 128, "bf16", 0.5, "fwd+bwd",
              note="2 groups, P=16384, G=64 x R=512 (T=98304), 8/8 heads, N(0, 0.5)"),
    5: Config(5, "8trees_1024_4x256_4x384", "tree", 16, 8, 256, "bf16", 1.0, "fwd+bwd",
              note="8 trees: root 1024 -> 4 x 256 -> 4 x 384 leaves (T=65536), GQA 16/8, d=256"),
}


# ----------------------------------------------------------------------------
# layouts
# ----------------------------------------------------------------------------
def group_specs(cfg: Config, seed: Optional[int] = None) -> GroupSpecs:
    """(P_g, [R_g0, R_g1, ...]) for every group of a token-form config."""
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
    raise ValueError(f"config {cfg.idx} is not token-form")


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


def layout_for(cfg: Config, seed: Optional[int] = None) -> Layout:
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
# tensors
# ----------------------------------------------------------------------------
TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


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


def config_tensors(cfg: Config, layout: Layout, seed: Optional[int] = None):
    return make_tensors(layout.T, cfg.hq, cfg.hkv, cfg.d, cfg.dtype, cfg.sigma,
                        cfg.idx if seed is None else seed,
                        with_grad_out=(cfg.passes != "fwd"))
