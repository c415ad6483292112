"""Dense visibility mask of shared-prefix / prefix-tree attention (CPU oracle).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.  The
oracle shares no code with the HIP library and never sees its tile map or its
per-token interval encoding: the mask is evaluated element by element from the
metadata, exactly as the pages state the rule.

Token form (unsloth ``prefix_grouper_kernel.py`` page, function ``_make_mask_mod``
and its docstring; the module docstring's "Mask semantics" gives the same rule
without the causal guard on the prefix branch, see reading A1 below)::

    keep(q, kv) = same_group(q, kv) and kv <= q and
                  ( is_prefix[kv] or ( not is_prefix[q] and suffix[kv] == suffix[q] ) )

Readings taken where the pages are open:

* A1 - prefix rows are causal: the implemented rule guards the prefix branch with
  kv <= q.  A suffix row still sees its whole prefix because the prefix precedes
  the suffixes in the packed layout.
* A2 - pad tokens (any negative group id) see nothing and are seen by nothing.  The
  page's docstring says pad rows attend to nothing and return 0.
* Tree form (Automodel PR #2564 page, PR description: every completion attends in
  full to the shared prompt and causally to itself; "multi-turn / shared-prefix
  prefix-tree"): a token of node b sees every token of each strict ancestor of b and
  the tokens of b at or before itself.  Node n owns the n-th contiguous run of
  ``node_lengths``; parents come from ``sample_paths`` (root first).  Tokens past
  ``sum(node_lengths)`` are pads.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np


class TokenMeta:
    """Per-token (group, suffix, is_prefix) labels."""

    kind = "tokens"

    def __init__(self, group, suffix, is_prefix):
        self.group = np.asarray(group, dtype=np.int64)
        self.suffix = np.asarray(suffix, dtype=np.int64)
        self.is_prefix = np.asarray(is_prefix).astype(bool)
        if not (self.group.shape == self.suffix.shape == self.is_prefix.shape):
            raise ValueError("label arrays differ in length")
        self.T = int(self.group.shape[0])

    def real(self) -> np.ndarray:
        return self.group >= 0

    def mask(self, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
        """Boolean [len(rows), len(cols)]: may row ``rows[a]`` attend to ``cols[b]``."""
        q = np.asarray(rows, dtype=np.int64)[:, None]
        kv = np.asarray(cols, dtype=np.int64)[None, :]
        g, s, p = self.group, self.suffix, self.is_prefix
        real = (g[q] >= 0) & (g[kv] >= 0)
        same_group = g[q] == g[kv]
        causal = kv <= q
        prefix_branch = p[kv]
        suffix_branch = (~p[q]) & (s[kv] == s[q])
        return real & same_group & causal & (prefix_branch | suffix_branch)

    def components(self) -> List[np.ndarray]:
        """Token index sets that can see each other at all (one per group id).

        Tokens of different groups never see each other (the same_group conjunct),
        so the dense computation may be restricted to one group at a time."""
        real = np.nonzero(self.group >= 0)[0]
        out = []
        for gid in np.unique(self.group[real]):
            out.append(np.nonzero(self.group == gid)[0])
        return out


class TreeMeta:
    """Prefix tree given as node_lengths + sample_paths (node indices root -> leaf)."""

    kind = "tree"

    def __init__(self, node_lengths: Sequence[int], sample_paths: Sequence[Sequence[int]],
                 T: Optional[int] = None):
        self.node_lengths = [int(x) for x in node_lengths]
        n = len(self.node_lengths)
        if any(x < 0 for x in self.node_lengths):
            raise ValueError("negative node length")
        parent = [None] * n
        for path in sample_paths:
            prev = -1
            for node in path:
                node = int(node)
                if not 0 <= node < n:
                    raise ValueError("path node out of range")
                if parent[node] is None:
                    parent[node] = prev
                elif parent[node] != prev:
                    raise ValueError(f"node {node} has two parents")
                prev = node
        if any(p is None for p in parent):
            raise ValueError("a node lies on no sample path")
        self.parent = [int(p) for p in parent]
        # strict-ancestor relation anc[a, b]: a is a strict ancestor of b
        anc = np.zeros((n, n), dtype=bool)
        for b in range(n):
            a = self.parent[b]
            seen = 0
            while a >= 0:
                anc[a, b] = True
                a = self.parent[a]
                seen += 1
                if seen > n:
                    raise ValueError("parent cycle")
        self.anc = anc
        t_real = int(sum(self.node_lengths))
        self.T = t_real if T is None else int(T)
        if self.T < t_real:
            raise ValueError("T shorter than the tree")
        node_of = np.full(self.T, -1, dtype=np.int64)
        pos = 0
        for i, ln in enumerate(self.node_lengths):
            node_of[pos:pos + ln] = i
            pos += ln
        self.node_of = node_of

    def real(self) -> np.ndarray:
        return self.node_of >= 0

    def mask(self, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
        q = np.asarray(rows, dtype=np.int64)[:, None]
        kv = np.asarray(cols, dtype=np.int64)[None, :]
        nq = self.node_of[q]
        nk = self.node_of[kv]
        real = (nq >= 0) & (nk >= 0)
        nq0 = np.where(nq >= 0, nq, 0)
        nk0 = np.where(nk >= 0, nk, 0)
        ancestor = self.anc[nk0, nq0]
        same_node_causal = (nk == nq) & (kv <= q)
        return real & (ancestor | same_node_causal)

    def components(self) -> List[np.ndarray]:
        """Token index sets of each tree (nodes sharing a root)."""
        n = len(self.node_lengths)
        root = list(range(n))
        for i in range(n):
            r = i
            while self.parent[r] >= 0:
                r = self.parent[r]
            root[i] = r
        root = np.asarray(root, dtype=np.int64)
        real = self.node_of >= 0
        tok_root = np.full(self.T, -1, dtype=np.int64)
        tok_root[real] = root[self.node_of[real]]
        out = []
        for r in np.unique(tok_root[real]):
            out.append(np.nonzero(tok_root == r)[0])
        return out


def meta_from_layout(layout):
    """Build the oracle's metadata object from a workloads.Layout (plain arrays only)."""
    if layout.kind == "draft":
        from .draft import DraftMeta
        x = layout.extra
        return DraftMeta(x["ctx_len"], x["block_size"], x["anchors"], x["keep"], x["ctx_doc"],
                         x["anchor_doc"], x["causal"], layout.T)
    if layout.kind == "tokens":
        return TokenMeta(layout.group, layout.suffix, layout.is_prefix)
    return TreeMeta(layout.node_lengths, layout.sample_paths, layout.T)


def dense_mask(meta) -> np.ndarray:
    """The full [T, T] mask (small T only)."""
    idx = np.arange(meta.T)
    return meta.mask(idx, idx)


def kept_pairs(meta, block_rows: int = 1024) -> int:
    """Number of kept (q, kv) pairs, counted from the element-wise mask."""
    total = 0
    for comp in meta.components():
        for r0 in range(0, len(comp), block_rows):
            total += int(meta.mask(comp[r0:r0 + block_rows], comp).sum())
    return total
