"""The unfolded view of a folded rollout layout, written independently of the oracle.

A folded group ``[prefix | s_0 | s_1 | ...]`` stands for G ordinary sequences
``[prefix | s_i]``; a prefix tree stands for one sequence per root-to-leaf path
(Automodel PR #2564 page, PR description: the prompt is encoded once instead of N
times; each completion sees the whole prompt and itself causally).  Plain causal
attention over an unfolded sequence is the meaning of the folded mask, so these
helpers give the tests a definition of visibility and of the kept-pair count that
does not go through the oracle's mask rule.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def group_sequences(specs) -> Tuple[List[np.ndarray], List[Tuple[int, int]]]:
    """Flat token indices of every unfolded sequence, plus (start, end) of each suffix.

    A group with no suffix contributes its prefix alone."""
    seqs, spans = [], []
    base = 0
    for p, rs in specs:
        prefix = np.arange(base, base + p)
        cur = base + p
        if not rs:
            seqs.append(prefix)
        for r in rs:
            seqs.append(np.concatenate([prefix, np.arange(cur, cur + r)]))
            spans.append((cur, cur + r))
            cur += r
        base = cur
    return seqs, spans


def tree_sequences(node_lengths: Sequence[int], paths: Sequence[Sequence[int]]):
    starts = np.concatenate([[0], np.cumsum(node_lengths)]).astype(np.int64)
    seqs = []
    for path in paths:
        seqs.append(np.concatenate([np.arange(starts[n], starts[n + 1]) for n in path])
                    if path else np.zeros(0, np.int64))
    return seqs


def visibility_from_sequences(T: int, seqs: Sequence[np.ndarray]) -> np.ndarray:
    """vis[q, kv]: kv is at or before q in some unfolded sequence that contains q."""
    vis = np.zeros((T, T), dtype=bool)
    for s in seqs:
        for i, q in enumerate(s):
            vis[q, s[: i + 1]] = True
    return vis


def kept_closed_form_groups(specs) -> int:
    """P(P+1)/2 + sum_i (R_i * P + R_i (R_i + 1) / 2) per group."""
    total = 0
    for p, rs in specs:
        total += p * (p + 1) // 2
        for r in rs:
            total += r * p + r * (r + 1) // 2
    return total


def kept_closed_form_tree(node_lengths: Sequence[int], paths: Sequence[Sequence[int]]) -> int:
    """L(L+1)/2 + L * (tokens in strict ancestors) per node."""
    anc_tokens = {}
    for path in paths:
        acc = 0
        for n in path:
            anc_tokens[n] = acc
            acc += node_lengths[n]
    return sum(ln * (ln + 1) // 2 + ln * anc_tokens[n] for n, ln in enumerate(node_lengths))


def n_visible_groups(specs, T: int) -> np.ndarray:
    """Number of keys each token sees: i+1 at prefix offset i, P+j+1 at suffix offset j."""
    n = np.zeros(T, dtype=np.int64)
    base = 0
    for p, rs in specs:
        n[base:base + p] = np.arange(1, p + 1)
        cur = base + p
        for r in rs:
            n[cur:cur + r] = p + np.arange(1, r + 1)
            cur += r
        base = cur
    return n
