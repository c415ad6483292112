"""Visibility rule of the packed-document draft mask (CPU oracle).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.  It
shares no code with the HIP library and never imports it.

What the mask is (Automodel PR #3023 page, PR description and the review comment
that lists the mask builder's arguments; Model-Optimizer PR #2757 page, the commit
note on the generation mask): a block-diffusion drafter's queries are draft blocks
only and its keys are the context followed by the drafts.  Block b, anchored at
context position a_b, holds ``block_size`` draft tokens; a block whose keep flag is
off is not trained.  A draft query of block b sees

* the context before its anchor, restricted (when documents are packed) to the
  anchor's document: context position c is visible iff c < a_b and
  ctx_doc[c] == anchor_doc[b];
* the draft tokens of its own block: all of them, or (the causal variant) those at
  or before its own offset in the block.

Nothing else: no other block's drafts, no later context, nothing from other
documents; a block whose keep flag is off sees nothing and is seen by nothing, and
context tokens are keys only (as query rows they see nothing).

The flat index layout shared with the library: positions [0, ctx_len) are the
context, block b's token j sits at ctx_len + b * block_size + j, and any position at
or beyond ctx_len + n_blocks * block_size is a pad.

Readings taken where the pages are open:

* D1 - "before its anchor" is strict: the block itself starts at the anchor (its
  first token is the anchor token), and at generation a block anchored at ctx_len
  sees the whole context and nothing past it.
* D2 - without document ids the whole context is one document.
* D3 - a block's document is given (``anchor_doc``), as the pages pass it; ids are
  compared for equality only, so documents need not be contiguous.
* D4 - the sliding-window variant named on the Model-Optimizer page is not part of
  this rule.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np


class DraftMeta:
    """Packed-document draft layout: context + blocks of draft tokens."""

    kind = "draft"

    def __init__(self, ctx_len: int, block_size: int, anchors: Sequence[int],
                 keep: Optional[Sequence[int]] = None, ctx_doc: Optional[Sequence[int]] = None,
                 anchor_doc: Optional[Sequence[int]] = None, causal: bool = False,
                 T: Optional[int] = None):
        self.S = int(ctx_len)
        self.bs = int(block_size)
        self.anchors = np.asarray(anchors, dtype=np.int64)
        self.N = int(self.anchors.shape[0])
        self.keep = (np.ones(self.N, dtype=bool) if keep is None
                     else np.asarray(keep).astype(bool))
        if (ctx_doc is None) != (anchor_doc is None):
            raise ValueError("ctx_doc and anchor_doc go together")
        self.ctx_doc = (np.zeros(self.S, np.int64) if ctx_doc is None
                        else np.asarray(ctx_doc, dtype=np.int64))
        self.anchor_doc = (np.zeros(self.N, np.int64) if anchor_doc is None
                           else np.asarray(anchor_doc, dtype=np.int64))
        if self.bs < 1 or self.S < 0:
            raise ValueError("block_size >= 1 and ctx_len >= 0")
        if self.ctx_doc.shape != (self.S,) or self.anchor_doc.shape != (self.N,) or \
                self.keep.shape != (self.N,):
            raise ValueError("array lengths")
        if ((self.anchors < 0) | (self.anchors > self.S)).any():
            raise ValueError("anchor outside [0, ctx_len]")
        self.causal = bool(causal)
        self.t_real = self.S + self.N * self.bs
        self.T = self.t_real if T is None else int(T)
        if self.T < self.t_real:
            raise ValueError("T shorter than the layout")

    def _decode(self, t: np.ndarray):
        """(is_ctx, is_draft, block, offset) of flat positions."""
        is_ctx = t < self.S
        is_draft = (t >= self.S) & (t < self.t_real)
        rel = np.where(is_draft, t - self.S, 0)
        return is_ctx, is_draft, rel // self.bs, rel % self.bs

    def real(self) -> np.ndarray:
        t = np.arange(self.T)
        return t < self.t_real

    def mask(self, rows, cols) -> np.ndarray:
        q = np.asarray(rows, dtype=np.int64)[:, None]
        kv = np.asarray(cols, dtype=np.int64)[None, :]
        if self.N == 0:  # no block: no query
            return np.zeros((q.shape[0], kv.shape[1]), dtype=bool)
        _, q_draft, qb, qj = self._decode(q)
        k_ctx, k_draft, kb, kj = self._decode(kv)
        q_live = q_draft & self.keep[qb]
        kvc = np.where(k_ctx, kv, 0)
        sees_ctx = k_ctx & (kv < self.anchors[qb]) & (self.ctx_doc[kvc] == self.anchor_doc[qb])
        same_block = k_draft & (kb == qb)
        in_block = same_block & ((kj <= qj) if self.causal else True)
        return q_live & (sees_ctx | in_block)

    def components(self) -> List[np.ndarray]:
        """Token sets that can see each other at all: per document, its context tokens
        and the kept blocks anchored in it (blocks never see another document)."""
        out = []
        for doc in np.unique(np.concatenate([self.ctx_doc, self.anchor_doc[self.keep]])):
            ctx = np.nonzero(self.ctx_doc == doc)[0]
            blocks = np.nonzero(self.keep & (self.anchor_doc == doc))[0]
            drafts = (self.S + blocks[:, None] * self.bs + np.arange(self.bs)[None, :]).ravel()
            comp = np.concatenate([ctx, np.sort(drafts)]).astype(np.int64)
            if len(comp):
                out.append(comp)
        return out
