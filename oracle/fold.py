"""Fold of rollout groups into the flat shared-prefix layout, and its unfold (CPU oracle).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.  It shares
no code with the HIP library and never imports it.

What the fold computes (Automodel PR #2564 page: PR description, "Changelog" entry for
``fold_shared_prefix_rollouts``, and the commit note on pre-shifted labels):

* one group = one prompt and the completions sampled from it; it is stored once as
  ``[prompt | c_0 | c_1 | ...]`` and groups follow one another (the unsloth
  ``prefix_grouper_kernel.py`` page packs several groups flat the same way);
* ``input_ids`` is that flat token sequence;
* ``labels`` are pre-shifted next-token targets: token t predicts token t + 1, and the
  last token of every completion is masked;
* ``position_ids`` restart per completion: a completion continues the prompt's
  positions, as if it followed the prompt alone.

Readings taken where the pages are open (each is the plainest one the rest supports):

* F1 - "token t predicts t + 1" is read on the flat sequence of the group: the label
  of a token is the next flat token of the same group, except at the last token of a
  completion (masked, as stated).  So the last prompt token is labelled with the first
  token of the group's first non-empty completion; when the group has no completion
  token it is masked.  (Only one completion's first token can be predicted from the
  shared prompt position.)
* F2 - masked labels carry a caller-chosen ignore value; pad positions (past the
  folded length, up to the padded length) carry the pad token id, the ignore label,
  position 0, and the pad metadata of the attention layout (group = suffix = -1,
  is_prefix = 0).
* F3 - the attention metadata of a folded group is the one the unsloth page's
  ``build_seg_info_multigroup`` builds: prompt tokens are prefix tokens of their
  group (suffix id -1); completion j overall (counted over all groups, in order) has
  suffix id j.
* F4 - unfold: sample (g, i) is the sequence ``[prompt_g | c_gi]``; the rows of a
  folded per-token tensor are gathered into that layout, samples in completion order,
  one after another.  A group without completions contributes no sample.

Plain Python over lists; sizes are the tests' (up to a few hundred thousand tokens).
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def fold(prompts: Sequence[Sequence[int]], completions: Sequence[Sequence[Sequence[int]]],
         T: int, pad_id: int = 0, ignore: int = -100):
    """Fold groups (prompts[g], completions[g] = list of token lists) into length T.

    Returns a dict of int32 arrays ``input_ids, labels, position_ids, group, suffix``
    and uint8 ``is_prefix``, each of length T, plus ``T_real`` (the folded length).
    """
    ids: List[int] = []
    labels: List[int] = []
    pos: List[int] = []
    group: List[int] = []
    suffix: List[int] = []
    is_prefix: List[int] = []
    sid = 0
    for g, (prompt, comps) in enumerate(zip(prompts, completions)):
        flat = list(prompt)
        last_of_completion = set()  # flat offsets (within the group) that are masked
        for c in comps:
            flat += list(c)
            if len(c):
                last_of_completion.add(len(flat) - 1)
        for t, tok in enumerate(flat):
            ids.append(int(tok))
            nxt_in_group = t + 1 < len(flat)
            if nxt_in_group and t not in last_of_completion:
                labels.append(int(flat[t + 1]))
            else:
                labels.append(ignore)
        pos += list(range(len(prompt)))
        group += [g] * len(prompt)
        suffix += [-1] * len(prompt)
        is_prefix += [1] * len(prompt)
        for c in comps:
            pos += [len(prompt) + j for j in range(len(c))]
            group += [g] * len(c)
            suffix += [sid] * len(c)
            is_prefix += [0] * len(c)
            sid += 1
    t_real = len(ids)
    if T < t_real:
        raise ValueError(f"T = {T} is shorter than the folded length {t_real}")
    n_pad = T - t_real
    ids += [pad_id] * n_pad
    labels += [ignore] * n_pad
    pos += [0] * n_pad
    group += [-1] * n_pad
    suffix += [-1] * n_pad
    is_prefix += [0] * n_pad
    i32 = lambda x: np.asarray(x, dtype=np.int32)  # noqa: E731
    return {"input_ids": i32(ids), "labels": i32(labels), "position_ids": i32(pos),
            "group": i32(group), "suffix": i32(suffix),
            "is_prefix": np.asarray(is_prefix, dtype=np.uint8), "T_real": t_real}


def sample_rows(prompt_lens: Sequence[int], comp_lens: Sequence[Sequence[int]]
                ) -> List[Tuple[int, int, int]]:
    """For every sample (g, i) in order: (flat start of prompt_g, P_g, flat start of c_gi)."""
    out = []
    start = 0
    for p, rs in zip(prompt_lens, comp_lens):
        c_start = start + p
        for r in rs:
            out.append((start, p, c_start))
            c_start += r
        start = c_start
    return out


def unfold(folded: np.ndarray, prompt_lens: Sequence[int],
           comp_lens: Sequence[Sequence[int]]) -> np.ndarray:
    """Rows of ``folded`` ([T, ...]) gathered into the per-sample layout (reading F4)."""
    pieces = []
    flat_r = [r for rs in comp_lens for r in rs]
    for (p_start, p, c_start), r in zip(sample_rows(prompt_lens, comp_lens), flat_r):
        pieces.append(folded[p_start:p_start + p])
        pieces.append(folded[c_start:c_start + r])
    if not pieces:
        return folded[:0].copy()
    return np.concatenate(pieces, axis=0)
