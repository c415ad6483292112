"""Pins of the fold / unfold oracle (CPU).

The fold stores a group's prompt once; every pin below ties its outputs to the
unfolded samples [prompt | c_i] it deduplicates, which are defined without the fold:
the tokens must come back by unfolding, the labels must be the ordinary next-token
labels of each unfolded sample wherever the folded layout can hold them, the
positions must be each token's index in its unfolded sample, and the attention
metadata must make a token see exactly what precedes it in its own unfolded sample.
"""
import numpy as np
import pytest

from oracle import fold as of
from oracle.mask import TokenMeta, dense_mask

IGN = -100


def _rollouts(rng, max_groups=3, max_p=6, max_g=4, max_r=6):
    prompts, comps = [], []
    tok = 1
    for _ in range(int(rng.integers(1, max_groups + 1))):
        p = int(rng.integers(0, max_p + 1))
        prompts.append(list(range(tok, tok + p)))
        tok += p
        cs = []
        for _ in range(int(rng.integers(0, max_g + 1))):
            r = int(rng.integers(0, max_r + 1))
            cs.append(list(range(tok, tok + r)))
            tok += r
        comps.append(cs)
    return prompts, comps


def _samples(prompts, comps):
    return [(g, i, list(p) + list(c)) for g, (p, cs) in enumerate(zip(prompts, comps))
            for i, c in enumerate(cs)]


CASES = [np.random.default_rng(s) for s in range(60)]


@pytest.mark.parametrize("rng", CASES)
def test_unfold_gives_back_every_sample(rng):
    prompts, comps = _rollouts(rng)
    f = of.fold(prompts, comps, T=sum(len(p) + sum(len(c) for c in cs)
                                      for p, cs in zip(prompts, comps)) + 3)
    pl = [len(p) for p in prompts]
    cl = [[len(c) for c in cs] for cs in comps]
    got = of.unfold(f["input_ids"], pl, cl)
    want = [t for _, _, s in _samples(prompts, comps) for t in s]
    assert got.tolist() == want


@pytest.mark.parametrize("rng", CASES)
def test_labels_are_the_unfolded_next_token_labels(rng):
    """At every folded position the label equals the next token of the unfolded sample
    the position belongs to, wherever that next token is the same for all samples
    sharing the position; completion ends are masked; the last prompt position holds
    the next token of the group's first sample with a non-empty completion."""
    prompts, comps = _rollouts(rng)
    f = of.fold(prompts, comps, T=sum(len(p) + sum(len(c) for c in cs)
                                      for p, cs in zip(prompts, comps)))
    start = 0
    for p, cs in zip(prompts, comps):
        P = len(p)
        for t in range(P - 1):  # every sample of the group has prompt[t+1] next
            assert f["labels"][start + t] == p[t + 1]
        if P:
            firsts = [c[0] for c in cs if len(c)]
            want = firsts[0] if firsts else IGN
            assert f["labels"][start + P - 1] == want
        off = start + P
        for c in cs:
            unf = list(p) + list(c)
            for j in range(len(c)):  # token j of c sits at unfolded index P + j
                nxt = unf[P + j + 1] if P + j + 1 < len(unf) else IGN
                assert f["labels"][off + j] == nxt
            off += len(c)
        start = off
    assert (f["labels"][f["T_real"]:] == IGN).all()


@pytest.mark.parametrize("rng", CASES)
def test_positions_are_indices_in_the_unfolded_sample(rng):
    prompts, comps = _rollouts(rng)
    f = of.fold(prompts, comps, T=sum(len(p) + sum(len(c) for c in cs)
                                      for p, cs in zip(prompts, comps)) + 5)
    pl = [len(p) for p in prompts]
    cl = [[len(c) for c in cs] for cs in comps]
    got = of.unfold(f["position_ids"], pl, cl).tolist()
    want = [j for _, _, s in _samples(prompts, comps) for j in range(len(s))]
    assert got == want
    assert (f["position_ids"][f["T_real"]:] == 0).all()


@pytest.mark.parametrize("rng", CASES[:30])
def test_metadata_gives_unfolded_visibility(rng):
    """With the fold's group / suffix / is_prefix, the attention rule lets a folded
    token see exactly the tokens that precede or equal it in its own unfolded sample
    (a prompt token: its prompt up to itself)."""
    prompts, comps = _rollouts(rng)
    T_real = sum(len(p) + sum(len(c) for c in cs) for p, cs in zip(prompts, comps))
    f = of.fold(prompts, comps, T=T_real + 2)
    M = dense_mask(TokenMeta(f["group"], f["suffix"], f["is_prefix"]))
    want = np.zeros_like(M)
    start = 0
    for p, cs in zip(prompts, comps):
        P = len(p)
        for t in range(P):
            want[start + t, start:start + t + 1] = True
        off = start + P
        for c in cs:
            for j in range(len(c)):
                want[off + j, start:start + P] = True
                want[off + j, off:off + j + 1] = True
            off += len(c)
        start = off
    assert (M == want).all()


def test_counts_of_unmasked_labels():
    """Closed form: a group keeps P - 1 prompt labels, one more on its last prompt
    token if any completion is non-empty (and P > 0), and R - 1 labels per non-empty
    completion."""
    rng = np.random.default_rng(123)
    for _ in range(40):
        prompts, comps = _rollouts(rng, max_groups=4, max_p=9, max_g=5, max_r=9)
        f = of.fold(prompts, comps, T=sum(len(p) + sum(len(c) for c in cs)
                                          for p, cs in zip(prompts, comps)))
        want = 0
        for p, cs in zip(prompts, comps):
            if len(p):
                want += len(p) - 1 + (1 if any(len(c) for c in cs) else 0)
            want += sum(len(c) - 1 for c in cs if len(c))
        assert int((f["labels"] != IGN).sum()) == want


def test_pads_and_errors():
    f = of.fold([[5, 6]], [[[7], []]], T=6, pad_id=9, ignore=-1)
    assert f["T_real"] == 3
    assert f["input_ids"].tolist() == [5, 6, 7, 9, 9, 9]
    assert f["labels"].tolist() == [6, 7, -1, -1, -1, -1]
    assert f["position_ids"].tolist() == [0, 1, 2, 0, 0, 0]
    assert f["group"].tolist() == [0, 0, 0, -1, -1, -1]
    assert f["suffix"].tolist() == [-1, -1, 0, -1, -1, -1]
    assert f["is_prefix"].tolist() == [1, 1, 0, 0, 0, 0]
    with pytest.raises(ValueError):
        of.fold([[1, 2, 3]], [[[4]]], T=3)
    # an empty completion still takes a suffix id; an empty prompt has no prompt label
    f = of.fold([[]], [[[1, 2], [], [3]]], T=3)
    assert f["suffix"].tolist() == [0, 0, 2]
    assert f["labels"].tolist() == [2, IGN, IGN]
    assert of.unfold(np.arange(3), [0], [[2, 0, 1]]).tolist() == [0, 1, 2]
