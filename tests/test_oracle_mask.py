"""Pins of the oracle's mask rule: brute force from the unfolded meaning, closed forms."""
import itertools

import numpy as np
import pytest

from oracle.mask import TokenMeta, TreeMeta, dense_mask, kept_pairs, meta_from_layout
from shared_prefix_block_amd import workloads as wl
from tests import unfolded as uf


def _tiny_group_specs():
    """Every single group with P in 0..4, G in 0..3, R_i in 0..4."""
    for p in range(5):
        for g in range(4):
            for rs in itertools.product(range(5), repeat=g):
                yield [(p, list(rs))]


def test_single_group_exhaustive_matches_unfolded():
    n = 0
    for specs in _tiny_group_specs():
        lay = wl.tokens_layout(specs)
        if lay.T == 0:
            continue
        meta = meta_from_layout(lay)
        seqs, _ = uf.group_sequences(specs)
        want = uf.visibility_from_sequences(lay.T, seqs)
        np.testing.assert_array_equal(dense_mask(meta), want, err_msg=str(specs))
        n += 1
    assert n > 700


@pytest.mark.parametrize("seed", range(60))
def test_multi_group_with_pads_matches_unfolded(seed):
    rng = np.random.default_rng(seed)
    specs = wl.random_group_specs(rng, max_groups=3, max_p=5, max_g=3, max_r=5)
    lay = wl.tokens_layout(specs, pad_multiple=int(rng.integers(1, 9)),
                           extra_pad=int(rng.integers(0, 3)))
    if lay.T == 0:
        return
    seqs, _ = uf.group_sequences(specs)
    want = uf.visibility_from_sequences(lay.T, seqs)
    np.testing.assert_array_equal(dense_mask(meta_from_layout(lay)), want)


@pytest.mark.parametrize("seed", range(60))
def test_random_trees_match_unfolded(seed):
    rng = np.random.default_rng(1000 + seed)
    nl, paths = wl.random_tree(rng, max_nodes=6, max_len=5, max_trees=2)
    extra = int(rng.integers(0, 4))
    lay = wl.tree_layout(nl, paths, extra_pad=extra)
    if lay.T == 0:
        return
    want = uf.visibility_from_sequences(lay.T, uf.tree_sequences(nl, paths))
    np.testing.assert_array_equal(dense_mask(meta_from_layout(lay)), want)


@pytest.mark.parametrize("seed", range(20))
def test_depth_two_tree_equals_token_form(seed):
    rng = np.random.default_rng(2000 + seed)
    specs = wl.random_group_specs(rng, max_groups=3, max_p=6, max_g=4, max_r=6)
    nl, paths = [], []
    for p, rs in specs:
        root = len(nl)
        nl.append(p)
        if not rs:
            paths.append([root])
        for r in rs:
            paths.append([root, len(nl)])
            nl.append(r)
    tok = wl.tokens_layout(specs)
    tree = wl.tree_layout(nl, paths)
    assert tok.T == tree.T
    if tok.T == 0:
        return
    np.testing.assert_array_equal(dense_mask(meta_from_layout(tok)),
                                  dense_mask(meta_from_layout(tree)))


def test_documented_rule_differs_only_on_prefix_rows():
    """Reading A1: the docstring form (no causal guard on the prefix branch) and the
    implemented form agree on every suffix row and differ only where a prefix row
    would see a later prefix token."""
    specs = [(4, [3, 2]), (3, [2])]
    lay = wl.tokens_layout(specs)
    g = lay.group.astype(np.int64)
    s = lay.suffix.astype(np.int64)
    p = lay.is_prefix.astype(bool)
    q = np.arange(lay.T)[:, None]
    kv = np.arange(lay.T)[None, :]
    documented = (g[q] == g[kv]) & (p[kv] | ((s[kv] == s[q]) & (kv <= q)))
    ours = dense_mask(meta_from_layout(lay))
    diff = documented != ours
    rows, cols = np.nonzero(diff)
    assert len(rows) > 0
    assert np.all(p[rows]) and np.all(p[cols]) and np.all(cols > rows)
    assert not diff[~p].any()


def test_pads_see_nothing_and_are_unseen():
    lay = wl.tokens_layout([(3, [2, 2])], pad_multiple=8)
    m = dense_mask(meta_from_layout(lay))
    pad = lay.group < 0
    assert pad.sum() == 1
    assert not m[pad].any() and not m[:, pad].any()


def test_tree_validation():
    with pytest.raises(ValueError):
        TreeMeta([2, 2, 2], [[0, 1], [2, 1]])  # node 1 with two parents
    with pytest.raises(ValueError):
        TreeMeta([2, 2, 2], [[0, 1]])  # node 2 on no path
    with pytest.raises(ValueError):
        TreeMeta([2, 2], [[0, 5]])


# ----------------------------------------------------------------------------
# kept-pair counts: element-wise mask vs closed forms (and the exact integers)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(30))
def test_kept_count_closed_form_random(seed):
    rng = np.random.default_rng(3000 + seed)
    specs = wl.random_group_specs(rng, max_groups=4, max_p=30, max_g=5, max_r=30)
    lay = wl.tokens_layout(specs, pad_multiple=16)
    assert kept_pairs(meta_from_layout(lay)) == uf.kept_closed_form_groups(specs)
    nl, paths = wl.random_tree(rng, max_nodes=8, max_len=30)
    tl = wl.tree_layout(nl, paths, extra_pad=5)
    assert kept_pairs(meta_from_layout(tl)) == uf.kept_closed_form_tree(nl, paths)


@pytest.mark.parametrize("idx,expected", [(1, 12_384), (2, 11_544_576), (5, 86_016_000)])
def test_kept_count_workloads(idx, expected):
    cfg = wl.WORKLOADS[idx]
    lay = wl.layout_for(cfg)
    meta = meta_from_layout(lay)
    if lay.kind == "tokens":
        closed = uf.kept_closed_form_groups(lay.specs)
    else:
        closed = uf.kept_closed_form_tree(lay.node_lengths, lay.sample_paths)
    assert closed == expected
    assert kept_pairs(meta) == expected


@pytest.mark.slow
@pytest.mark.parametrize("idx", [3, 4])
def test_kept_count_large_workloads(idx):
    cfg = wl.WORKLOADS[idx]
    lay = wl.layout_for(cfg)
    closed = uf.kept_closed_form_groups(lay.specs)
    if idx == 4:
        assert closed == 1_359_003_648
    assert kept_pairs(meta_from_layout(lay), block_rows=2048) == closed


# ---------------------------------------------------------------------------
# layouts that are not packed: interleaved runs, ids out of order, other node orders
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(40))
def test_interleaved_prompt_first_matches_unfolded(seed):
    """Runs merged token by token (each prompt before its group's completions, ids
    relabelled, pads anywhere): still plain causal attention over every unfolded
    sample, whose tokens keep their flat order."""
    rng = np.random.default_rng(3000 + seed)
    specs = wl.random_group_specs(rng, max_groups=3, max_p=5, max_g=3, max_r=5)
    lay = wl.shuffled_tokens_layout(specs, rng, prompt_first=True,
                                    n_pad=int(rng.integers(0, 4)))
    if lay.T == 0:
        return
    seqs, _ = uf.group_sequences(specs)
    pos = lay.extra["pos"]
    want = uf.visibility_from_sequences(lay.T, [pos[s] for s in seqs])
    np.testing.assert_array_equal(dense_mask(meta_from_layout(lay)), want)


@pytest.mark.parametrize("seed", range(40))
def test_interleaved_any_order_is_tree_rule_and_flat_causality(seed):
    """Prompt tokens may follow completion tokens.  The token rule is then the tree
    rule of the same groups (a prompt node with one child per completion, pinned
    against the unfolded samples above) restricted to kv <= q in the new order: a
    prompt token placed after a completion token stays hidden from it."""
    rng = np.random.default_rng(3100 + seed)
    specs = wl.random_group_specs(rng, max_groups=3, max_p=5, max_g=3, max_r=5)
    lay = wl.shuffled_tokens_layout(specs, rng, prompt_first=False,
                                    n_pad=int(rng.integers(0, 4)))
    if lay.T == 0:
        return
    nl, paths = [], []
    for p, rs in specs:
        root = len(nl)
        nl.append(p)
        if not rs:
            paths.append([root])
        for r in rs:
            paths.append([root, len(nl)])
            nl.append(r)
    packed = dense_mask(meta_from_layout(wl.tree_layout(nl, paths)))
    pos = lay.extra["pos"]
    want = np.zeros((lay.T, lay.T), dtype=bool)
    want[np.ix_(pos, pos)] = packed
    want &= np.tril(np.ones((lay.T, lay.T), dtype=bool))
    np.testing.assert_array_equal(dense_mask(meta_from_layout(lay)), want)


def test_interleaving_hides_later_prompt_tokens():
    """Worked case: prompt [a b], completion [c d] laid out a c b d.  c sees a and
    itself but not b (placed after it); d sees a, b, c and itself; b sees a, b."""
    g = [0, 0, 0, 0]
    s = [-1, 5, -1, 5]
    p = [1, 0, 1, 0]
    m = dense_mask(TokenMeta(g, s, p))
    want = np.array([[1, 0, 0, 0],
                     [1, 1, 0, 0],
                     [1, 0, 1, 0],
                     [1, 1, 1, 1]], dtype=bool)
    np.testing.assert_array_equal(m, want)


@pytest.mark.parametrize("seed", range(40))
def test_reordered_trees_match_unfolded(seed):
    """Breadth-first and random parent-first node orders (subtrees no longer
    contiguous): visibility is still causal attention over each root-to-leaf path,
    and the kept count keeps its closed form."""
    rng = np.random.default_rng(3200 + seed)
    nl, paths = wl.random_tree(rng, max_nodes=7, max_len=5, max_trees=2)
    nl, paths = wl.reorder_tree(nl, paths, None if seed % 2 else rng)
    lay = wl.tree_layout(nl, paths, extra_pad=int(rng.integers(0, 3)))
    if lay.T == 0:
        return
    meta = meta_from_layout(lay)
    want = uf.visibility_from_sequences(lay.T, uf.tree_sequences(nl, paths))
    np.testing.assert_array_equal(dense_mask(meta), want)
    assert kept_pairs(meta) == uf.kept_closed_form_tree(nl, paths)
