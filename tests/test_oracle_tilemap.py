"""Pins of the oracle's tile classification: brute-force enumeration and closed forms."""
import numpy as np
import pytest

from oracle import tilemap as ot
from oracle.mask import meta_from_layout
from shared_prefix_block_amd import workloads as wl
from tests import unfolded as uf


def _brute_counts(vis, T, bm, bn):
    """Pure-Python tile enumeration over a visibility matrix built from the unfolded view."""
    nq, nk = -(-T // bm), -(-T // bn)
    out = np.zeros((nq, nk), np.int64)
    for i in range(nq):
        for j in range(nk):
            c = 0
            for q in range(i * bm, min(T, (i + 1) * bm)):
                for kv in range(j * bn, min(T, (j + 1) * bn)):
                    c += bool(vis[q, kv])
            out[i, j] = c
    return out


SHAPES = [(4, 4), (8, 4), (4, 8), (3, 5), (7, 2), (1, 1), (16, 16)]


@pytest.mark.parametrize("seed", range(24))
def test_tile_counts_brute_force(seed):
    rng = np.random.default_rng(500 + seed)
    if seed % 3 == 2:
        nl, paths = wl.random_tree(rng, max_nodes=6, max_len=9)
        lay = wl.tree_layout(nl, paths, extra_pad=int(rng.integers(0, 5)))
        seqs = uf.tree_sequences(nl, paths)
    else:
        specs = wl.random_group_specs(rng, max_groups=3, max_p=10, max_g=3, max_r=10)
        lay = wl.tokens_layout(specs, pad_multiple=int(rng.integers(1, 9)))
        seqs, _ = uf.group_sequences(specs)
    if lay.T == 0:
        return
    vis = uf.visibility_from_sequences(lay.T, seqs)
    meta = meta_from_layout(lay)
    bm, bn = SHAPES[seed % len(SHAPES)]
    counts = ot.tile_counts(meta, bm, bn)
    np.testing.assert_array_equal(counts, _brute_counts(vis, lay.T, bm, bn))
    kinds = ot.tile_kinds(counts, bm, bn)
    T = lay.T
    for i, j in zip(*np.nonzero(kinds == 2)):
        assert (i + 1) * bm <= T and (j + 1) * bn <= T
        assert vis[i * bm:(i + 1) * bm, j * bn:(j + 1) * bn].all()
    for i, j in zip(*np.nonzero(kinds == 0)):
        assert not vis[i * bm:(i + 1) * bm, j * bn:(j + 1) * bn].any()


def _check_sparse(m):
    kinds = m["kinds"]
    nq, nk = kinds.shape
    rebuilt = np.zeros_like(kinds)
    for i in range(nq):
        cols = m["col"][m["row_ptr"][i]:m["row_ptr"][i + 1]]
        assert np.all(np.diff(cols) > 0)
        rebuilt[i, cols] = m["kind"][m["row_ptr"][i]:m["row_ptr"][i + 1]]
    np.testing.assert_array_equal(rebuilt, kinds)
    rebuilt[:] = 0
    for j in range(nk):
        rows = m["row"][m["col_ptr"][j]:m["col_ptr"][j + 1]]
        assert np.all(np.diff(rows) > 0)
        rebuilt[rows, j] = m["kind_csc"][m["col_ptr"][j]:m["col_ptr"][j + 1]]
    np.testing.assert_array_equal(rebuilt, kinds)


@pytest.mark.parametrize("idx", [1, 2, 5])
@pytest.mark.parametrize("bm,bn", [(128, 128), (128, 64), (64, 64)])
def test_workload_tile_maps_sum_to_closed_form(idx, bm, bn):
    cfg = wl.WORKLOADS[idx]
    lay = wl.layout_for(cfg)
    m = ot.tile_map(meta_from_layout(lay), bm, bn)
    if lay.kind == "tokens":
        closed = uf.kept_closed_form_groups(lay.specs)
    else:
        closed = uf.kept_closed_form_tree(lay.node_lengths, lay.sample_paths)
    assert int(m["counts"].sum()) == closed
    _check_sparse(m)


def test_workload_tile_kind_totals_128():
    """Full / partial / empty tile totals at 128 x 128 for workloads 1, 2 and 5."""
    want = {1: (0, 3, 1), 2: (624, 160, 24_816), 5: (4_992, 512, 256_640)}
    for idx, (full, part, empty) in want.items():
        lay = wl.layout_for(wl.WORKLOADS[idx])
        m = ot.tile_map(meta_from_layout(lay), 128, 128)
        k = m["kinds"]
        assert (int((k == 2).sum()), int((k == 1).sum()), int((k == 0).sum())) == \
            (full, part, empty), idx
