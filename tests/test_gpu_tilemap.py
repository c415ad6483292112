"""GPU tile-map builder vs the oracle: bit-exact kinds, CSR and CSC."""
import os

import numpy as np
import pytest
import torch

from oracle import tilemap as ot
from oracle.mask import TokenMeta, dense_mask, meta_from_layout
from shared_prefix_block_amd import psa
from shared_prefix_block_amd import workloads as wl
from tests.gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _gpu_map(lay, bm, bn):
    return psa.layout_tile_map(lay, "cuda", block_m=bm, block_n=bn)


def _assert_same_map(got, want, info):
    np.testing.assert_array_equal(got["kinds"], want["kinds"])
    np.testing.assert_array_equal(got["row_ptr"], want["row_ptr"])
    np.testing.assert_array_equal(got["col"], want["col"])
    np.testing.assert_array_equal(got["kind"], want["kind"])
    np.testing.assert_array_equal(got["col_ptr"], want["col_ptr"])
    np.testing.assert_array_equal(got["row"], want["row"])
    np.testing.assert_array_equal(got["kind_csc"], want["kind_csc"])
    assert info["n_full"] == want["n_full"] and info["n_partial"] == want["n_partial"]
    assert info["nnz"] == len(want["col"])


SHAPES = [(128, 128), (128, 64), (64, 64), (3, 5), (7, 2), (1, 1), (16, 16), (64, 128)]


@pytest.mark.parametrize("seed", range(40))
def test_tilemap_fuzz_bit_exact(seed):
    rng = np.random.default_rng(9000 + seed)
    if seed % 3 == 2:
        nl, paths = wl.random_tree(rng, max_nodes=8, max_len=60)
        lay = wl.tree_layout(nl, paths, extra_pad=int(rng.integers(0, 40)))
    else:
        specs = wl.random_group_specs(rng, max_groups=4, max_p=70, max_g=5, max_r=70)
        lay = wl.tokens_layout(specs, pad_multiple=int(rng.integers(1, 130)))
    bm, bn = SHAPES[seed % len(SHAPES)]
    say(f"tilemap fuzz seed={seed} kind={lay.kind} T={lay.T} tile={bm}x{bn}")
    m = _gpu_map(lay, bm, bn)
    got = m.export()
    meta = meta_from_layout(lay)
    _assert_same_map(got, ot.tile_map(meta, bm, bn), m.info)
    # the per-token interval ends reproduce the oracle's mask exactly
    if lay.T:
        q = np.arange(lay.T)[:, None]
        kv = np.arange(lay.T)[None, :]
        from_end = (kv <= q) & (q < got["end"][None, :])
        np.testing.assert_array_equal(from_end, dense_mask(meta))


@pytest.mark.parametrize("idx", [1, 2, 5])
@pytest.mark.parametrize("bm,bn", [(128, 128), (128, 64), (64, 64)])
def test_tilemap_workloads(idx, bm, bn):
    lay = wl.layout_for(wl.WORKLOADS[idx])
    say(f"tilemap workload {idx} T={lay.T} tile={bm}x{bn}")
    m = _gpu_map(lay, bm, bn)
    _assert_same_map(m.export(), ot.tile_map(meta_from_layout(lay), bm, bn), m.info)


@pytest.mark.parametrize("idx", [3, 4])
def test_tilemap_large_workloads_golden(idx):
    g = np.load(os.path.join(GOLDEN, f"tilemap_cfg{idx}_128x128.npz"))
    lay = wl.layout_for(wl.WORKLOADS[idx])
    assert int(g["T"]) == lay.T
    kinds = g["kinds"]
    want = {"kinds": kinds, "n_full": int((kinds == 2).sum()),
            "n_partial": int((kinds == 1).sum())}
    want["row_ptr"], want["col"], want["kind"] = ot.csr(kinds)
    want["col_ptr"], want["row"], want["kind_csc"] = ot.csc(kinds)
    say(f"tilemap workload {idx} T={lay.T} (golden)")
    m = _gpu_map(lay, 128, 128)
    _assert_same_map(m.export(), want, m.info)


def test_tilemap_deterministic():
    lay = wl.layout_for(wl.WORKLOADS[3])
    a = _gpu_map(lay, 128, 128).export()
    b = _gpu_map(lay, 128, 128).export()
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("specs,pad", [
    ([], 0), ([], 5), ([(1, [])], 0), ([(0, [1])], 0), ([(0, [])], 3), ([(5, [0, 0])], 0),
    ([(0, [0, 3]), (0, []), (2, [0])], 7),
])
def test_tilemap_degenerate(specs, pad):
    lay = wl.tokens_layout(specs, extra_pad=pad)
    say(f"tilemap degenerate T={lay.T}")
    m = _gpu_map(lay, 128, 128)
    got = m.export()
    assert m.info["T"] == lay.T
    _assert_same_map(got, ot.tile_map(meta_from_layout(lay), 128, 128), m.info)


def _labels(group, suffix, is_prefix):
    dev = "cuda"
    return (torch.tensor(group, dtype=torch.int32, device=dev),
            torch.tensor(suffix, dtype=torch.int32, device=dev),
            torch.tensor(is_prefix, dtype=torch.uint8, device=dev))


@pytest.mark.parametrize("group,suffix,is_prefix", [
    ([1, 1, 0, 0], [-1, -1, -1, -1], [1, 1, 1, 1]),            # group ids decrease
    ([0, 0, -1, 0], [-1, 3, -1, 3], [1, 0, 0, 0]),             # a group split by a pad
    ([0, 0, 0, 0], [-1, 4, -1, 4], [1, 0, 1, 0]),              # prompt after completion
    ([0, 0, 0, 0, 0], [-1, 2, 1, 2, 2], [1, 0, 0, 0, 0]),      # completion ids decrease
    ([0, 0, 0, 0, 0], [-1, 2, 3, 2, 2], [1, 0, 0, 0, 0]),      # a completion split
])
def test_unpacked_token_layouts_take_node_form(group, suffix, is_prefix):
    """Labellings the interval form cannot hold get the node form, and the same mask
    as the oracle's rule token by token."""
    g, s, p = _labels(group, suffix, is_prefix)
    m = psa.build_tile_map_tokens(g, s, p, 2, 3)
    assert m.info["form"] == psa.FORM_NODES
    meta = TokenMeta(group, suffix, is_prefix)
    _assert_same_map(m.export(), ot.tile_map(meta, 2, 3), m.info)


def test_long_unpacked_layout_found_late():
    """A break of the packed layout far into a long sequence (past several scan chunks)
    is still found, and the node form takes over."""
    lay = wl.tokens_layout([(3000, [2000] * 4), (100, [50, 60])])
    s = lay.suffix.copy()
    s[-60:-30] = 10**6  # breaks the last completion into two runs with a smaller id after
    g, sf, p = _labels(lay.group, s, lay.is_prefix)
    m = psa.build_tile_map_tokens(g, sf, p, 128, 128)
    assert m.info["form"] == psa.FORM_NODES
    meta = TokenMeta(lay.group, s, lay.is_prefix)
    _assert_same_map(m.export(), ot.tile_map(meta, 128, 128), m.info)
