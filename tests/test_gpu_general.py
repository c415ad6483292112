"""Layouts that are not packed (the map's node form): GPU vs the oracle.

Token labellings with interleaved runs, ids out of order and prompt tokens after
completion tokens, and prefix trees whose nodes are not in depth-first order, go
through the node form of the tile map (psa.FORM_NODES).  The tile map must match the
oracle bit for bit, the exported node encoding must reproduce the oracle's mask, and
the attention must meet the parity bar.  On packed layouts the node form, forced,
must give the interval form's map and bit-identical outputs.
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import tilemap as ot
from oracle.mask import dense_mask, meta_from_layout
from shared_prefix_block_amd import psa
from shared_prefix_block_amd import workloads as wl
from tests.gpu_common import compare, need_gpu, say
from tests.test_gpu_attention import CASES, DT, _sample
from tests.test_gpu_tilemap import SHAPES, _assert_same_map

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _general_layout(rng, which, max_len=70):
    if which == "tree":
        nl, paths = wl.random_tree(rng, max_nodes=9, max_len=max_len)
        nl, paths = wl.reorder_tree(nl, paths, rng if rng.random() < 0.5 else None)
        return wl.tree_layout(nl, paths, extra_pad=int(rng.integers(0, 40)))
    specs = wl.random_group_specs(rng, max_groups=4, max_p=max_len, max_g=5, max_r=max_len)
    return wl.shuffled_tokens_layout(specs, rng, prompt_first=(which == "prompt_first"),
                                     n_pad=int(rng.integers(0, 40)),
                                     chunk=int(rng.choice([1, 3, 16, 64])))


KINDS = ["prompt_first", "any_order", "tree"]


@pytest.mark.parametrize("seed", range(36))
def test_tilemap_general_bit_exact(seed):
    rng = np.random.default_rng(5000 + seed)
    lay = _general_layout(rng, KINDS[seed % 3])
    bm, bn = SHAPES[seed % len(SHAPES)]
    say(f"general tilemap seed={seed} {KINDS[seed % 3]} T={lay.T} tile={bm}x{bn}")
    m = psa.layout_tile_map(lay, "cuda", block_m=bm, block_n=bn)
    got = m.export()
    meta = meta_from_layout(lay)
    _assert_same_map(got, ot.tile_map(meta, bm, bn), m.info)
    if lay.T:
        q = np.arange(lay.T)[:, None]
        kv = np.arange(lay.T)[None, :]
        key, lo, w = got["key"], got["lo"], got["w"]
        from_nodes = (kv <= q) & (lo[None, :] <= key[:, None]) & (key[:, None] < (lo + w)[None, :])
        np.testing.assert_array_equal(from_nodes, dense_mask(meta))


def test_node_form_is_chosen_and_numbered():
    """A prompt token after a completion token of its group: the node form, with the
    prompt numbered before its completions and its range covering them."""
    g = torch.tensor([7, 7, 7, 7, -1, 3], dtype=torch.int32, device="cuda")
    s = torch.tensor([-1, 2, -1, 2, -1, 0], dtype=torch.int32, device="cuda")
    p = torch.tensor([1, 0, 1, 0, 0, 1], dtype=torch.uint8, device="cuda")
    m = psa.build_tile_map_tokens(g, s, p, 128, 128)
    assert m.info["form"] == psa.FORM_NODES
    e = m.export_nodes()
    # nodes in (group id, prompt first, completion ids) order: (3, prompt) = 1,
    # (7, prompt) = 2, (7, completion 2) = 3
    assert e["key"].tolist() == [2, 3, 2, 3, 0, 1]
    assert e["lo"].tolist() == [2, 3, 2, 3, 0, 1]
    assert e["w"].tolist() == [2, 1, 2, 1, 0, 1]
    end = np.zeros(6, np.int32)  # a node-form map has no end[] to export
    st = psa.load().psa_tile_map_export(m.handle, ctypes.c_void_p(end.ctypes.data),
                                        *([ctypes.c_void_p(0)] * 7))
    assert psa.STATUS[st] == "PSA_ERR_VALUE"


def test_tree_non_dfs_gets_node_form():
    nl, paths = [4, 4, 4, 4], [[0, 2], [0, 1, 3]]  # 3 is a child of 1 but follows 2
    m = psa.build_tile_map_tree(nl, paths, device="cuda", block_m=128, block_n=128)
    assert m.info["form"] == psa.FORM_NODES
    m2 = psa.build_tile_map_tree([4, 4, 4], [[0, 1], [0, 2]], device="cuda", block_m=128,
                                 block_n=128)
    assert m2.info["form"] == psa.FORM_INTERVAL


def _outputs(lay, m, hq, hkv, d, dtype, seed):
    q, k, v, do = (x.cuda() for x in wl.make_tensors(lay.T, hq, hkv, d, dtype, 1.0, seed))
    o, lse = psa.fwd(m, q, k, v)
    dq, dk, dv = psa.bwd(m, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("case", range(len(CASES)))
def test_forced_node_form_matches_interval_form(case):
    """Packed layouts through the node form: the same map, bit-identical outputs."""
    hq, hkv, d, dtype = CASES[case]
    rng = np.random.default_rng(5100 + case)
    if case % 2:
        nl, paths = wl.random_tree(rng, max_nodes=8, max_len=120)
        lay = wl.tree_layout(nl, paths, extra_pad=int(rng.integers(0, 60)))
    else:
        specs = wl.random_group_specs(rng, max_groups=4, max_p=160, max_g=5, max_r=160)
        lay = wl.tokens_layout(specs, pad_multiple=int(rng.integers(1, 130)))
    if lay.T == 0:
        return
    say(f"forced node form case={case} {lay.kind} T={lay.T} d={d} {dtype}")
    tdt = DT[dtype]
    mi = psa.layout_tile_map(lay, "cuda", dtype=tdt, d=d)
    mn = psa.layout_tile_map(lay, "cuda", dtype=tdt, d=d, form="nodes")
    assert mi.info["form"] == psa.FORM_INTERVAL and mn.info["form"] == psa.FORM_NODES
    a, b = mi.export(), mn.export()
    for key in ("kinds", "row_ptr", "col", "kind", "col_ptr", "row", "kind_csc"):
        np.testing.assert_array_equal(a[key], b[key])
    for x, y in zip(_outputs(lay, mi, hq, hkv, d, dtype, case),
                    _outputs(lay, mn, hq, hkv, d, dtype, case)):
        assert torch.equal(x, y)


@pytest.mark.parametrize("seed", range(24))
def test_attention_general_fuzz(seed):
    """Node runs up to 130 tokens, every dtype."""
    hq, hkv, d, dtype = CASES[seed % len(CASES)]
    rng = np.random.default_rng(5200 + seed)
    lay = _general_layout(rng, KINDS[seed % 3], max_len=130)
    if lay.T == 0:
        return
    tdt = DT[dtype]
    say(f"general attention seed={seed} {KINDS[seed % 3]} T={lay.T} hq={hq} hkv={hkv} "
        f"d={d} {dtype}")
    q, k, v, do = wl.make_tensors(lay.T, hq, hkv, d, dtype, 1.0, seed)
    m = psa.layout_tile_map(lay, "cuda", dtype=tdt, d=d)
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    o, lse = psa.fwd(m, qd, kd, vd)
    dq, dk, dv = psa.bwd(m, qd, kd, vd, o, lse, dod)
    torch.cuda.synchronize()
    wo, wl_, wdq, wdk, wdv = oa.backward(meta_from_layout(lay), q, k, v, do)
    compare("o", o, wo, tdt)
    compare("lse", lse, wl_, tdt)
    compare("dq", dq, wdq, tdt)
    compare("dk", dk, wdk, tdt)
    compare("dv", dv, wdv, tdt)


@pytest.mark.parametrize("form", ["auto", "nodes"])
def test_fp32_long_accumulation_chain(form):
    """A 17-node tree of 1368 tokens (and pads) with fp32 inputs, d = 128: keys near
    its root collect dV from ~10^3 rows at magnitudes ~5.  With one fp32 accumulator
    chain over all of them the rounding of the running sum alone reached 1.1e-5 here
    (above the 1e-5 bar); the kernels now add each sub-step's products to the sums as
    a partial block.  The same tree as the fuzz case of seed 17."""
    rng = np.random.default_rng(5200 + 17)
    lay = _general_layout(rng, "tree", max_len=130)
    assert lay.T_real == 1368 and len(lay.node_lengths) == 17
    hq, hkv, d, dtype = 4, 2, 128, "fp32"
    say(f"fp32 long chain form={form} T={lay.T}")
    q, k, v, do = wl.make_tensors(lay.T, hq, hkv, d, dtype, 1.0, 17)
    m = psa.layout_tile_map(lay, "cuda", dtype=torch.float32, d=d, form=form)
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    o, lse = psa.fwd(m, qd, kd, vd)
    dq, dk, dv = psa.bwd(m, qd, kd, vd, o, lse, dod)
    torch.cuda.synchronize()
    wo, wl_, wdq, wdk, wdv = oa.backward(meta_from_layout(lay), q, k, v, do)
    for name, got, want in (("o", o, wo), ("lse", lse, wl_), ("dq", dq, wdq), ("dk", dk, wdk),
                            ("dv", dv, wdv)):
        err, _ = compare(name, got, want, torch.float32)
        say(f"  {name}: max-abs {err:.3e}")


@pytest.mark.parametrize("which", ["chunked", "tokens", "tree"])
def test_general_full_size_sampled(which):
    """Workload sizes in the node form: the 8-group batch (P=512, 8 x 256) with its
    completions generated side by side (runs of 64 tokens in turns, or token by
    token with prompt tokens anywhere), and the 8 trees in breadth-first node order."""
    rng = np.random.default_rng(77)
    if which == "tree":
        cfg = wl.WORKLOADS[5]
        nl, paths = wl.tree_spec()
        nl, paths = wl.reorder_tree(nl, paths)
        lay = wl.tree_layout(nl, paths)
    else:
        cfg = wl.WORKLOADS[2]
        specs = wl.group_specs(cfg)
        lay = wl.shuffled_tokens_layout(specs, rng, prompt_first=(which == "chunked"),
                                        chunk=64 if which == "chunked" else 1)
    tdt = DT[cfg.dtype]
    say(f"general full size {which}: T={lay.T} hq={cfg.hq} hkv={cfg.hkv} d={cfg.d}")
    q, k, v, do = wl.make_tensors(lay.T, cfg.hq, cfg.hkv, cfg.d, cfg.dtype, cfg.sigma, cfg.idx)
    m = psa.layout_tile_map(lay, "cuda", dtype=tdt, d=cfg.d)
    assert m.info["form"] == psa.FORM_NODES
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    o, lse = psa.fwd(m, qd, kd, vd)
    dq, dk, dv = psa.bwd(m, qd, kd, vd, o, lse, dod)
    torch.cuda.synchronize()
    meta = meta_from_layout(lay)
    rows = _sample(lay.T, 40, rng)
    wo, wl_, wdq = oa.grad_rows(meta, q, k, v, do, rows)
    compare("o", o[rows], wo, tdt)
    compare("lse", lse[:, rows], wl_, tdt)
    compare("dq", dq[rows], wdq, tdt)
    cols = _sample(lay.T, 24, rng)
    wdk, wdv = oa.grad_cols(meta, q, k, v, do, cols)
    compare("dk", dk[cols], wdk, tdt)
    compare("dv", dv[cols], wdv, tdt)
