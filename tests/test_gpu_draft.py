"""The packed-document draft mask on the GPU (node-form map, bidirectional or causal
blocks) vs the oracle: bit-exact maps, attention at the parity bar."""
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


def _random_draft(rng, max_doc=300, max_blocks=12):
    n_docs = int(rng.integers(1, 4))
    lens = [int(rng.integers(0, max_doc + 1)) for _ in range(n_docs)]
    bs = int(rng.choice([1, 2, 5, 16, 32]))
    per = [int(rng.integers(0, max_blocks + 1)) for _ in range(n_docs)]
    ids = [int(x) for x in rng.choice(1000, size=n_docs, replace=False) - 500]
    return wl.draft_layout(lens, bs, per, rng, causal=bool(rng.random() < 0.5),
                           keep_frac=float(rng.choice([1.0, 0.7])),
                           extra_pad=int(rng.integers(0, 70)), doc_ids=ids)


@pytest.mark.parametrize("seed", range(30))
def test_draft_tilemap_bit_exact(seed):
    rng = np.random.default_rng(7000 + seed)
    lay = _random_draft(rng)
    bm, bn = SHAPES[seed % len(SHAPES)]
    x = lay.extra
    say(f"draft tilemap seed={seed} T={lay.T} S={x['ctx_len']} bs={x['block_size']} "
        f"N={len(x['anchors'])} causal={x['causal']} tile={bm}x{bn}")
    m = psa.layout_tile_map(lay, "cuda", block_m=bm, block_n=bn)
    assert m.info["form"] == psa.FORM_NODES and m.info["causal"] == int(x["causal"])
    got = m.export()
    meta = meta_from_layout(lay)
    _assert_same_map(got, ot.tile_map(meta, bm, bn), m.info)
    if lay.T:
        q = np.arange(lay.T)[:, None]
        kv = np.arange(lay.T)[None, :]
        key, lo, w = got["key"], got["lo"], got["w"]
        order = (kv <= q) if x["causal"] else np.ones((lay.T, lay.T), bool)
        from_nodes = order & (lo[None, :] <= key[:, None]) & (key[:, None] < (lo + w)[None, :])
        np.testing.assert_array_equal(from_nodes, dense_mask(meta))


def test_draft_anchor_out_of_range():
    a = torch.tensor([3, 9, 2], dtype=torch.int32, device="cuda")
    with pytest.raises(psa.PsaError) as ei:
        psa.build_tile_map_draft(8, 4, a, block_m=128, block_n=128)
    assert ei.value.name == "PSA_ERR_LAYOUT" and "block 1" in str(ei.value)


@pytest.mark.parametrize("seed", range(16))
def test_draft_attention_fuzz(seed):
    rng = np.random.default_rng(7100 + seed)
    lay = _random_draft(rng, max_doc=400, max_blocks=10)
    if lay.T == 0:
        return
    hq, hkv, d, dtype = CASES[seed % len(CASES)]
    tdt = DT[dtype]
    x = lay.extra
    say(f"draft attention seed={seed} T={lay.T} S={x['ctx_len']} bs={x['block_size']} "
        f"causal={x['causal']} hq={hq} hkv={hkv} d={d} {dtype}")
    q, k, v, do = wl.make_tensors(lay.T, hq, hkv, d, dtype, 1.0, seed)
    m = psa.layout_tile_map(lay, "cuda", dtype=tdt, d=d)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = psa.fwd(m, qd, kd, vd)
    dq, dk, dv = psa.bwd(m, qd, kd, vd, o, lse, dod)
    torch.cuda.synchronize()
    wo, wl_, wdq, wdk, wdv = oa.backward(meta_from_layout(lay), q, k, v, do)
    compare("o", o, wo, tdt)
    compare("lse", lse, wl_, tdt)
    compare("dq", dq, wdq, tdt)
    compare("dk", dk, wdk, tdt)
    compare("dv", dv, wdv, tdt)


@pytest.mark.parametrize("causal", [False, True])
def test_draft_generation_block(causal):
    """One block anchored at the end of the context (the generation layout)."""
    S, bs = 300, 16
    a = torch.tensor([S], dtype=torch.int32, device="cuda")
    m = psa.build_tile_map_draft(S, bs, a, causal=causal, dtype=torch.bfloat16, d=128)
    from oracle.draft import DraftMeta
    meta = DraftMeta(S, bs, [S], causal=causal)
    q, k, v, do = wl.make_tensors(S + bs, 4, 2, 128, "bf16", 1.0, 3)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = psa.fwd(m, qd, kd, vd)
    dq, dk, dv = psa.bwd(m, qd, kd, vd, o, lse, dod)
    torch.cuda.synchronize()
    wo, wl_, wdq, wdk, wdv = oa.backward(meta, q, k, v, do)
    for name, g, w in (("o", o, wo), ("lse", lse, wl_), ("dq", dq, wdq), ("dk", dk, wdk),
                       ("dv", dv, wdv)):
        compare(name, g, w, torch.bfloat16)


def test_draft_workload_sampled():
    """The draft workload at full size (4 packed documents of 4096 context tokens, 512
    blocks of 16 each, bidirectional): sampled rows and keys vs the oracle."""
    cfg = wl.WORKLOADS[6]
    lay = wl.layout_for(cfg)
    tdt = DT[cfg.dtype]
    say(f"draft workload: T={lay.T} hq={cfg.hq} hkv={cfg.hkv} d={cfg.d}")
    q, k, v, do = wl.workload_tensors(cfg, lay)
    m = psa.layout_tile_map(lay, "cuda", dtype=tdt, d=cfg.d)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = psa.fwd(m, qd, kd, vd)
    dq, dk, dv = psa.bwd(m, qd, kd, vd, o, lse, dod)
    torch.cuda.synchronize()
    meta = meta_from_layout(lay)
    rng = np.random.default_rng(6)
    S = lay.extra["ctx_len"]
    rows = _sample(lay.T, 40, rng, extra=[S, S + 15, S + 16, lay.T - 1])
    wo, wl_, wdq = oa.grad_rows(meta, q, k, v, do, rows)
    compare("o", o[rows], wo, tdt)
    compare("lse", lse[:, rows], wl_, tdt)
    compare("dq", dq[rows], wdq, tdt)
    cols = _sample(lay.T, 24, rng, extra=[0, 4095, 4096, S - 1, S])
    wdk, wdv = oa.grad_cols(meta, q, k, v, do, cols)
    compare("dk", dk[cols], wdk, tdt)
    compare("dv", dv[cols], wdv, tdt)
