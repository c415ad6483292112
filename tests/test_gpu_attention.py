"""GPU forward / backward vs the float64 oracle (the parity bar), plus closed forms."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle.mask import meta_from_layout
from shared_prefix_block_amd import psa
from shared_prefix_block_amd import workloads as wl
from tests import unfolded as uf
from tests.gpu_common import compare, need_gpu, say

pytestmark = pytest.mark.gpu
DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _run(lay, hq, hkv, d, dtype, seed, sigma=1.0, backward=True, scale=None,
         grad_dtype=torch.float32, split=False):
    q, k, v, do = wl.make_tensors(lay.T, hq, hkv, d, dtype, sigma, seed)
    tdt = DT[dtype]
    m = psa.layout_tile_map(lay, "cuda", dtype=tdt, d=d)
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    o, lse = psa.fwd(m, qd, kd, vd, scale)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = psa.bwd(m, qd, kd, vd, o, lse, dod, scale, grad_dtype=grad_dtype,
                             split=split)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return (q, k, v, do), out


def _check_full(lay, hq, hkv, d, dtype, seed, sigma=1.0, backward=True, scale=None):
    say(f"attention full: T={lay.T} kind={lay.kind} hq={hq} hkv={hkv} d={d} {dtype} "
        f"seed={seed} bwd={backward}")
    (q, k, v, do), got = _run(lay, hq, hkv, d, dtype, seed, sigma, backward, scale)
    meta = meta_from_layout(lay)
    tdt = DT[dtype]
    if backward:
        o, lse, dq, dk, dv = oa.backward(meta, q, k, v, do, scale=scale)
        compare("dq", got["dq"], dq, tdt)
        compare("dk", got["dk"], dk, tdt)
        compare("dv", got["dv"], dv, tdt)
    else:
        o, lse = oa.forward(meta, q, k, v, scale=scale)
    compare("o", got["o"], o, tdt)
    compare("lse", got["lse"], lse, tdt)


CASES = [  # (hq, hkv, d, dtype)
    (2, 2, 64, "fp32"), (4, 2, 128, "fp32"), (2, 1, 64, "bf16"), (4, 2, 128, "bf16"),
    (2, 2, 256, "bf16"), (3, 1, 128, "bf16"), (4, 4, 64, "fp32"), (8, 2, 128, "bf16"),
]


@pytest.mark.parametrize("seed", range(16))
def test_fuzz_tokens(seed):
    rng = np.random.default_rng(700 + seed)
    specs = wl.random_group_specs(rng, max_groups=4, max_p=150, max_g=5, max_r=150)
    lay = wl.tokens_layout(specs, pad_multiple=int(rng.integers(1, 130)),
                           extra_pad=int(rng.integers(0, 3)))
    if lay.T == 0:
        return
    hq, hkv, d, dt = CASES[seed % len(CASES)]
    _check_full(lay, hq, hkv, d, dt, seed)


@pytest.mark.parametrize("seed", range(6))
def test_fuzz_fp32_d256(seed):
    """fp32 at head_dim 256: the dQ and dK launches that each take half the columns,
    the dV pass, one LDS buffer where two do not fit; token layouts and trees."""
    rng = np.random.default_rng(900 + seed)
    if seed % 2:
        nl, paths = wl.random_tree(rng, max_nodes=8, max_len=130)
        lay = wl.tree_layout(nl, paths, extra_pad=int(rng.integers(0, 50)))
    else:
        specs = wl.random_group_specs(rng, max_groups=3, max_p=200, max_g=4, max_r=150)
        lay = wl.tokens_layout(specs, pad_multiple=int(rng.integers(1, 130)))
    if lay.T == 0:
        return
    hq, hkv = [(2, 2), (4, 2), (3, 1)][seed % 3]
    _check_full(lay, hq, hkv, 256, "fp32", seed)


@pytest.mark.parametrize("seed", range(8))
def test_fuzz_trees(seed):
    rng = np.random.default_rng(800 + seed)
    nl, paths = wl.random_tree(rng, max_nodes=9, max_len=100)
    lay = wl.tree_layout(nl, paths, extra_pad=int(rng.integers(0, 50)))
    if lay.T == 0:
        return
    hq, hkv, d, dt = CASES[(seed + 3) % len(CASES)]
    _check_full(lay, hq, hkv, d, dt, seed)


VARIANTS = [(64, "fp32"), (128, "fp32"), (256, "fp32"), (64, "bf16"), (128, "bf16"),
            (256, "bf16")]


@pytest.mark.parametrize("d,dtype", VARIANTS)
def test_pad_rows_every_variant(d, dtype):
    """Rows that see no key (pads between and after groups, a lone node) in every
    compiled variant: O = 0, LSE = -inf, zero gradients, the rest at parity."""
    _check_full(wl.tree_layout([9], [[0]], extra_pad=14), 2, 2, d, dtype, 1)
    lay = wl.tokens_layout([(5, [7, 0, 3]), (0, [4])], pad_multiple=64, extra_pad=3)
    _check_full(lay, 2, 1, d, dtype, 2)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_bf16_gradient_outputs(d):
    """Gradients stored in bf16: the parity bar plus the rounding of the stored value."""
    rng = np.random.default_rng(40 + d)
    specs = wl.random_group_specs(rng, max_groups=3, max_p=200, max_g=4, max_r=150)
    lay = wl.tokens_layout(specs, pad_multiple=64)
    say(f"bf16 gradients d={d} T={lay.T}")
    (q, k, v, do), got = _run(lay, 4, 2, d, "bf16", 9, grad_dtype=torch.bfloat16)
    _, _, dq, dk, dv = oa.backward(meta_from_layout(lay), q, k, v, do)
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert got[name].dtype == torch.bfloat16
        compare(name, got[name], ref, torch.bfloat16, out_round=2.0 ** -9)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_split_mode_is_more_accurate(d):
    """PSA_BWD_SPLIT_PDS carries P and dS to ~17 bits.  dV = P^T dO then sits within a
    tenth of the bf16 bar; dK and dQ also carry the rounding of the bf16 O that
    D = rowsum(dO * O) is formed from (part of the interface), so they get the bar."""
    rng = np.random.default_rng(60 + d)
    specs = wl.random_group_specs(rng, max_groups=3, max_p=300, max_g=4, max_r=200)
    lay = wl.tokens_layout(specs, pad_multiple=32)
    say(f"split mode d={d} T={lay.T}")
    (q, k, v, do), got = _run(lay, 4, 2, d, "bf16", 11, split=True)
    _, _, dq, dk, dv = oa.backward(meta_from_layout(lay), q, k, v, do)
    err = float((got["dv"].double().cpu() - torch.as_tensor(dv)).abs().max())
    assert err <= 2e-3, ("dv", err)
    compare("dq", got["dq"], dq, torch.bfloat16)
    compare("dk", got["dk"], dk, torch.bfloat16)


def test_bwd_flags_rejected():
    lay = wl.tokens_layout([(40, [30, 20])])
    q, k, v, do = (x.cuda() for x in wl.make_tensors(lay.T, 2, 2, 64, "bf16"))
    m = psa.layout_tile_map(lay, "cuda", dtype=torch.bfloat16, d=64)
    o, lse = psa.fwd(m, q, k, v)
    for bad in (0, psa.BWD_SPLIT_PDS, 32, psa.STAGE_ALL | 8, -1):
        with pytest.raises(RuntimeError, match="flags"):
            psa.bwd(m, q, k, v, o, lse, do, stages=bad)
    torch.cuda.synchronize()


@pytest.mark.parametrize("d,dtype", [(64, "fp32"), (128, "fp32"), (256, "fp32"), (128, "bf16"),
                                     (256, "bf16")])
def test_forward_without_lse(d, dtype):
    """The no-grad forward (lse NULL) writes the same O as the full forward and leaves
    the memory an LSE would go to alone."""
    lay = wl.tokens_layout([(70, [40, 25]), (30, [50, 0])], pad_multiple=128)
    say(f"forward without LSE: T={lay.T} d={d} {dtype}")
    q, k, v, _ = wl.make_tensors(lay.T, 4, 2, d, dtype, 1.0, 5)
    m = psa.layout_tile_map(lay, "cuda", dtype=DT[dtype], d=d)
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    o1, lse1 = psa.fwd(m, qd, kd, vd)
    guard = torch.full((4, lay.T), 7.0, device="cuda")
    o2, lse2 = psa.fwd(m, qd, kd, vd, with_lse=False)
    torch.cuda.synchronize()
    assert lse2 is None
    assert torch.equal(o1, o2)
    assert bool((guard == 7.0).all())
    compare("o", o2, oa.forward(meta_from_layout(lay), q, k, v)[0], DT[dtype])


@pytest.mark.parametrize("d,dtype", [(64, "fp32"), (256, "fp32"), (128, "bf16"), (256, "bf16")])
def test_stage_orders_agree(d, dtype):
    """psa_bwd runs dQ with the preparation of its rows first, then dK/dV; the stages run
    one by one (prepare, dK/dV, dQ) must give the same gradients, both at the parity bar
    against the oracle, with pad rows and partial tiles in the layout."""
    lay = wl.tokens_layout([(70, [40, 25, 0]), (5, [60])], pad_multiple=128)
    hq, hkv, seed = 4, 2, 11
    say(f"stage orders: T={lay.T} d={d} {dtype}")
    q, k, v, do = wl.make_tensors(lay.T, hq, hkv, d, dtype, 1.0, seed)
    tdt = DT[dtype]
    m = psa.layout_tile_map(lay, "cuda", dtype=tdt, d=d)
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    o, lse = psa.fwd(m, qd, kd, vd)
    fused = psa.bwd(m, qd, kd, vd, o, lse, dod)
    ws = torch.empty(psa.bwd_workspace_size(m, qd, kd), dtype=torch.uint8, device="cuda")
    outs = tuple(torch.full(x.shape, float("nan"), device="cuda") for x in (qd, kd, vd))
    for st in (psa.STAGE_PREPARE, psa.STAGE_DKDV, psa.STAGE_DQ):
        psa.bwd(m, qd, kd, vd, o, lse, dod, workspace=ws, stages=st, out=outs)
    torch.cuda.synchronize()
    _, _, dq, dk, dv = oa.backward(meta_from_layout(lay), q, k, v, do)
    for got in (fused, outs):
        compare("dq", got[0], dq, tdt)
        compare("dk", got[1], dk, tdt)
        compare("dv", got[2], dv, tdt)
    for a, b in zip(fused, outs):  # the same sums up to the order of D's fp32 additions
        assert torch.allclose(a, b, rtol=1e-4, atol=1e-5)


@pytest.mark.parametrize("T", [1, 2, 31, 127, 128, 129, 300])
def test_single_causal_sequence_ragged(T):
    """One group with no completion = plain causal attention, at ragged lengths."""
    _check_full(wl.tokens_layout([(T, [])]), 2, 1, 128, "bf16", T)
    _check_full(wl.tokens_layout([(T, [])]), 2, 2, 64, "fp32", T)


def test_degenerate_layouts():
    for specs, pad in [([(0, [0, 0])], 5), ([(3, [0, 4, 0])], 0), ([(0, [70, 1])], 130),
                       ([(200, [])] * 3, 1)]:
        lay = wl.tokens_layout(specs, extra_pad=pad)
        _check_full(lay, 2, 1, 64, "fp32", 3)


def test_all_pad_rows():
    lay = wl.tokens_layout([], extra_pad=200)
    (_, _, _, _), got = _run(lay, 2, 2, 64, "fp32", 0)
    assert torch.all(got["o"] == 0) and torch.all(torch.isneginf(got["lse"]))
    assert torch.all(got["dq"] == 0) and torch.all(got["dk"] == 0) and torch.all(got["dv"] == 0)


def test_custom_scale():
    lay = wl.tokens_layout([(40, [30, 50])], pad_multiple=16)
    _check_full(lay, 4, 2, 128, "bf16", 5, scale=0.05)
    _check_full(lay, 2, 2, 64, "fp32", 5, scale=0.3)


# ----------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration the bench times
# ----------------------------------------------------------------------------
def _sample(T, n, rng, extra=()):
    base = set(int(x) for x in rng.choice(T, size=min(n, T), replace=False))
    base |= {0, T - 1} | {int(x) for x in extra if 0 <= x < T}
    return np.asarray(sorted(base), dtype=np.int64)


def _prompt_keys(lay, g):
    """Prompt keys of group g: its first and last, the keys on both sides of every
    128-key tile edge inside the prompt (at most 4 edges, spread), and the middle."""
    start = sum(p + sum(rs) for p, rs in lay.specs[:g])
    p = lay.specs[g][0]
    keys = {start, start + p - 1, start + p // 2}
    edges = [t for t in range(start + 1, start + p) if t % 128 == 0]
    for t in edges[:: max(1, len(edges) // 4)][:4]:
        keys |= {t - 1, t}
    return np.asarray(sorted(keys), dtype=np.int64)


def _boundaries(lay):
    """Token positions around group / completion / node boundaries and tile edges."""
    pts = []
    if lay.kind == "tokens":
        base = 0
        for p, rs in lay.specs:
            pts += [base, base + p - 1, base + p]
            cur = base + p
            for r in rs:
                pts += [cur, cur + r - 1]
                cur += r
            base = cur
    else:
        starts = np.cumsum([0] + list(lay.node_lengths))
        for s in starts:
            pts += [int(s) - 1, int(s)]
    pts += [lay.T_real - 1, lay.T_real]
    return pts[:400]


@pytest.mark.parametrize("idx,split", [(1, False), (2, False), (3, False), (4, False),
                                       (5, False), (2, True), (4, True)])
def test_workload_parity_sampled(idx, split):
    cfg = wl.WORKLOADS[idx]
    lay = wl.layout_for(cfg)
    backward = cfg.passes != "fwd"
    say(f"workload {idx}: T={lay.T} hq={cfg.hq} hkv={cfg.hkv} d={cfg.d} {cfg.dtype} "
        f"split={split}")
    (q, k, v, do), got = _run(lay, cfg.hq, cfg.hkv, cfg.d, cfg.dtype, cfg.idx, cfg.sigma,
                              backward, split=split)
    meta = meta_from_layout(lay)
    tdt = DT[cfg.dtype]
    rng = np.random.default_rng(idx)
    rows = _sample(lay.T, 48 if idx != 1 else lay.T, rng, _boundaries(lay))
    if backward:
        o, lse, dq = oa.grad_rows(meta, q, k, v, do, rows)
        compare("dq", got["dq"][rows], dq, tdt)
    else:
        o, lse = oa.forward(meta, q, k, v, rows=rows)
    compare("o", got["o"][rows], o, tdt)
    compare("lse", got["lse"][:, rows], lse, tdt)
    if not backward:
        return
    # key rows: completion keys (cheap) everywhere; prompt keys where the group is small
    if lay.kind == "tokens":
        suffix_keys = np.nonzero(lay.is_prefix == 0)[0]
        suffix_keys = suffix_keys[lay.group[suffix_keys] >= 0]
        cols = list(rng.choice(suffix_keys, size=24, replace=False))
        small = max(p + sum(rs) for p, rs in lay.specs) <= 4096
        if small:
            pre = np.nonzero(lay.is_prefix == 1)[0]
            cols += list(rng.choice(pre, size=8, replace=False))
    else:
        starts = np.cumsum([0] + list(lay.node_lengths))
        leaf_tokens = np.arange(starts[2], starts[6])  # first tree: branch 0 and its leaves
        cols = list(rng.choice(leaf_tokens, size=24, replace=False)) + [0, 1, 1023]
    cols = np.asarray(sorted(set(int(c) for c in cols)), dtype=np.int64)
    dk, dv = oa.grad_cols(meta, q, k, v, do, cols)
    compare("dk", got["dk"][cols], dk, tdt)
    compare("dv", got["dv"][cols], dv, tdt)
    if lay.kind == "tokens" and not small:
        # prompt keys of a large group, element by element on one kv head: the keys
        # with the longest CSC lists (every completion tile of the group walks them),
        # where the oracle has to recompute every row of the group
        g = int(np.argmax([p for p, _ in lay.specs]))
        pcols = _prompt_keys(lay, g)
        heads = [g % cfg.hkv]
        say(f"workload {idx}: {len(pcols)} prompt keys of group {g} (P={lay.specs[g][0]}), "
            f"kv head {heads[0]}")
        dkp, dvp = oa.grad_cols(meta, q, k, v, do, pcols, kv_heads=heads)
        compare("dk prompt keys", got["dk"][pcols][:, heads], dkp, tdt)
        compare("dv prompt keys", got["dv"][pcols][:, heads], dvp, tdt)
    # whole-tensor identities: sum_kv dV = sum_q dO (rows with a key), sum_kv dK = 0
    rep = cfg.hq // cfg.hkv
    dv_sum = got["dv"].double().sum(0).cpu()  # [hkv, d]
    do_sum = do[: lay.T_real].double().sum(0).view(cfg.hkv, rep, cfg.d).sum(1)
    dk_sum = got["dk"].double().sum(0).cpu()
    n = lay.T_real
    # each output element carries at most half a bf16 ulp of rounding; bound the sums
    tol = 2e-2 * math.sqrt(n) if cfg.dtype == "bf16" else 1e-5 * math.sqrt(n)
    assert float((dv_sum - do_sum).abs().max()) < tol
    assert float(dk_sum.abs().max()) < tol


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_zero_query_closed_form(idx):
    """Q = 0 pins the kernel's mask row by row without the oracle: every visible score is
    0, so LSE = ln(#visible keys) and O = the mean of the visible V rows."""
    cfg = wl.WORKLOADS[idx]
    lay = wl.layout_for(cfg)
    _, k, v, _ = wl.make_tensors(lay.T, cfg.hq, cfg.hkv, cfg.d, cfg.dtype, cfg.sigma, idx,
                                 with_grad_out=False)
    q = torch.zeros(lay.T, cfg.hq, cfg.d, dtype=DT[cfg.dtype])
    m = psa.layout_tile_map(lay, "cuda", dtype=DT[cfg.dtype], d=cfg.d)
    o, lse = psa.fwd(m, q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    if lay.kind == "tokens":
        seqs, _ = uf.group_sequences(lay.specs)
    else:
        seqs = uf.tree_sequences(lay.node_lengths, lay.sample_paths)
    n_vis = np.zeros(lay.T, np.int64)
    mean_v = np.zeros((lay.T, cfg.hkv, cfg.d))
    vv = v.double().numpy()
    for s in seqs:
        csum = np.cumsum(vv[s], axis=0) / np.arange(1, len(s) + 1)[:, None, None]
        n_vis[s] = np.arange(1, len(s) + 1)
        mean_v[s] = csum
    with np.errstate(divide="ignore"):
        want_lse = np.where(n_vis > 0, np.log(np.maximum(n_vis, 1)), -np.inf)
    lse_h = lse.cpu().double().numpy()
    rep = cfg.hq // cfg.hkv
    for h in range(cfg.hq):
        compare(f"lse[{h}]", lse_h[h], want_lse, torch.float32)
    o_h = o.float().cpu().double().numpy()
    for h in range(0, cfg.hq, max(1, cfg.hq // 4)):
        compare(f"o[{h}]", o_h[:, h], mean_v[:, h // rep], DT[cfg.dtype])


def test_map_mismatch_errors():
    lay = wl.tokens_layout([(40, [30, 50])])
    q, k, v, do = (x.cuda() for x in wl.make_tensors(lay.T, 2, 2, 128, "bf16", 1.0, 0))
    m_other = psa.layout_tile_map(wl.tokens_layout([(41, [30, 50])]), "cuda")
    with pytest.raises(psa.PsaError) as ei:
        psa.fwd(m_other, q, k, v)
    assert ei.value.name == "PSA_ERR_MAP_MISMATCH"
    m_shape = psa.layout_tile_map(lay, "cuda", block_m=64, block_n=64)
    with pytest.raises(psa.PsaError) as ei:
        psa.fwd(m_shape, q, k, v)
    assert ei.value.name == "PSA_ERR_MAP_MISMATCH"
    m = psa.layout_tile_map(lay, "cuda")
    q96 = torch.zeros(lay.T, 2, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(psa.PsaError) as ei:
        psa.fwd(m, q96, q96[:, :2].contiguous(), q96[:, :2].contiguous())
    assert ei.value.name == "PSA_ERR_UNSUPPORTED"
    o, lse = psa.fwd(m, q, k, v)
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(psa.PsaError) as ei:
        psa.bwd(m, q, k, v, o, lse, do, workspace=small)
    assert ei.value.name == "PSA_ERR_WORKSPACE"
    # caller buffers the kernels would read or write past: refused before any launch
    with pytest.raises(ValueError, match="lse"):
        psa.fwd(m, q, k, v, lse=torch.empty(2, lay.T - 1, device="cuda"))
    with pytest.raises(ValueError, match="out"):
        psa.fwd(m, q, k, v, out=torch.empty(q.shape, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="lse"):
        psa.bwd(m, q, k, v, o, lse[:1], do)
    with pytest.raises(ValueError, match="dq"):
        psa.bwd(m, q, k, v, o, lse, do, out=(torch.empty(q.shape, dtype=torch.bfloat16,
                                                         device="cuda"),) + tuple(
            torch.empty(k.shape, device="cuda") for _ in range(2)))
    with pytest.raises(ValueError, match="workspace"):
        psa.bwd(m, q, k, v, o, lse, do, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError, match="do"):
        psa.bwd(m, q, k, v, o, lse, do[:, :1].contiguous())
    torch.cuda.synchronize()


def test_autograd_wrapper():
    lay = wl.tokens_layout([(33, [20, 17])], pad_multiple=8)
    q, k, v, do = wl.make_tensors(lay.T, 4, 2, 64, "fp32", 1.0, 4)
    m = psa.layout_tile_map(lay, "cuda", dtype=torch.float32, d=64)
    qd, kd, vd = (x.cuda().requires_grad_(True) for x in (q, k, v))
    o = psa.PrefixAttention.apply(qd, kd, vd, m)
    o.backward(do.cuda())
    _, _, dq, dk, dv = oa.backward(meta_from_layout(lay), q, k, v, do)
    compare("dq", qd.grad, dq, torch.float32)
    compare("dk", kd.grad, dk, torch.float32)
    compare("dv", vd.grad, dv, torch.float32)
