"""fp8 (OCP e4m3) no-grad forward vs the oracle run on the same e4m3 values.

The kernel's scores are exact e4m3 products summed in fp32, and V widens to bf16
without rounding, so the only rounding beyond fp32 accumulation is P's rounding to
bf16 for P V, as in the bf16 path: the bf16 parity bar applies, with the output's own
bf16 rounding allowed for (O is written in bf16)."""
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle.mask import meta_from_layout
from shared_prefix_block_amd import psa
from shared_prefix_block_amd import workloads as wl
from tests import unfolded as uf
from tests.gpu_common import compare, need_gpu, say
from tests.test_gpu_attention import _boundaries, _sample
from tests.test_gpu_draft import _random_draft
from tests.test_gpu_general import _general_layout

pytestmark = pytest.mark.gpu
F8 = torch.float8_e4m3fn
BF = torch.bfloat16
OUT_ROUND = 2.0 ** -9


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _fwd8(lay, hq, hkv, d, seed, sigma=1.0, with_lse=True, form=None):
    q, k, v, _ = wl.make_tensors(lay.T, hq, hkv, d, "fp8", sigma, seed, with_grad_out=False)
    kw = {} if form is None else {"form": form}
    m = psa.layout_tile_map(lay, "cuda", dtype=F8, d=d, **kw)
    o, lse = psa.fwd(m, q.cuda(), k.cuda(), v.cuda(), with_lse=with_lse)
    torch.cuda.synchronize()
    assert o.dtype == BF and o.shape == (lay.T, hq, d)
    return (q, k, v), o, lse, m


def _check(lay, hq, hkv, d, seed, sigma=1.0, form=None):
    say(f"fp8 forward: kind={lay.kind} T={lay.T} hq={hq} hkv={hkv} d={d} seed={seed}")
    (q, k, v), o, lse, _ = _fwd8(lay, hq, hkv, d, seed, sigma, form=form)
    want_o, want_lse = oa.forward(meta_from_layout(lay), q, k, v)
    compare("o", o, want_o, BF, out_round=OUT_ROUND)
    compare("lse", lse, want_lse, BF)


SHAPES8 = [(2, 1, 64), (4, 2, 128), (2, 2, 256), (8, 2, 128), (3, 3, 64), (4, 1, 256)]


@pytest.mark.parametrize("seed", range(12))
def test_fp8_fuzz_tokens(seed):
    rng = np.random.default_rng(9100 + seed)
    specs = wl.random_group_specs(rng, max_groups=4, max_p=150, max_g=5, max_r=150)
    lay = wl.tokens_layout(specs, pad_multiple=int(rng.integers(1, 130)),
                           extra_pad=int(rng.integers(0, 3)))
    if lay.T == 0:
        return
    hq, hkv, d = SHAPES8[seed % len(SHAPES8)]
    # the absolute bar is set for inputs of unit scale (as in the bf16 tests)
    _check(lay, hq, hkv, d, seed, sigma=float(rng.choice([0.5, 1.0])))


@pytest.mark.parametrize("seed", range(9))
def test_fp8_fuzz_general(seed):
    """Unpacked layouts and non-DFS trees: the node-form kernels."""
    rng = np.random.default_rng(9200 + seed)
    lay = _general_layout(rng, ["prompt_first", "any_order", "tree"][seed % 3])
    if lay.T == 0:
        return
    hq, hkv, d = SHAPES8[(seed + 1) % len(SHAPES8)]
    _check(lay, hq, hkv, d, seed)


@pytest.mark.parametrize("seed", range(6))
def test_fp8_fuzz_draft(seed):
    rng = np.random.default_rng(9300 + seed)
    lay = _random_draft(rng)
    if lay.T == 0:
        return
    hq, hkv, d = SHAPES8[(seed + 2) % len(SHAPES8)]
    _check(lay, hq, hkv, d, seed)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_forms_agree(d):
    """A packed layout forced into node form gives the interval form's O bit for bit."""
    lay = wl.tokens_layout([(200, [90, 150, 0, 40]), (0, [70]), (130, [260, 5])],
                           pad_multiple=128)
    _, o1, l1, m1 = _fwd8(lay, 4, 2, d, 3)
    _, o2, l2, m2 = _fwd8(lay, 4, 2, d, 3, form="nodes")
    assert m1.info["form"] == psa.FORM_INTERVAL and m2.info["form"] == psa.FORM_NODES
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_without_lse_and_pads():
    """lse NULL writes the same O; pad rows get O = 0 (and LSE = -inf with an LSE)."""
    lay = wl.tokens_layout([(70, [40, 25]), (30, [50, 0])], pad_multiple=128)
    _, o1, lse1, m = _fwd8(lay, 4, 2, 128, 5)
    (q, k, v), o2, lse2, _ = _fwd8(lay, 4, 2, 128, 5, with_lse=False)
    assert lse2 is None
    assert torch.equal(o1, o2)
    pads = slice(lay.T_real, lay.T)
    assert lay.T > lay.T_real
    assert bool((o1[pads] == 0).all())
    assert bool(torch.isneginf(lse1[:, pads]).all())


def test_fp8_zero_query_closed_form():
    """Q = 0: every visible score is 0, so LSE = ln(#visible keys) and O is the mean of
    the visible V rows, here taken from the layout's own sample sequences."""
    lay = wl.tokens_layout([(100, [60, 30]), (50, [80])], pad_multiple=64)
    _, k, v, _ = wl.make_tensors(lay.T, 2, 1, 64, "fp8", 1.0, 8, with_grad_out=False)
    q = torch.zeros(lay.T, 2, 64, dtype=F8)
    m = psa.layout_tile_map(lay, "cuda", dtype=F8, d=64)
    o, lse = psa.fwd(m, q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    seqs, _ = uf.group_sequences(lay.specs)
    vv = v.double().numpy()[:, 0]
    n_vis = np.zeros(lay.T, np.int64)
    mean_v = np.zeros((lay.T, 64))
    for s in seqs:
        n_vis[s] = np.arange(1, len(s) + 1)
        mean_v[s] = np.cumsum(vv[s], axis=0) / n_vis[s][:, None]
    with np.errstate(divide="ignore"):
        want_lse = np.where(n_vis > 0, np.log(np.maximum(n_vis, 1)), -np.inf)
    for h in range(2):
        compare(f"lse[{h}]", lse[h].cpu(), want_lse, torch.float32)
        compare(f"o[{h}]", o[:, h], mean_v, BF, out_round=OUT_ROUND)


@pytest.mark.parametrize("idx", [2, 4, 5, 6])
def test_fp8_workload_sampled(idx):
    """The workloads' full-size layouts in e4m3, at sampled rows and their boundaries."""
    cfg = wl.WORKLOADS[idx]
    lay = wl.layout_for(cfg)
    say(f"fp8 workload {idx}: T={lay.T} hq={cfg.hq} hkv={cfg.hkv} d={cfg.d}")
    (q, k, v), o, lse, _ = _fwd8(lay, cfg.hq, cfg.hkv, cfg.d, cfg.idx, cfg.sigma)
    rng = np.random.default_rng(idx)
    extra = _boundaries(lay) if lay.kind in ("tokens", "tree") else ()
    rows = _sample(lay.T, 48, rng, extra)
    want_o, want_lse = oa.forward(meta_from_layout(lay), q, k, v, rows=rows)
    compare("o", o[rows], want_o, BF, out_round=OUT_ROUND)
    compare("lse", lse[:, rows], want_lse, BF)


def test_fp8_rejections():
    lay = wl.tokens_layout([(40, [30, 20])], pad_multiple=64)
    q, k, v, do = (x.cuda() for x in wl.make_tensors(lay.T, 2, 2, 64, "fp8", 1.0, 1))
    m = psa.layout_tile_map(lay, "cuda", dtype=F8, d=64)
    o, lse = psa.fwd(m, q, k, v)
    with pytest.raises(RuntimeError, match="compiled"):  # no backward in e4m3
        psa.bwd_workspace_size(m, q, k)
    with pytest.raises(ValueError, match="out"):
        psa.fwd(m, q, k, v, out=torch.empty(q.shape, dtype=F8, device="cuda"))
    q96 = torch.zeros(lay.T, 2, 96, dtype=F8, device="cuda")
    with pytest.raises(RuntimeError):
        psa.fwd(m, q96, q96[:, :2].contiguous(), q96[:, :2].contiguous())
    torch.cuda.synchronize()
