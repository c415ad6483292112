"""GPU fold / unfold of rollout groups vs the oracle: bit-exact (integer and byte work)."""
import numpy as np
import pytest
import torch

from oracle import fold as of
from shared_prefix_block_amd import psa
from shared_prefix_block_amd import workloads as wl
from tests.gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu
KEYS = ("input_ids", "labels", "position_ids", "group", "suffix", "is_prefix")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _random_rollouts(rng, max_groups=5, max_p=300, max_g=6, max_r=300, p_zero=0.15):
    prompts, comps = [], []
    for _ in range(int(rng.integers(1, max_groups + 1))):
        p = 0 if rng.random() < p_zero else int(rng.integers(0, max_p + 1))
        prompts.append(rng.integers(0, 150000, p).astype(np.int32))
        cs = []
        for _ in range(int(rng.integers(0, max_g + 1))):
            r = 0 if rng.random() < p_zero else int(rng.integers(0, max_r + 1))
            cs.append(rng.integers(0, 150000, r).astype(np.int32))
        comps.append(cs)
    return prompts, comps


def _device_tokens(prompts, comps):
    pt = np.concatenate([np.asarray(p, np.int32) for p in prompts] + [np.zeros(0, np.int32)])
    ct = np.concatenate([np.asarray(c, np.int32) for cs in comps for c in cs] +
                        [np.zeros(0, np.int32)])
    return torch.from_numpy(pt).cuda(), torch.from_numpy(ct).cuda()


def _check_fold(prompts, comps, T, pad_id=7, ignore=-100):
    r = psa.Rollouts([len(p) for p in prompts], [[len(c) for c in cs] for cs in comps])
    pt, ct = _device_tokens(prompts, comps)
    got = psa.fold_rollouts(r, pt, ct, T, pad_id=pad_id, ignore_index=ignore)
    torch.cuda.synchronize()
    want = of.fold(prompts, comps, T, pad_id=pad_id, ignore=ignore)
    for k in KEYS:
        g = got[k].cpu().numpy()
        assert np.array_equal(g, want[k]), (k, np.flatnonzero(g != want[k])[:10])
    return r, got


@pytest.mark.parametrize("seed", range(12))
def test_fold_fuzz(seed):
    rng = np.random.default_rng(seed)
    prompts, comps = _random_rollouts(rng)
    n = sum(len(p) + sum(len(c) for c in cs) for p, cs in zip(prompts, comps))
    extra = int(rng.integers(0, 300))
    say(f"fold fuzz seed={seed} folded={n} T={n + extra}")
    _check_fold(prompts, comps, n + extra, pad_id=int(rng.integers(0, 9)),
                ignore=int(rng.integers(-200, -1)))


def test_fold_degenerate():
    say("fold degenerate layouts")
    _check_fold([np.zeros(0, np.int32)], [[]], T=0 + 5)                 # nothing but pads
    _check_fold([np.arange(1, 9, dtype=np.int32)], [[]], T=8)           # no completion
    _check_fold([np.zeros(0, np.int32)], [[np.arange(3, dtype=np.int32),
                                           np.zeros(0, np.int32)]], T=3)  # empty prompt
    _check_fold([np.arange(5, dtype=np.int32)] * 2,
                [[np.zeros(0, np.int32), np.arange(10, 12, dtype=np.int32)], []], T=12)


@pytest.mark.parametrize("idx", [2, 3])
def test_fold_workload_layouts(idx):
    """The workloads' rollout shapes, random token ids: the fold matches the oracle, and
    its attention metadata is the layout the attention tests and the bench use."""
    cfg = wl.WORKLOADS[idx]
    specs = wl.group_specs(cfg)
    rng = np.random.default_rng(idx)
    prompts = [rng.integers(0, 150000, p).astype(np.int32) for p, _ in specs]
    comps = [[rng.integers(0, 150000, r).astype(np.int32) for r in rs] for _, rs in specs]
    lay = wl.layout_for(cfg)
    say(f"fold workload {idx}: T={lay.T}")
    _, got = _check_fold(prompts, comps, lay.T)
    assert np.array_equal(got["group"].cpu().numpy(), lay.group)
    assert np.array_equal(got["suffix"].cpu().numpy(), lay.suffix)
    assert np.array_equal(got["is_prefix"].cpu().numpy(), lay.is_prefix)
    # the metadata feeds the tile-map builder as it is
    m = psa.build_tile_map_tokens(got["group"], got["suffix"], got["is_prefix"], 128, 128)
    assert m.info["n_full"] + m.info["n_partial"] > 0


@pytest.mark.parametrize("row_shape,dtype", [((), torch.float32), ((3,), torch.int32),
                                              ((4,), torch.float32), ((32, 128), torch.bfloat16),
                                              ((5, 2), torch.bfloat16)])
def test_unfold_rows(row_shape, dtype):
    rng = np.random.default_rng(len(row_shape) * 7 + row_shape[0] if row_shape else 1)
    prompts, comps = _random_rollouts(rng, max_groups=4, max_p=200, max_g=5, max_r=200)
    pl = [len(p) for p in prompts]
    cl = [[len(c) for c in cs] for cs in comps]
    r = psa.Rollouts(pl, cl)
    T = r.fold_len + 37
    say(f"unfold rows {row_shape} {dtype}: T={T} out={r.unfold_len}")
    src = torch.randn((T,) + row_shape).to(dtype) if dtype != torch.int32 else \
        torch.randint(-1000, 1000, (T,) + row_shape, dtype=torch.int32)
    got = psa.unfold_rows(r, src.cuda())
    torch.cuda.synchronize()
    want = of.unfold(src.view(torch.int16 if dtype == torch.bfloat16 else dtype).numpy(), pl, cl)
    g = got.cpu()
    g = g.view(torch.int16) if dtype == torch.bfloat16 else g
    assert g.shape[0] == r.unfold_len
    assert np.array_equal(g.numpy(), want)


def test_unfold_round_trip_of_the_fold():
    """Unfolding the folded tokens gives every sample [prompt | completion] back."""
    rng = np.random.default_rng(99)
    prompts, comps = _random_rollouts(rng, max_groups=6)
    r, got = _check_fold(prompts, comps, T=sum(len(p) + sum(len(c) for c in cs)
                                               for p, cs in zip(prompts, comps)) + 64)
    back = psa.unfold_rows(r, got["input_ids"]).cpu().numpy()
    want = np.concatenate([np.concatenate([p, c]) for p, cs in zip(prompts, comps) for c in cs]
                          + [np.zeros(0, np.int32)])
    assert np.array_equal(back, want)
