"""A sequence past 2^32 bytes per tensor: 512 groups of a 1024-token prompt and 8
completions of 512 (T = 2,621,440), 8 q heads / 2 kv heads, d = 128, bf16.  Q, O and
dO hold 5.4 GB each and dQ (fp32) 10.7 GB, so every byte offset past 2^32 goes
through the kernels' address arithmetic.  Groups never see one another, so sampled
rows and keys of the first, a middle and the last group are checked against the
oracle run on that group alone."""
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle.mask import meta_from_layout
from shared_prefix_block_amd import psa
from shared_prefix_block_amd import workloads as wl
from tests.gpu_common import compare, need_gpu, say

pytestmark = pytest.mark.gpu


def test_offsets_past_four_gigabytes():
    need_gpu()
    spec = (1024, [512] * 8)
    n_groups, hq, hkv, d = 512, 8, 2, 128
    lay = wl.tokens_layout([spec] * n_groups)
    T, L = lay.T, 1024 + 8 * 512
    assert T * hq * d * 2 > 2 ** 32
    say(f"large: T={T} hq={hq} hkv={hkv} d={d} ({T * hq * d * 2 / 1e9:.1f} GB per q tensor)")
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(11)
    q = torch.randn(T, hq, d, device=dev, generator=gen).to(torch.bfloat16)
    k = torch.randn(T, hkv, d, device=dev, generator=gen).to(torch.bfloat16)
    v = torch.randn(T, hkv, d, device=dev, generator=gen).to(torch.bfloat16)
    do = torch.randn(T, hq, d, device=dev, generator=gen).to(torch.bfloat16)
    m = psa.layout_tile_map(lay, dev, dtype=torch.bfloat16, d=d)
    o, lse = psa.fwd(m, q, k, v)
    dq, dk, dv = psa.bwd(m, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    say("large: kernels done")
    one = wl.tokens_layout([spec])
    meta = meta_from_layout(one)
    rng = np.random.default_rng(5)
    for g in (0, n_groups // 2, n_groups - 1):
        s0 = g * L
        sl = slice(s0, s0 + L)
        qg, kg, vg, dog = (x[sl].cpu() for x in (q, k, v, do))
        rows = np.unique(np.concatenate([rng.choice(L, 12, replace=False), [0, 1023, 1024, L - 1]]))
        wo, wlse, wdq = oa.grad_rows(meta, qg, kg, vg, dog, rows)
        compare(f"o[g{g}]", o[s0 + rows], wo, torch.bfloat16)
        compare(f"lse[g{g}]", lse[:, s0 + rows], wlse, torch.bfloat16)
        compare(f"dq[g{g}]", dq[s0 + rows], wdq, torch.bfloat16)
        cols = np.unique(np.concatenate([rng.choice(L, 8, replace=False), [0, L - 1]]))
        wdk, wdv = oa.grad_cols(meta, qg, kg, vg, dog, cols)
        compare(f"dk[g{g}]", dk[s0 + cols], wdk, torch.bfloat16)
        compare(f"dv[g{g}]", dv[s0 + cols], wdv, torch.bfloat16)
