"""psa_bwd_noalloc (the backward without a workspace or any allocation) against psa_bwd.

Both run the same kernels in the same order; the no-alloc call only takes its
workspace from the library's fixed device array.  Its gradients must equal psa_bwd's
bit for bit, on two calls in a row, the second on a smaller input (the array keeps the
first call's contents), and sizes past the array's limit are refused before any
launch."""
import ctypes

import numpy as np
import pytest
import torch

from shared_prefix_block_amd import psa
from shared_prefix_block_amd import workloads as wl
from tests.gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu
DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _noalloc(m, q, k, v, o, lse, do, grad_dtype):
    lib = psa.load()
    T, hq, d = q.shape
    outs = (torch.full(q.shape, float("nan"), dtype=grad_dtype, device=q.device),
            torch.full(k.shape, float("nan"), dtype=grad_dtype, device=q.device),
            torch.full(v.shape, float("nan"), dtype=grad_dtype, device=q.device))
    P = psa._ptr
    st = lib.psa_bwd_noalloc(m.handle, psa._dtype_code(q.dtype), psa._dtype_code(grad_dtype), T,
                             hq, k.shape[1], d, 0.0, P(q), P(k), P(v), P(o), P(lse), P(do),
                             P(outs[0]), P(outs[1]), P(outs[2]), psa._stream(q.device))
    psa._check(st)
    return outs


def _case(lay, hq, hkv, d, dtype, seed, grad_dtype=torch.float32):
    say(f"no-alloc backward: T={lay.T} hq={hq} hkv={hkv} d={d} {dtype} grads {grad_dtype}")
    q, k, v, do = (x.cuda() for x in wl.make_tensors(lay.T, hq, hkv, d, dtype, 1.0, seed))
    m = psa.layout_tile_map(lay, "cuda", dtype=DT[dtype], d=d)
    o, lse = psa.fwd(m, q, k, v)
    want = psa.bwd(m, q, k, v, o, lse, do, grad_dtype=grad_dtype)
    got = _noalloc(m, q, k, v, o, lse, do, grad_dtype)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        assert torch.equal(a, b), name


def test_noalloc_matches_bwd_on_two_calls_the_second_smaller():
    rng = np.random.default_rng(7)
    big = wl.tokens_layout(wl.random_group_specs(rng, max_groups=4, max_p=700, max_g=6,
                                                 max_r=400), pad_multiple=128)
    small = wl.tokens_layout([(37, [20, 0, 45])], pad_multiple=16)
    _case(big, 8, 2, 128, "bf16", 1)
    _case(small, 2, 1, 64, "fp32", 2)


def test_noalloc_other_variants():
    """d = 256 bf16 (two dK/dV passes), bf16 gradient outputs, a tree through the
    interval form."""
    tree = wl.tree_layout([40, 30, 25, 50], [[0, 1, 3], [0, 2]], extra_pad=11)
    _case(tree, 4, 2, 256, "bf16", 3)
    _case(wl.tokens_layout([(90, [60, 31])], pad_multiple=64), 4, 4, 128, "bf16", 4,
          grad_dtype=torch.bfloat16)


def test_noalloc_refuses_sizes_past_its_array():
    """T x hq past the fixed array: PSA_ERR_WORKSPACE before any launch (the tensor
    pointers are NULL; a NULL check would refuse them next, so nothing can launch)."""
    lib = psa.load()
    lay = wl.tokens_layout([(4096, [])])
    m = psa.layout_tile_map(lay, "cuda", dtype=torch.bfloat16, d=64)
    z = ctypes.c_void_p(0)
    st = lib.psa_bwd_noalloc(m.handle, psa.PSA_BF16, psa.PSA_FP32, lay.T, 2048, 1, 64, 0.0,
                             z, z, z, z, z, z, z, z, z, psa._stream(torch.device("cuda")))
    assert psa.STATUS[st] == "PSA_ERR_WORKSPACE"
    assert b"fixed 33554432" in lib.psa_last_error()
    st = lib.psa_bwd_noalloc(m.handle, psa.PSA_BF16, psa.PSA_FP32, lay.T, 8, 1, 64, 0.0,
                             z, z, z, z, z, z, z, z, z, psa._stream(torch.device("cuda")))
    assert psa.STATUS[st] == "PSA_ERR_NULL"
    torch.cuda.synchronize()
