"""Argument checks of the Python binding that need no GPU: the buffers the kernels
read or write whole are refused before any call when their shape, dtype, layout or
device is not the one the kernels assume."""
import pytest
import torch

from shared_prefix_block_amd import psa


def test_check_buf_accepts_the_exact_buffer():
    t = torch.empty(4, 10, dtype=torch.float32)
    psa._check_buf(t, (4, 10), torch.float32, t.device, "lse")


@pytest.mark.parametrize("bad", [
    torch.empty(4, 9),                      # one row short
    torch.empty(4, 10, dtype=torch.bfloat16),
    torch.empty(10, 4).t(),                 # right shape, not contiguous
    torch.empty(40),
])
def test_check_buf_refuses(bad):
    with pytest.raises(ValueError, match="lse"):
        psa._check_buf(bad, (4, 10), torch.float32, torch.device("cpu"), "lse")


def test_check_qkv_refuses_host_and_mismatched_tensors():
    q = torch.empty(8, 2, 64)
    with pytest.raises(ValueError, match="device"):
        psa._check_qkv(q, q, q)
    with pytest.raises(ValueError):
        psa._check_qkv(q[0], q, q)


def test_dtype_codes():
    assert psa._dtype_code(torch.float32) == psa.PSA_FP32
    assert psa._dtype_code(torch.bfloat16) == psa.PSA_BF16
    assert psa._dtype_code(torch.float8_e4m3fn) == psa.PSA_FP8_E4M3
    with pytest.raises(TypeError):
        psa._dtype_code(torch.float16)


def _rollouts():
    return psa.Rollouts([3, 2], [[2, 1], []])  # fold length 8, unfold length 3+2 + 3+1 = 9


def test_fold_refuses_token_buffers_of_the_wrong_length():
    r = _rollouts()
    with pytest.raises(ValueError, match="prompt_tok must hold 5"):
        psa.fold_rollouts(r, torch.zeros(4, dtype=torch.int32), torch.zeros(3, dtype=torch.int32), 8)
    with pytest.raises(ValueError, match="comp_tok must hold 3"):
        psa.fold_rollouts(r, torch.zeros(5, dtype=torch.int32), torch.zeros(4, dtype=torch.int32), 8)
    with pytest.raises(ValueError, match="device tensor"):  # right sizes, host memory
        psa.fold_rollouts(r, torch.zeros(5, dtype=torch.int32), torch.zeros(3, dtype=torch.int32), 8)


def test_unfold_refuses_short_and_host_sources():
    r = _rollouts()
    assert (r.fold_len, r.unfold_len) == (8, 9)
    with pytest.raises(ValueError, match="folded layout's 8 rows"):
        psa.unfold_rows(r, torch.zeros(7, 4))
    with pytest.raises(ValueError, match="device tensor"):
        psa.unfold_rows(r, torch.zeros(8, 4))


def test_unfold_output_and_workspace_checks():
    r = _rollouts()
    cpu = torch.device("cpu")
    with pytest.raises(ValueError, match="out"):  # one row short of the 9 unfolded rows
        psa._check_buf(torch.empty(8, 4), (r.unfold_len, 4), torch.float32, cpu, "out")
    with pytest.raises(ValueError, match="smaller than"):
        psa._check_ws(torch.empty(1, dtype=torch.uint8), r, cpu)
    with pytest.raises(ValueError, match="contiguous tensor on"):
        psa._check_ws(torch.empty(4096, dtype=torch.uint8)[::2], r, cpu)
    psa._check_ws(torch.empty(4096, dtype=torch.uint8), r, cpu)


def test_draft_builder_refuses_arrays_of_the_wrong_length():
    a = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="keep must hold 4"):
        psa.build_tile_map_draft(10, 4, a, keep=torch.ones(3, dtype=torch.uint8))
    with pytest.raises(ValueError, match="ctx_doc must hold 10"):
        psa.build_tile_map_draft(10, 4, a, ctx_doc=torch.zeros(9, dtype=torch.int32),
                                 anchor_doc=torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="anchor_doc must hold 4"):
        psa.build_tile_map_draft(10, 4, a, ctx_doc=torch.zeros(10, dtype=torch.int32),
                                 anchor_doc=torch.zeros(5, dtype=torch.int32))
    with pytest.raises(ValueError, match="both or neither"):
        psa.build_tile_map_draft(10, 4, a, ctx_doc=torch.zeros(10, dtype=torch.int32))
    with pytest.raises(TypeError, match="device tensors"):  # right sizes, host memory
        psa.build_tile_map_draft(10, 4, a)
