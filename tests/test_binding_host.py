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
