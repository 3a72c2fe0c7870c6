"""The measurement copy probe moves every element (whole and partial tiles,
scrambled and in-order granules, the last n % 4 floats), also in place."""
import pytest
import torch

from gpu_util import DEV
from linear_attention_recurrent_kda_amd import api

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1, 7, 4096, (1 << 20) + 3, (1 << 23) + 1, (1 << 25) + 13])
def test_copy_probe_copies_everything(n):
    src = torch.arange(n, dtype=torch.float32, device=DEV)
    dst = torch.full_like(src, -1.0)
    api.kda_copy_probe(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


@pytest.mark.parametrize("n", [4099, (1 << 21) + 1029, (1 << 23)])
def test_copy_probe_in_place_keeps_every_element(n):
    buf = torch.arange(n, dtype=torch.float32, device=DEV)
    ref = buf.clone()
    api.kda_copy_probe(buf, buf)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)
