"""The library's copy kernel (the HBM roofline calibration) copies every byte
(marked gpu): sizes with and without a partial last trip of the unrolled loop."""
import pytest
import torch

import gated_deltanet_chunked_gdn_amd as gdn
from gated_deltanet_chunked_gdn_amd.ops import device_copy

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (1 << 24) + 48, 3 * (1 << 26) + 16 * 257])
def test_device_copy_bitwise(nbytes):
    g = torch.Generator(device="cuda").manual_seed(nbytes % 1000)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    device_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
