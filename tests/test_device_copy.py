"""kda_device_copy, the streaming-bandwidth reference: a byte-exact copy for
sizes that end inside a block step and for sizes of many block steps."""
import pytest
import torch

import gated_delta_rule_99_amd as kda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16", [1, 255, 1024, 1025, 4096 * 3 + 17, (1 << 22) + 5])
def test_device_copy_is_exact(n16):
    dev = torch.device("cuda")
    g = torch.Generator(device="cpu").manual_seed(n16)
    src = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), dtype=torch.int32, generator=g).to(dev)
    # a guard word after the destination must stay untouched
    buf = torch.full((n16 * 4 + 4,), 7, dtype=torch.int32, device=dev)
    dst = buf[: n16 * 4]
    kda.kda_device_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), src.cpu())
    assert torch.equal(buf[n16 * 4:].cpu(), torch.full((4,), 7, dtype=torch.int32))
