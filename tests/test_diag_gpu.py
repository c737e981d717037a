"""GPU check of the diagnostic copy kernel (the byte-counter reference of the
profiles): a plain copy is exact at any size that is a multiple of 16 bytes."""
import pytest
import torch

from w8a8_quantized_speculative_amd import binding
from tests.gpu_helpers import announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48, 64 << 20])
def test_stream_copy_is_exact(nbytes):
    announce("stream_copy", nbytes)
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    binding.quasar_stream_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
