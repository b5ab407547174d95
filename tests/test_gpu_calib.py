"""The bandwidth calibration kernel moves every byte: a streaming copy equals
its source (sizes with a ragged tail past the unrolled grid-stride body), and
a read-only pass leaves its buffer untouched."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, (1 << 20) + 48, (64 << 20) + 16 * 777])
def test_calib_stream_copy_is_exact(nbytes):
    import long_context_sparse_14_amd as dsa
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    keep = src.clone()
    dsa.calib_stream(src, dst)
    dsa.calib_stream(src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert torch.equal(src, keep)
