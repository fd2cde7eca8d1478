"""The streaming probe (a measurement aid beside the kernels) copies a buffer
bit for bit in copy mode, for sizes that leave a ragged tail after its
unrolled grid-stride loop, and leaves dst alone in read mode."""

import pytest
import torch

import linear_attention_recurrent_gdn_amd as gdn

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [4, 4 * 1000 + 4, 4 * (256 * 2048 * 8) + 4 * 77, 1 << 24])
def test_copy_is_exact_and_read_leaves_dst(n):
    g = torch.Generator(device="cuda").manual_seed(n)
    src = torch.randn(n, device="cuda", generator=g)
    dst = torch.full((n,), 7.0, device="cuda")
    gdn.gdn_stream_probe(src, dst, copy=False)
    torch.cuda.synchronize()
    assert torch.all(dst == 7.0)
    gdn.gdn_stream_probe(src, dst, copy=True)
    torch.cuda.synchronize()
    assert torch.equal(dst.view(torch.int32), src.view(torch.int32))


def test_empty_is_a_no_op():
    src = torch.empty(0, device="cuda")
    dst = torch.zeros(4, device="cuda")
    gdn.gdn_stream_probe(src, dst, copy=True)
    torch.cuda.synchronize()
    assert torch.all(dst == 0.0)
