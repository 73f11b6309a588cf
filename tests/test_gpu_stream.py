"""GPU tests of the measurement aids.  moe_stream_read: the sink words are the
XOR of what each lane read, checked against the same fold of the buffer on
the host (every byte of the buffer read once, in place).  moe_mfma_rate: with
every operand 1.0, each MFMA adds its reduction length to every accumulator
element, so each lane's sum has a closed form (exact in fp32 at these sizes)."""
import numpy as np
import pytest
import torch

from top_routing_grouped_amd import moe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mib", [1, 3])
def test_stream_read_folds_every_word(mib):
    n = mib << 18  # int32 words: mib MiB
    g = torch.Generator(device="cuda").manual_seed(1234 + mib)
    buf = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, device="cuda", generator=g)
    sink = torch.full((n * 4 // 1024,), -1, dtype=torch.int32, device="cuda")
    moe.stream_read(buf, sink)
    torch.cuda.synchronize()
    # block b (64 KB) = 64 KB-rows of 64 lanes x 4 words; lane l folds rows 0..63 and its 4 words
    w = buf.cpu().numpy().view(np.uint32).reshape(-1, 64, 64, 4)
    want = np.bitwise_xor.reduce(np.bitwise_xor.reduce(w, axis=3), axis=1).reshape(-1)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)


def test_stream_read_rejects_sizes_off_the_grid():
    buf = torch.zeros(1000, dtype=torch.int32, device="cuda")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.stream_read(buf, sink)


@pytest.mark.parametrize("shape,per_iter", [(0, 8 * 4 * 32), (1, 8 * 16 * 16)])
@pytest.mark.parametrize("workgroups,iterations", [(1, 1), (3, 7), (512, 40), (2, 65535), (1, 65536)])
def test_mfma_rate_sums_every_mfma(shape, per_iter, workgroups, iterations):
    sink = torch.full((workgroups * 256,), -1.0, dtype=torch.float32, device="cuda")
    moe.mfma_rate(shape, workgroups, iterations, sink)
    torch.cuda.synchronize()
    assert torch.all(sink == float(per_iter * iterations)).item()
