"""GPU tests of the measurement aids.  moe_stream_read: the sink words are the
XOR of what each lane read, checked against the same fold of the buffer on
the host (every byte of the buffer read once, in place).  moe_mfma_rate: with
every operand 1.0, each MFMA adds its reduction length to every accumulator
element, so each lane's sum has a closed form (exact in fp32 at these sizes).
moe_l2_read_rate: each lane's word is the sum of the pieces its lane pattern
maps it to, recomputed on the host from the same buffer."""
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


def _l2_lane_offsets(pattern: int) -> np.ndarray:
    """Byte offsets in a 64 KB region (16 rows of 4096 bytes) that lane l reads
    across the 64 instructions of one pass: [64 lanes, 64 chunks]."""
    lane, c = np.arange(64)[:, None], np.arange(64)[None, :]
    if pattern == 0:
        return 1024 * c + 16 * lane
    if pattern == 1:
        return (lane % 16) * 4096 + 64 * c + 16 * (lane // 16)
    return (lane // 4) * 4096 + 64 * c + 16 * (lane % 4)


@pytest.mark.parametrize("pattern", [0, 1, 2])
@pytest.mark.parametrize("workgroups,iterations", [(1, 1), (3, 5), (1024, 3)])
def test_l2_read_rate_sums_what_each_lane_reads(pattern, workgroups, iterations):
    """Each lane's word is `iterations` times the sum (mod 2^32) of the 16-byte
    pieces its pattern maps it to, in the region its workgroup and wave read."""
    g = torch.Generator().manual_seed(11 + pattern)
    host = torch.randint(-2**31, 2**31 - 1, (1 << 18,), dtype=torch.int32, generator=g)
    buf = host.to("cuda")
    sink = torch.zeros(workgroups * 256, dtype=torch.int32, device="cuda")
    moe.l2_read_rate(pattern, workgroups, iterations, buf, sink)
    torch.cuda.synchronize()
    words = host.numpy().view(np.uint32).astype(np.uint64)
    offs = _l2_lane_offsets(pattern)                       # [lane, chunk] bytes
    piece = (offs[..., None] // 4 + np.arange(4)).reshape(64, -1)  # word indices in a region
    region_sums = np.stack([words[r * 16384 + piece].sum(axis=1) for r in range(16)])  # [region, lane]
    w = np.arange(workgroups)[:, None, None]
    v = np.arange(4)[None, :, None]
    region = ((w >> 8) & 3) * 4 + v
    want = (region_sums[region, np.arange(64)[None, None, :]] * iterations) % (1 << 32)
    got = sink.cpu().numpy().view(np.uint32).reshape(workgroups, 4, 64)
    assert np.array_equal(got, want.astype(np.uint32))


def test_l2_read_rate_rejects_a_small_buffer():
    buf = torch.zeros((1 << 18) - 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.l2_read_rate(0, 1, 1, buf, sink)
