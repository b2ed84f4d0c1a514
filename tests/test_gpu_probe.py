"""The read probe reads exactly the blocks it is given: its word sum (mod
2^32) equals the host's sum over the same slots, for contiguous and gathered
blocks, block sizes of one history page and of a whole 4 KB row."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("block_bytes,n_slots,gather", [(1280, 3000, False), (1280, 3000, True), (4096, 517, False),
                                                        (1536, 777, True), (16, 5000, True),
                                                        (16, 600000, False)])
def test_read_probe_sums_the_blocks_it_reads(block_bytes, n_slots, gather):
    import bit_rotated_kv_oscar_amd as oscar
    rng = np.random.default_rng(block_bytes + n_slots)
    host = rng.integers(0, 256, size=n_slots * block_bytes, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    words = host.view(np.uint32).reshape(n_slots, -1).astype(np.uint64)
    if gather:
        ids = rng.permutation(n_slots)[: n_slots // 2 + 7].astype(np.int32)
        ids[3] = n_slots + 10          # outside the buffer: skipped
        ids[5] = -1                    # skipped
        want = int(words[[i for i in ids if 0 <= i < n_slots]].sum()) % (1 << 32)
        sink = oscar.read_probe(buf, len(ids), block_bytes, torch.from_numpy(ids).cuda())
    else:
        want = int(words.sum()) % (1 << 32)
        sink = oscar.read_probe(buf, n_slots, block_bytes)
    torch.cuda.synchronize()
    got = int(sink.cpu().numpy().view(np.uint32)[0])
    assert got == want
