"""The read-bandwidth calibration kernel (hsa_stream_read) reads every 16-byte word
of its source once, each lane folding its own words: a 128-bit value planted once in
each lane's stream makes every lane's fold equal the kernel's store trigger, and the
sink then holds that value in all 256 slots; an all-zero source leaves the sink alone."""
import pytest
import torch

from helpers import note

pytestmark = pytest.mark.gpu

MAGIC = (0x9e3779b9, 0x7f4a7c15, 0x94d049bb, 0x2545f491)
WG, THREADS, PER_LANE = 512, 256, 8


def _words(t):
    return t.view(torch.int32).view(-1, 4)


@pytest.mark.parametrize("mib,u", [(16, 0), (16, 7), (48, 3)])
def test_stream_read_reads_every_lane_word(mib, u):
    import hybrid_sparse_compressed_amd as hsa

    note("stream_read mib=%d plant u=%d" % (mib, u))
    n16 = (mib << 20) // 16
    rounds = n16 // (WG * THREADS * PER_LANE)
    src = torch.zeros(n16 * 16, dtype=torch.uint8, device="cuda")
    magic = torch.tensor([m - (1 << 32) if m >= 1 << 31 else m for m in MAGIC], dtype=torch.int32,
                         device="cuda")
    w = _words(src)
    g = torch.arange(WG, device="cuda").view(-1, 1)
    t = torch.arange(THREADS, device="cuda").view(1, -1)
    r = rounds - 1  # the plant goes into the last round of each lane's stream
    pos = (g * rounds * THREADS * PER_LANE + r * THREADS * PER_LANE + u * THREADS + t).reshape(-1)
    w[pos] = magic
    sink = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    hsa.hsa_stream_read(src, sink)
    torch.cuda.synchronize()
    assert torch.equal(_words(sink), magic.view(1, 4).expand(THREADS, 4))

    sink.fill_(0x5a)
    hsa.hsa_stream_read(torch.zeros(16 << 20, dtype=torch.uint8, device="cuda"), sink)
    torch.cuda.synchronize()
    assert bool((sink == 0x5a).all())
