"""The decoder's task mapping at the sizes where it changes: one stream of
exactly one full round (sixteen waves of 64 sub-chunks on every CU), one
sub-chunk more (a second round of one run), a ragged size just past it, one
just short of it, and a stream smaller than one run per CU.  A run of 64
sub-chunks lost or decoded twice shows up as a round trip that differs from
the input or as a status flag; the streams themselves are checked against
the oracle elsewhere."""

import pytest

import synth
from oracle import stats

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ec():
    import lossless_entropy_coding_amd as ec
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ec.lib()
    return ec


def _sizes(task_subchunks):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    full = cus * task_subchunks * 256          # one task per CU
    return [full, full + 256, full + 256 + 17, full - 1000, 64 * 256 * 7 + 5]


@pytest.mark.parametrize("name,task", [("huffman", 1024), ("qlc", 1024)])
def test_round_trip_at_task_round_boundaries(ec, name, task):
    counts = [int(c) for c in stats.histogram(synth.draw("ffn1", 100, 1 << 20))]
    cb = ec.Codebook.huffman(counts) if name == "huffman" else ec.Codebook.qlc(counts)
    g = torch.Generator(device=DEV)
    for n in _sizes(task):
        print("case rounds", name, n, flush=True)
        g.manual_seed(n)
        x = (torch.randn(n, device=DEV, generator=g) * 0.5).to(torch.float8_e4m3fn).view(torch.uint8)
        out, out_len, status = ec.encode(cb, x, 16384)
        y, dstatus = ec.decode(cb, out, n, in_len=out.numel())
        torch.cuda.synchronize()
        assert int(status.item()) == 0 and int(dstatus.item()) == 0, n
        assert torch.equal(y, x), n
