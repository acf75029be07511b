"""entropy_encode_noalloc (no allocation in the library) against
entropy_encode: the same stream, length and status, on two calls in a row,
the second with a smaller input (the fixed chunk-size array keeps the first
call's contents)."""

import numpy as np
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


def _counts():
    return [int(c) for c in stats.histogram(synth.draw("normal", 1, 1 << 18))]


@pytest.mark.parametrize("codec", ["qlc", "huffman", "eg"])
def test_noalloc_encode_equals_encode(ec, codec):
    counts = _counts()
    cb = {"qlc": lambda: ec.Codebook.qlc(counts), "huffman": lambda: ec.Codebook.huffman(counts),
          "eg": lambda: ec.Codebook.exp_golomb(counts, -1)}[codec]()
    # first call: 5001 chunks of 256 (more than one launch places), then a
    # smaller input with larger chunks
    for n, C, seed in [(5000 * 256 + 77, 256, 21), (100_001, 4096, 22)]:
        print("case %s n=%d C=%d" % (codec, n, C), flush=True)
        x = torch.from_numpy(synth.draw("ffn1", seed, n)).to(DEV)
        ref, ref_len, ref_status = ec.encode(cb, x, C)
        cap = ref.numel()
        out = torch.full((cap,), 0xAB, dtype=torch.uint8, device=DEV)
        out_len = torch.zeros(1, dtype=torch.int64, device=DEV)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        ec.encode_noalloc(cb, x, C, out, out_len, status)
        torch.cuda.synchronize()
        L = int(ref_len.item())
        assert int(status.item()) == int(ref_status.item()) == 0
        assert int(out_len.item()) == L
        assert torch.equal(out[:L], ref[:L])
        y, st = ec.decode(cb, out[:L], n)
        torch.cuda.synchronize()
        assert int(st.item()) == 0 and torch.equal(y, x)


def test_noalloc_encode_rejects_what_it_cannot_do_without_allocating(ec):
    counts = _counts()
    fresh = ec.Codebook.qlc(counts)          # never used on the GPU: no device tables yet
    x = torch.from_numpy(synth.draw("ffn1", 23, 4096)).to(DEV)
    out = torch.empty(1 << 16, dtype=torch.uint8, device=DEV)
    out_len = torch.zeros(1, dtype=torch.int64, device=DEV)
    with pytest.raises(ec.ECError, match="invalid argument"):
        ec.encode_noalloc(fresh, x, 4096, out, out_len)
    cb = ec.Codebook.qlc(counts)
    ec.encode(cb, x, 4096)                   # puts its tables on the device
    torch.cuda.synchronize()
    big = torch.zeros(65536 * 256 + 1, dtype=torch.uint8, device=DEV)   # 65537 chunks of 256
    with pytest.raises(ec.ECError, match="unsupported"):
        ec.encode_noalloc(cb, big, 256, out, out_len)
    ec.encode_noalloc(cb, x, 4096, out, out_len)
    torch.cuda.synchronize()
