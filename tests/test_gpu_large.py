"""A stream beyond 4 GiB: a shard of 5 * 2^30 + 12345 e4m3 bytes, so that
payload positions pass 2^32 bits and the payload itself 2^32 bytes, with
327681 chunks (the encoder's separate offsets launch).  The round trip is
checked on the GPU; the histogram against torch.bincount over pieces; and
sampled chunks (the first, the first whose payload starts beyond 2^32 bits,
the first beyond 2^32 bytes, the last) against the oracle coding that chunk
alone (a chunk's payload and sub-chunk ends do not depend on where it
sits)."""

import numpy as np
import pytest

from oracle import codebooks as cbm
from oracle import stats
from oracle import stream as st

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ec():
    import lossless_entropy_coding_amd as ec
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ec.lib()
    return ec


def test_stream_beyond_four_gib(ec):
    n = 5 * (1 << 30) + 12345
    C = 16384
    print("case large stream n=%d" % n, flush=True)
    x = torch.empty(n, dtype=torch.uint8, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    piece = 1 << 28
    for s in range(0, n, piece):
        m = min(piece, n - s)
        x[s:s + m] = (torch.randn(m, device=DEV, generator=g) * 0.5).to(torch.float8_e4m3fn).view(torch.uint8)

    h = ec.byte_histogram(x)
    want = torch.zeros(256, dtype=torch.int64, device=DEV)
    for s in range(0, n, piece):
        want += torch.bincount(x[s:s + piece].to(torch.int32), minlength=256)
    torch.cuda.synchronize()
    assert torch.equal(h[0], want)

    counts = [int(c) for c in stats.histogram(synth.draw("ffn1", 100, 1 << 20))]
    for name in ("qlc", "huffman"):
        print("case large stream codec %s" % name, flush=True)
        if name == "qlc":
            cb, ocb = ec.Codebook.qlc(counts), cbm.qlc_codebook(counts)
        else:
            cb, ocb = ec.Codebook.huffman(counts), cbm.huffman_codebook(counts)
        out, out_len, status = ec.encode(cb, x, C)
        y, dstatus = ec.decode(cb, out, n, in_len=out.numel())
        torch.cuda.synchronize()
        assert int(status.item()) == 0 and int(dstatus.item()) == 0
        assert torch.equal(y, x)
        del y

        n_chunks, sub_at, _, payload_offset = st.layout(n, C)
        spc = C // 256
        (magic, version, codec, flags, hn, hC, hnch, hpo, hpb, cb_id) = st.HEADER.unpack_from(
            out[:64].cpu().numpy().tobytes(), 0)
        assert magic == st.MAGIC and codec == ocb.codec and cb_id == ocb.codebook_id
        assert (hn, hC, hnch, hpo) == (n, C, n_chunks, payload_offset)
        assert int(out_len.item()) == payload_offset + hpb
        chunk_off = out[64:sub_at].cpu().numpy().view("<u8")
        assert int(chunk_off[-1]) == hpb and hpb > (1 << 32)
        past_bits = int(np.searchsorted(chunk_off, (1 << 32) // 8))   # first chunk starting past 2^32 bits
        past_bytes = int(np.searchsorted(chunk_off, 1 << 32))         # ... past 2^32 bytes
        assert 0 < past_bits < past_bytes < n_chunks
        for k in (0, past_bits, past_bytes, n_chunks - 1):
            xk = x[k * C:min(n, (k + 1) * C)].cpu().numpy()
            pay, co, se = st.encode_payload(xk, ocb, C)
            a, b = int(chunk_off[k]), int(chunk_off[k + 1])
            assert b - a == pay.size, k
            got = out[payload_offset + a:payload_offset + b].cpu().numpy()
            assert np.array_equal(got, pay), k
            ends = out[sub_at + 4 * k * spc:sub_at + 4 * (k + 1) * spc].cpu().numpy().view("<u4")
            assert np.array_equal(ends[:se.size], se), k
        del out
        torch.cuda.empty_cache()
