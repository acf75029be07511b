"""GPU parity of the one-read encode: byte_histogram_sized makes the chunk
sizes in the histogram's pass over the input, entropy_encode_sized packs
with them.

Counts equal the oracle's histogram; every chunk size equals the oracle's
count of code bits in that chunk (rounded up to 16 bytes); the streams equal
the oracle's byte for byte (and those of the two-pass entropy_encode at
sizes the oracle would take too long for).  Sizes made for another codebook
are flagged; shapes the fused pass does not take are refused.
"""

import numpy as np
import pytest

import synth
from oracle import codebooks as cbm
from oracle import stats
from oracle import stream as st

from _util import deep_counts

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ec():
    import lossless_entropy_coding_amd as ec
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ec.lib()
    return ec


def _counts(recipe="ffn1", seed=1, n=1 << 18):
    return [int(c) for c in stats.histogram(synth.draw(recipe, seed, n))]


def _codebooks(ec, counts):
    """Four codebooks of different codecs: (library, oracle) pairs."""
    return [(ec.Codebook.qlc(counts), cbm.qlc_codebook(counts)),
            (ec.Codebook.huffman(counts), cbm.huffman_codebook(counts)),
            (ec.Codebook.exp_golomb(counts, -1), cbm.eg_codebook(counts)),
            (ec.Codebook.qlc(counts, *ec.QLC_ADAPTED),
             cbm.qlc_codebook(counts, cbm.QLC_ADAPTED_AREAS, cbm.QLC_ADAPTED_SUFFIX))]


def _oracle_sizes(x, ora, C):
    """Chunk sizes in 16-byte units: the oracle's code bits per chunk."""
    L = np.asarray(ora.length, dtype=np.int64)[x]
    n_chunks = (x.size + C - 1) // C
    bits = np.add.reduceat(L, np.arange(0, x.size, C)) if x.size else np.zeros(0, np.int64)
    assert bits.size == n_chunks
    return (bits + 127) // 128


# (recipe, n, C): small launches (16 KiB pieces) and large ones (64 KiB),
# chunks below a wave's kilobyte (every lane adds its own sums) and above,
# a ragged last chunk
CASES = [("ffn1", 16, 256), ("ffn1", 4096 + 16 * 7, 256), ("ffn2", 100_000, 512), ("grad", 65_536 + 16, 1024),
         ("normal", 200_000, 4096), ("ffn1", 1 << 20, 16384), ("ffn2", (5 << 20) + 48, 2048),
         ("ffn1", (32 << 20) + 160, 256), ("grad", 40 << 20, 16384)]


@pytest.mark.parametrize("k", range(len(CASES)))
def test_sizes_and_streams_match_oracle(ec, k):
    recipe, n, C = CASES[k]
    n_cb = (4, 2, 3, 1)[k % 4]   # one or two codebooks: 16-bit length entries; three or four: 32-bit
    print("case sized %s n=%d C=%d codebooks=%d" % (recipe, n, C, n_cb), flush=True)
    pairs = _codebooks(ec, _counts(recipe))[:n_cb]
    x = synth.draw(recipe, 77, n)
    xd = torch.from_numpy(x).to(DEV)
    hist, sizes = ec.byte_histogram_sized(xd, [p[0] for p in pairs], C)
    torch.cuda.synchronize()
    assert np.array_equal(hist.cpu().numpy()[0].astype(np.uint64), stats.histogram(x))
    sz = sizes.cpu().numpy()
    small = n <= (1 << 20)   # the oracle's encoder takes seconds beyond
    for j, (cb, ora) in enumerate(pairs):
        assert np.array_equal(sz[j, 0], _oracle_sizes(x, ora, C)), j
        out, out_len, status = ec.encode_sized(cb, xd, C, sizes[j, 0])
        torch.cuda.synchronize()
        assert int(status.item()) == 0, j
        got = out[: int(out_len.item())].cpu().numpy().tobytes()
        if small:
            assert got == st.encode_stream(x, ora, C), j
        else:
            ref, ref_len, _ = ec.encode(cb, xd, C)
            torch.cuda.synchronize()
            assert got == ref[: int(ref_len.item())].cpu().numpy().tobytes(), j
        y, dstatus = ec.decode(cb, out, n)
        torch.cuda.synchronize()
        assert int(dstatus.item()) == 0 and torch.equal(y, xd), j


@pytest.mark.parametrize("S,seg_n,C", [(3, 50_000, 1024), (64, 1 << 22, 16384), (5, 4096, 256)])
def test_batch_sizes_and_streams(ec, S, seg_n, C):
    print("case sized batch S=%d n=%d C=%d" % (S, seg_n, C), flush=True)
    counts = _counts("ffn1")
    cb_q, cb_h = ec.Codebook.qlc(counts), ec.Codebook.huffman(counts)
    if S == 64:
        x = synth.batch_shards(S, seg_n, first_seed=1000)
    else:
        x = np.stack([synth.draw("ffn1", 500 + s, seg_n) for s in range(S)])
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    hist, sizes = ec.byte_histogram_sized(xd, [cb_q, cb_h], C)
    ref_hist = ec.byte_histogram(xd)
    torch.cuda.synchronize()
    assert torch.equal(hist, ref_hist)
    for j, cb in enumerate([cb_q, cb_h]):
        out, lens, status = ec.encode_batch_sized(cb, xd, C, sizes[j])
        ref, ref_lens, ref_status = ec.encode_batch(cb, xd, C)
        torch.cuda.synchronize()
        assert not status.any() and not ref_status.any()
        assert torch.equal(lens, ref_lens)
        for s in range(S):
            L = int(lens[s].item())
            assert torch.equal(out[s, :L], ref[s, :L]), (j, s)
    if S <= 5:
        ora = cbm.huffman_codebook(counts)
        for s in range(S):
            assert np.array_equal(sizes[1, s].cpu().numpy(), _oracle_sizes(x[s], ora, C)), s


def test_workgroups_of_several_pieces(ec):
    """More than 4096 pieces of 64 KiB: workgroups take several pieces and
    store each piece's sizes before the next (40 segments of 16 MiB)."""
    print("case sized 40 x 16 MiB", flush=True)
    counts = _counts("ffn1")
    cb_q, cb_h = ec.Codebook.qlc(counts), ec.Codebook.huffman(counts)
    S, seg_n, C = 40, 16 << 20, 4096
    x = np.random.default_rng(5).integers(0, 256, (S, seg_n), dtype=np.uint8)
    xd = torch.from_numpy(x).to(DEV)
    hist, sizes = ec.byte_histogram_sized(xd, [cb_q, cb_h], C)
    torch.cuda.synchronize()
    sz = sizes.cpu().numpy()
    h = hist.cpu().numpy()
    oras = [cbm.qlc_codebook(counts), cbm.huffman_codebook(counts)]
    for s in range(S):
        assert np.array_equal(h[s].astype(np.uint64), stats.histogram(x[s])), s
        for j in range(2):
            assert np.array_equal(sz[j, s], _oracle_sizes(x[s], oras[j], C)), (j, s)


def test_empty_input(ec):
    counts = _counts("ffn1")
    cb = ec.Codebook.huffman(counts)
    x = torch.zeros(16, dtype=torch.uint8, device=DEV)[:0]
    hist, sizes = ec.byte_histogram_sized(x, [cb], 4096)
    out, out_len, status = ec.encode_sized(cb, x, 4096, sizes[0, 0])
    torch.cuda.synchronize()
    assert not hist.any() and int(status.item()) == 0
    assert out[: int(out_len.item())].cpu().numpy().tobytes() == st.encode_stream(
        np.zeros(0, np.uint8), cbm.huffman_codebook(counts), 4096)


def test_sizes_of_another_codebook_are_flagged(ec):
    counts = _counts("ffn1")
    cb_q, cb_h = ec.Codebook.qlc(counts), ec.Codebook.huffman(counts)
    x = torch.from_numpy(synth.draw("ffn1", 9, 1 << 16)).to(DEV)
    _, sizes = ec.byte_histogram_sized(x, [cb_q, cb_h], 4096)
    _, _, status = ec.encode_sized(cb_h, x, 4096, sizes[0, 0])   # the QLC sizes
    torch.cuda.synchronize()
    assert int(status.item()) & ec.S_CODEBOOK_MISMATCH


def test_shapes_the_fused_pass_refuses(ec):
    counts = _counts("ffn1")
    cb = ec.Codebook.huffman(counts)
    x = torch.from_numpy(synth.draw("ffn1", 9, 1 << 16)).to(DEV)
    for C in (768, 12288):                      # not a power of two
        with pytest.raises(ec.ECError):
            ec.byte_histogram_sized(x, [cb], C)
    with pytest.raises(ec.ECError):             # not a whole number of 16-byte vectors
        ec.byte_histogram_sized(x[:1000], [cb], 256)
    with pytest.raises(ec.ECError):             # five codebooks
        ec.byte_histogram_sized(x, [cb] * 5, 256)
    _, sizes = ec.byte_histogram_sized(x, [cb], 4096)
    with pytest.raises(ec.ECError):             # chunks of more than 16384 symbols
        ec.encode_sized(cb, x, 32768, sizes[0, 0])
    deep = ec.Codebook.huffman([int(c) for c in deep_counts(30)])
    _, sizes = ec.byte_histogram_sized(x, [deep], 4096)
    with pytest.raises(ec.ECError):             # codes over 26 bits
        ec.encode_sized(deep, x, 4096, sizes[0, 0])
    torch.cuda.synchronize()
