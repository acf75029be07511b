"""GPU parity of the batch decoder's task mapping.

Each workgroup takes a range of consecutive workgroup-tasks (16 runs of one
stream), keeps a stream's tables in LDS across its tasks and loads them
again when the next stream has other tables.  The decoded bytes must equal
the oracle's input for every shape: one run in all, ragged last runs, task
counts that do not divide among the workgroups (some take none), one
codebook for all streams and one per stream, calls in a row, two streams at
once, and corrupt segments, which are flagged in their own status word only.
"""

import numpy as np
import pytest

import synth
from oracle import codebooks as cbm
from oracle import stats
from oracle import stream as st

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ec():
    import lossless_entropy_coding_amd as ec
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ec.lib()
    return ec


def _counts(recipe="ffn1", seed=100):
    return [int(c) for c in stats.histogram(synth.draw(recipe, seed, 1 << 18))]


def _codebooks(ec, name, counts):
    if name == "qlc":
        return ec.Codebook.qlc(counts), cbm.qlc_codebook(counts)
    if name == "huffman":
        return ec.Codebook.huffman(counts), cbm.huffman_codebook(counts)
    return ec.Codebook.exp_golomb(counts, -1), cbm.eg_codebook(counts)


def _oracle_batch(x, ocb, C):
    """The oracle's streams of the rows of x, packed at a 16-byte stride."""
    streams = [st.encode_stream(row, ocb, C) for row in x]
    stride = (max(len(s) for s in streams) + 15) // 16 * 16
    buf = np.zeros((len(streams), stride), dtype=np.uint8)
    for i, s in enumerate(streams):
        buf[i, :len(s)] = np.frombuffer(s, dtype=np.uint8)
    return torch.from_numpy(buf).to(DEV)


# (S, seg_n, C): one run in all, ragged last runs, tasks that do not divide
# among the workgroups
SMALL = [(3, 200, 256), (2, 16384, 4096), (5, 70_001, 16384), (9, 3 * 16384 + 4099, 4096), (17, 40_000, 1024)]


@pytest.mark.parametrize("codec", ["qlc", "huffman", "eg"])
@pytest.mark.parametrize("S,seg_n,C", SMALL)
def test_one_codebook_batch_matches_oracle(ec, codec, S, seg_n, C):
    print("case tasks %s S=%d n=%d C=%d" % (codec, S, seg_n, C), flush=True)
    cb, ocb = _codebooks(ec, codec, _counts())
    x = np.stack([synth.draw("ffn1", 300 + s, seg_n) for s in range(S)])
    data = _oracle_batch(x, ocb, C)
    for _ in range(2):   # calls in a row
        y, status = ec.decode_batch(cb, data, seg_n)
        torch.cuda.synchronize()
        assert not status.any()
        assert np.array_equal(y.cpu().numpy(), x)


@pytest.mark.parametrize("codec", ["qlc", "huffman"])
def test_many_tasks_per_workgroup(ec, codec):
    """64 streams of 1 MiB (16384 runs, four tasks per workgroup): one
    codebook object (tables kept) and 64 equal codebook objects (tables
    loaded again at every stream)."""
    print("case tasks 64 x 1 MiB %s" % codec, flush=True)
    counts = _counts()
    cb, _ = _codebooks(ec, codec, counts)
    S, seg_n, C = 64, 1 << 20, 16384
    x = synth.batch_shards(S, seg_n, first_seed=2000)
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    out, lens, status = ec.encode_batch(cb, xd, C)
    torch.cuda.synchronize()
    assert not status.any()
    y, dstatus = ec.decode_batch(cb, out, seg_n)
    others = [_codebooks(ec, codec, counts)[0] for _ in range(S)]
    y2, dstatus2 = ec.decode_batch(others, out, seg_n)
    torch.cuda.synchronize()
    assert not dstatus.any() and not dstatus2.any()
    assert torch.equal(y, xd) and torch.equal(y2, xd)


def test_uneven_task_ranges(ec):
    """100 streams of 768 KiB: 300 workgroup-tasks over 256 workgroups, two
    each for the first 150 and none for the rest; per-stream codebooks."""
    print("case tasks 100 x 768 KiB", flush=True)
    S, seg_n, C = 100, 768 << 10, 4096
    x = synth.batch_shards(S, seg_n, first_seed=3000)
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    cnts = [[int(c) for c in stats.histogram(x[s])] for s in range(S)]
    cbs = [ec.Codebook.huffman(c) for c in cnts]
    out, lens, status = ec.encode_batch(cbs, xd, C)
    torch.cuda.synchronize()
    assert not status.any()
    for s in (0, 57, 99):   # sampled streams against the oracle
        want = st.encode_stream(x[s], cbm.huffman_codebook(cnts[s]), C)
        assert out[s, : int(lens[s].item())].cpu().numpy().tobytes() == want, s
    y, dstatus = ec.decode_batch(cbs, out, seg_n)
    torch.cuda.synchronize()
    assert not dstatus.any() and torch.equal(y, xd)


def test_two_streams_at_once(ec):
    """Two batches decoded concurrently on two streams."""
    cb, ocb = _codebooks(ec, "huffman", _counts())
    S, seg_n, C = 12, 300_000, 4096
    xa = np.stack([synth.draw("ffn1", 400 + s, seg_n) for s in range(S)])
    xb = np.stack([synth.draw("ffn2", 500 + s, seg_n) for s in range(S)])
    xad = torch.from_numpy(xa).to(DEV)
    xbd = torch.from_numpy(xb).to(DEV)
    oa, _, sa = ec.encode_batch(cb, xad, C)
    ob, _, sb = ec.encode_batch(cb, xbd, C)
    torch.cuda.synchronize()
    assert not sa.any() and not sb.any()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ya = torch.empty_like(xad)
    yb = torch.empty_like(xbd)
    for _ in range(4):
        ya.zero_()
        yb.zero_()
        torch.cuda.synchronize()
        _, sta = ec.decode_batch(cb, oa, seg_n, out=ya, stream=s1)
        _, stb = ec.decode_batch(cb, ob, seg_n, out=yb, stream=s2)
        torch.cuda.synchronize()
        assert not sta.any() and not stb.any()
        assert torch.equal(ya, xad) and torch.equal(yb, xbd)


def test_corrupt_segments_are_flagged_alone(ec):
    """A bad header and a flipped payload bit, each in one segment: only
    their status words are set, and the other segments still decode."""
    cb, ocb = _codebooks(ec, "qlc", _counts())
    S, seg_n, C = 11, 50_000, 4096
    x = np.stack([synth.draw("ffn1", 600 + s, seg_n) for s in range(S)])
    data = _oracle_batch(x, ocb, C).cpu().numpy()
    data[3, 0] ^= 1                          # magic
    h = st.parse_header(data[7].tobytes())
    pos = h["payload_offset"] + h["payload_bytes"] // 2
    data[7, pos] ^= 0x10
    d = torch.from_numpy(data).to(DEV)
    y, status = ec.decode_batch(cb, d, seg_n)
    torch.cuda.synchronize()
    st_ = status.cpu().numpy()
    yy = y.cpu().numpy()
    assert st_[3] & ec.S_BAD_HEADER
    assert st_[7] & ec.S_CORRUPT or not np.array_equal(yy[7], x[7])
    for s in range(S):
        if s not in (3, 7):
            assert st_[s] == 0, s
            assert np.array_equal(yy[s], x[s]), s
    # a clean batch after the corrupt one
    y, status = ec.decode_batch(cb, _oracle_batch(x, ocb, C), seg_n)
    torch.cuda.synchronize()
    assert not status.any() and np.array_equal(y.cpu().numpy(), x)
