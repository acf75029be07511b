"""GPU parity of the device-resident three-stage path: one Huffman codebook
per shard built on the GPU from the shard's histogram row, then batch encode
and decode with those device tables, with no host round trip.

Every device table must equal, byte for byte, the host builder's table for
the same counts (whose format the host tests pin against the oracle), and
its code lengths, codes and id must equal the oracle's Huffman codebook.
Streams must equal the oracle's byte for byte (code lengths embedded) and
decode to the input.  A row whose code would exceed 40 bits must be flagged
and its table must be unusable.
"""

import numpy as np
import pytest

import synth
from oracle import codebooks as cbm
from oracle import stats
from oracle import stream as st

from _util import TABLE_BYTES, deep_counts, parse_table

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ec():
    import lossless_entropy_coding_amd as ec
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ec.lib()
    return ec


def _special_rows():
    rng = np.random.default_rng(7)
    rows = [[0] * 256, [1] * 256, [10 ** 9] + [0] * 255, list(range(256)),
            [int(v) for v in rng.integers(0, 4, 256) * 1000],            # many ties
            [int(v) for v in rng.integers(0, 1 << 40, 256)],             # large counts
            # at and just past the largest counts of the builder's 32-bit merge
            [(1 << 22) - 1] * 256, [(1 << 22) - 1 - 997 * i for i in range(256)], [1 << 22] + [5] * 255,
            [(1 << 23) - 1] * 256, [(1 << 23) - 1 - 997 * i for i in range(256)], [1 << 23] + [5] * 255,
            # weights growing geometrically (the merge takes new nodes at once)
            [int(10 ** 6 * 0.7 ** i) for i in range(256)], [int(10 ** 6 * 0.93 ** i) for i in range(256)]]
    for d in (20, 26, 27, 33, 40, 41, 47):
        rows.append([int(c) for c in deep_counts(d)])
    for s in range(12):
        rows.append([int(c) for c in stats.histogram(synth.draw(["ffn1", "ffn2", "grad", "normal"][s % 4],
                                                                 900 + s, 1 << 16))])
    return rows


def test_device_codebooks_match_host_and_oracle(ec):
    rows = _special_rows()
    S = len(rows)
    counts = torch.tensor(rows, dtype=torch.int64, device=DEV)
    tables, status = ec.build_huffman_device(counts)
    torch.cuda.synchronize()
    assert tables.shape == (S, TABLE_BYTES)
    tb = tables.cpu().numpy()
    stv = status.cpu().numpy()
    for i, row in enumerate(rows):
        ora = cbm.huffman_codebook(row)
        got = tb[i].tobytes()
        if ora.max_len > 40:
            assert stv[i] == ec.S_BAD_CODEBOOK, i
            assert not tb[i].any(), i
            continue
        assert stv[i] == 0, i
        assert got == ec.Codebook.huffman(row).export(), i
        t = parse_table(got)
        assert t["code_len"] == ora.length and t["code"] == ora.code, i
        assert t["codebook_id"] == ora.codebook_id and t["max_len"] == ora.max_len, i


N_SHARD = (5 << 20) + 784   # batch rows are 16-byte strided; the last chunk is ragged


def _shards():
    """Shards of different statistics: realistic e4m3 recipes; two shards
    whose own codes reach 27 and 28 bits (their tables have no 32-bit encode
    entries, so the row-by-row packer takes their chunks), built from the
    deep-chain counts with the surplus given to the chain's heaviest symbol
    (which keeps the depth); a constant shard."""
    n = N_SHARD
    xs = [synth.draw(r, 300 + k, n) for k, r in enumerate(["ffn1", "ffn2", "grad", "normal"])]
    rng = np.random.default_rng(11)
    for d in (27, 28):
        c = deep_counts(d).copy()
        c[d - 9] += n - int(c.sum())
        xs.append(rng.permutation(np.repeat(np.arange(256, dtype=np.uint8), c)))
    xs.append(np.full(n, 0x38, np.uint8))
    return np.stack(xs)


@pytest.mark.parametrize("C", [4096, 16384])
def test_device_three_stage_matches_oracle(ec, C):
    x = _shards()
    S, n = x.shape
    print("case device three-stage C=%d S=%d n=%d" % (C, S, n), flush=True)
    x_d = torch.from_numpy(x).to(DEV)
    hist = ec.byte_histogram(x_d)
    tables, bstatus = ec.build_huffman_device(hist)
    out, lens, estatus = ec.encode_batch_device(tables, x_d, C, embed_lengths=True)
    # the receiver rebuilds each codebook from the lengths its stream carries
    rtables, rstatus = ec.huffman_tables_from_streams(out)
    y, dstatus = ec.decode_batch_device(rtables, out, n)
    torch.cuda.synchronize()
    assert not bstatus.cpu().numpy().any()
    assert not estatus.cpu().numpy().any()
    assert not rstatus.cpu().numpy().any()
    assert not dstatus.cpu().numpy().any()
    assert torch.equal(rtables, tables)
    assert torch.equal(y, x_d)
    h = hist.cpu().numpy()
    L = lens.cpu().numpy()
    deepest = []
    for i in range(S):
        assert np.array_equal(h[i].astype(np.uint64), stats.histogram(x[i])), i
        ora = cbm.huffman_codebook([int(c) for c in h[i]])
        deepest.append(ora.max_len)
        want = st.encode_stream(x[i], ora, C, embed_lengths=True)
        assert int(L[i]) == len(want), i
        assert out[i, : int(L[i])].cpu().numpy().tobytes() == want, i
        assert len(want) <= ec.own_max_encoded_bytes(n, C, True)
    assert deepest[4:6] == [27, 28]


def test_unusable_table_is_flagged(ec):
    """A row whose code would exceed 40 bits: the builder flags it, an encode
    with its table flags it, the decoder rejects the stream; the other rows
    of the same launches are unaffected."""
    C = 4096
    good = [int(c) for c in stats.histogram(synth.draw("ffn1", 5, 1 << 16))]
    rows = [good, [int(c) for c in deep_counts(41)], good]
    tables, bstatus = ec.build_huffman_device(torch.tensor(rows, dtype=torch.int64, device=DEV))
    x = np.stack([synth.draw("ffn1", 10 + i, 3 * C + 80) for i in range(3)])
    x_d = torch.from_numpy(x).to(DEV)
    out, lens, estatus = ec.encode_batch_device(tables, x_d, C)
    y, dstatus = ec.decode_batch_device(tables, out, x.shape[1])
    torch.cuda.synchronize()
    assert bstatus.cpu().numpy().tolist() == [0, ec.S_BAD_CODEBOOK, 0]
    assert estatus.cpu().numpy().tolist() == [0, ec.S_BAD_CODEBOOK, 0]
    assert dstatus.cpu().numpy().tolist() == [0, ec.S_CODEBOOK_MISMATCH, 0]
    ora = cbm.huffman_codebook(good)
    for i in (0, 2):
        want = st.encode_stream(x[i], ora, C)
        assert out[i, : int(lens[i].item())].cpu().numpy().tobytes() == want
        assert torch.equal(y[i], x_d[i])


def test_counts_at_the_64_bit_weight_limit(ec):
    """A count of 2^55 or more could overflow the 64-bit node weights: the
    builder flags the row and leaves its table unusable; a count just below
    builds the host's table."""
    rows = [[1 << 55] + [0] * 255, [(1 << 55) - 1] + [3] * 255, [0] * 255 + [(1 << 60) + 7]]
    tables, status = ec.build_huffman_device(torch.tensor(rows, dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    tb = tables.cpu().numpy()
    assert status.cpu().numpy().tolist() == [ec.S_BAD_CODEBOOK, 0, ec.S_BAD_CODEBOOK]
    assert not tb[0].any() and not tb[2].any()
    assert tb[1].tobytes() == ec.Codebook.huffman(rows[1]).export()
    ora = cbm.huffman_codebook(rows[1])
    assert parse_table(tb[1].tobytes())["code_len"] == ora.length


@pytest.mark.parametrize("codec", ["qlc", "qlc_adapted", "eg", "eg8", "huffman"])
def test_uploaded_host_tables(ec, codec):
    """Host-built codebooks exported and uploaded as a device table array
    serve the device-table entry points like device-built ones."""
    C = 4096
    counts = [int(c) for c in stats.histogram(synth.draw("ffn2", 77, 1 << 16))]
    if codec.startswith("qlc"):
        lay = ec.QLC_ADAPTED if codec == "qlc_adapted" else ec.QLC_BASE
        cbs = [ec.Codebook.qlc(counts, *lay)] * 2
        ocb = cbm.qlc_codebook(counts, *lay)
        cid = ec.CODEC_QLC
    elif codec.startswith("eg"):
        k = 8 if codec == "eg8" else -1
        cbs = [ec.Codebook.exp_golomb(counts, k)] * 2
        ocb = cbm.eg_codebook(counts, None if k < 0 else k)
        cid = ec.CODEC_EXP_GOLOMB
    else:
        cbs = [ec.Codebook.huffman(counts)] * 2
        ocb = cbm.huffman_codebook(counts)
        cid = ec.CODEC_HUFFMAN
    blob = np.frombuffer(b"".join(c.export() for c in cbs), np.uint8)
    tables = torch.from_numpy(blob.copy()).to(DEV).view(2, -1)
    x = np.stack([synth.draw("ffn2", 40 + i, 7 * C + 112) for i in range(2)])
    x_d = torch.from_numpy(x).to(DEV)
    cap = ec.max_encoded_bytes(cbs[0], x.shape[1], C)
    out = torch.empty((2, (cap + 255) // 256 * 256), dtype=torch.uint8, device=DEV)
    out, lens, estatus = ec.encode_batch_device(tables, x_d, C, out=out)
    y, dstatus = ec.decode_batch_device(tables, out, x.shape[1], codec=cid)
    torch.cuda.synchronize()
    assert not estatus.cpu().numpy().any() and not dstatus.cpu().numpy().any()
    assert torch.equal(y, x_d)
    for i in range(2):
        want = st.encode_stream(x[i], ocb, C)
        assert out[i, : int(lens[i].item())].cpu().numpy().tobytes() == want


def test_tables_from_streams(ec):
    """Receiver-side tables: equal to the host builder's tables for the
    oracle's code lengths; a stream without embedded lengths, a stream whose
    lengths are not a complete code and an index past in_len are flagged,
    and their segments do not decode."""
    C = 4096
    rows = [[int(c) for c in stats.histogram(synth.draw(r, 60 + i, 1 << 16))]
            for i, r in enumerate(["ffn1", "grad", "ffn2", "normal"])]
    rows.append([int(c) for c in deep_counts(40)])
    S = len(rows)
    n = 2 * C + 48
    x = np.stack([synth.draw("ffn1", 70 + i, n) for i in range(S)])
    x_d = torch.from_numpy(x).to(DEV)
    tables, _ = ec.build_huffman_device(torch.tensor(rows, dtype=torch.int64, device=DEV))
    cap = ec.max_encoded_bytes(ec.Codebook.huffman(rows[-1]), n, C, True)
    out = torch.zeros((S, (cap + 255) // 256 * 256), dtype=torch.uint8, device=DEV)
    out, lens, estatus = ec.encode_batch_device(tables, x_d, C, embed_lengths=True, out=out)
    torch.cuda.synchronize()
    assert not estatus.cpu().numpy().any()
    good = out.clone()
    # segment 1: lengths that overfill the code space; segment 2: lengths
    # that underfill it; segment 3: flags say no lengths are embedded
    nch = (n + C - 1) // C
    lens_at = 64 + 8 * (nch + 1) + 4 * nch * (C // 256)
    out[1, lens_at + 7] = max(1, int(out[1, lens_at + 7].item()) - 1)
    out[2, lens_at + 9] = int(out[2, lens_at + 9].item()) + 1
    out[3, 7] = 0
    rtables, rstatus = ec.huffman_tables_from_streams(out)
    y, dstatus = ec.decode_batch_device(rtables, out, n)
    torch.cuda.synchronize()
    assert rstatus.cpu().numpy().tolist() == [0, ec.S_BAD_CODEBOOK, ec.S_BAD_CODEBOOK, ec.S_BAD_HEADER, 0]
    d = dstatus.cpu().numpy().tolist()
    assert d[0] == 0 and d[4] == 0 and all(v & ec.S_CODEBOOK_MISMATCH for v in d[1:4])
    rt = rtables.cpu().numpy()
    for i in (0, 4):
        ora = cbm.huffman_codebook(rows[i])
        assert rt[i].tobytes() == ec.Codebook.huffman_from_lengths(ora.length).export()
        assert torch.equal(y[i], x_d[i])
    for i in (1, 2, 3):
        assert not rt[i].any()
    # an index that does not fit in in_len
    _, st_short = ec.huffman_tables_from_streams(good, in_len=lens_at + 255)
    torch.cuda.synchronize()
    assert st_short.cpu().numpy().tolist() == [ec.S_BAD_HEADER] * S
