"""Pins for the oracle's stream container and bit-serial encoder/decoders.

The checks do not reuse the encoder's own arithmetic: bit strings are built
here as Python strings from the codebooks, offsets from numpy cumulative
sums, and sizes from sum(count * length).
"""

import os

import numpy as np
import pytest

import synth
from oracle import codebooks as cbm
from oracle import stats
from oracle import stream as st

from _util import deep_counts, padding_flips

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _codebooks(counts):
    return {
        "qlc": cbm.qlc_codebook(counts),
        "qlc_adapted": cbm.qlc_codebook(counts, cbm.QLC_ADAPTED_AREAS, cbm.QLC_ADAPTED_SUFFIX),
        "huffman": cbm.huffman_codebook(counts),
        "eg": cbm.eg_codebook(counts),
        "eg0": cbm.eg_codebook(counts, 0),
        "eg8": cbm.eg_codebook(counts, 8),
    }


def _bitstring_of(x, cb):
    return "".join(format(cb.code[s], "0%db" % cb.length[s]) for s in x)


def _payload_bits(stream_bytes, h, c):
    """Bits of chunk c as a string, in the container's bit order (32-bit LE
    words, most significant bit first)."""
    lo = h["payload_offset"] + int(h["chunk_off"][c])
    hi = h["payload_offset"] + int(h["chunk_off"][c + 1])
    words = np.frombuffer(stream_bytes[lo:hi], dtype="<u4")
    return "".join(format(int(w), "032b") for w in words)


SIZES = [0, 1, 255, 256, 257, 4095, 4096, 4097, 3 * 4096 + 17]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("name", ["qlc", "qlc_adapted", "huffman", "eg", "eg0", "eg8"])
def test_round_trip_and_layout(n, name):
    counts = stats.histogram(synth.draw("normal", 1, 1 << 16))
    cb = _codebooks(counts)[name]
    x = synth.draw("ffn1", 7, n)
    C = 4096
    s = st.encode_stream(x, cb, C)
    h = st.parse_header(s)
    assert h["n"] == n and h["chunk_symbols"] == C and h["codec"] == cb.codec
    assert h["n_chunks"] == -(-n // C)
    assert h["payload_offset"] % 256 == 0
    assert len(s) == h["payload_offset"] + h["payload_bytes"]
    y = st.decode_stream(s, cb)
    assert (y == x).all()
    # per chunk: the payload bit string is the concatenated codes, zero padded;
    # sub-chunk ends are the cumulative code lengths every 256 symbols
    lens = np.array(cb.length, dtype=np.int64)
    for c in range(h["n_chunks"]):
        xs = x[c * C:(c + 1) * C]
        bits = _payload_bits(s, h, c)
        want = _bitstring_of(xs, cb)
        assert bits[:len(want)] == want and set(bits[len(want):]) <= {"0"}
        assert len(bits) == -(-len(want) // 128) * 128
        cum = np.cumsum(lens[xs]) if xs.size else np.zeros(0, np.int64)
        ends = h["sub_end"][c * (C // 256):(c + 1) * (C // 256)]
        for j in range(C // 256):
            k = min((j + 1) * 256, xs.size)
            assert ends[j] == (cum[k - 1] if k > 0 else 0)
    assert sum(len(_bitstring_of(x[c * C:(c + 1) * C], cb)) for c in range(h["n_chunks"])) == \
        cbm.coded_bits(stats.histogram(x), cb.length)


def test_all_symbols_and_repeated_symbol():
    counts = stats.histogram(synth.draw("normal", 1, 1 << 16))
    for cb in _codebooks(counts).values():
        x = np.tile(np.arange(256, dtype=np.uint8), 33)
        assert (st.decode_stream(st.encode_stream(x, cb, 1024), cb) == x).all()
        x = np.full(70000, 0x7E, dtype=np.uint8)
        assert (st.decode_stream(st.encode_stream(x, cb, 16384), cb) == x).all()


@pytest.mark.parametrize("depth", [39, 40, 41])
def test_deep_huffman_codes_round_trip(depth):
    cb = cbm.huffman_codebook(deep_counts(depth))
    assert cb.max_len == depth
    rng = np.random.default_rng(5)
    x = rng.integers(0, 256, 20000).astype(np.uint8)
    x[::97] = np.argmax(cb.length)        # the deepest code appears often
    s = st.encode_stream(x, cb, 4096)
    assert (st.decode_stream(s, cb) == x).all()


def test_embedded_lengths_rebuild_the_codebook():
    x = synth.draw("ffn1", 9, 50000)
    cb = cbm.huffman_codebook(stats.histogram(x))
    s = st.encode_stream(x, cb, 16384, embed_lengths=True)
    h = st.parse_header(s)
    assert h["flags"] == 1 and h["code_len"] == cb.length
    assert (st.decode_stream(s, None) == x).all()


def test_hand_worked_qlc_bits():
    """Three symbols with ranks 0, 1 and 40 under the base scheme code as
    000|000, 000|001 and 101|0000: 19 bits, MSB first in one 32-bit word."""
    counts = np.zeros(256, dtype=np.int64)
    counts[0x10] = 1000         # rank 0
    counts[0x20] = 999          # rank 1
    # ranks 2.. follow byte order among zero counts; find the byte with rank 40
    cb = cbm.qlc_codebook(counts)
    s40 = cb.rank_to_sym[40]
    x = np.array([0x10, 0x20, s40], dtype=np.uint8)
    s = st.encode_stream(x, cb, 256)
    h = st.parse_header(s)
    word = int.from_bytes(s[h["payload_offset"]:h["payload_offset"] + 4], "little")
    assert word == int("000000" "000001" "1010000" + "0" * 13, 2)
    assert h["payload_bytes"] == 16 and list(h["sub_end"]) == [19]
    assert list(h["chunk_off"]) == [0, 16]


def test_empty_stream_layout():
    cb = cbm.qlc_codebook(np.ones(256, dtype=np.int64))
    s = st.encode_stream(np.zeros(0, np.uint8), cb, 16384)
    assert len(s) == 256
    h = st.parse_header(s)
    assert h["n_chunks"] == 0 and list(h["chunk_off"]) == [0] and h["payload_bytes"] == 0
    assert st.decode_stream(s, cb).size == 0


def test_index_size_at_16k_chunks():
    n_chunks, sub_at, _, po = st.layout(1 << 26, 16384)
    assert n_chunks == 4096 and po == 1081600   # 64 + 8*4097 + 4*4096*64, rounded to 256


def test_corruption_is_detected_or_changes_the_output():
    x = synth.draw("normal", 3, 20000)
    counts = stats.histogram(synth.draw("normal", 1, 1 << 16))
    rng = np.random.default_rng(0)
    for cb in _codebooks(counts).values():
        s = bytearray(st.encode_stream(x, cb, 4096))
        h = st.parse_header(bytes(s))
        for _ in range(40):
            pos = h["payload_offset"] + int(rng.integers(0, h["payload_bytes"]))
            t = bytearray(s)
            t[pos] ^= 1 << int(rng.integers(0, 8))
            try:
                y = st.decode_stream(bytes(t), cb)
            except st.CorruptStream:
                continue
            assert not (y == x).all()


def test_a_set_padding_bit_is_corrupt():
    # the container fixes the bits after a chunk's last code as zero
    x = synth.draw("normal", 3, 20000)
    counts = stats.histogram(synth.draw("normal", 1, 1 << 16))
    for name in ("qlc", "huffman", "eg"):
        cb = _codebooks(counts)[name]
        s = st.encode_stream(x, cb, 4096)
        assert (st.decode_stream(s, cb) == x).all()
        flips = padding_flips(s)
        assert len(flips) >= 2
        for _, t in flips:
            with pytest.raises(st.CorruptStream):
                st.decode_stream(t, cb)


def test_header_checks():
    x = synth.draw("normal", 3, 5000)
    counts = stats.histogram(x)
    a = cbm.qlc_codebook(counts)
    b = cbm.huffman_codebook(counts)
    s = st.encode_stream(x, a, 4096)
    with pytest.raises(st.CorruptStream):
        st.decode_stream(s, b)                     # other codebook
    with pytest.raises(st.CorruptStream):
        st.decode_stream(s, a, n=4999)             # wrong length
    t = bytearray(s)
    t[0] ^= 0xFF
    with pytest.raises(st.CorruptStream):
        st.decode_stream(bytes(t), a)              # bad magic


def test_golden_stream_file():
    """A small stream written by tests/golden/make_golden.py (oracle only)."""
    path = os.path.join(GOLDEN, "qlc_tiny_stream.hex")
    meta, hexdata = open(path).read().split("\n", 1)
    fields = dict(kv.split("=") for kv in meta.lstrip("# ").split())
    s = bytes.fromhex("".join(hexdata.split()))
    x = synth.draw("normal", int(fields["seed"]), int(fields["n"]))
    counts = stats.histogram(synth.draw("normal", int(fields["calib_seed"]), int(fields["calib_n"])))
    cb = cbm.qlc_codebook(counts)
    assert st.encode_stream(x, cb, int(fields["chunk"])) == s
    assert (st.decode_stream(s, cb) == x).all()
