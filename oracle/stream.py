"""Oracle stream container: header + index + bit-serial payload.

Test infrastructure (see the package docstring).

The pages fix the codes, not a byte format.  This container is the plain one
the library also writes; it is restated here from its definition, not
shared with the library:

    offset  size  field
    0       4     magic 0x53384345 (bytes "EC8S")
    4       2     version = 1
    6       1     codec (1 QLC, 2 Huffman, 3 Exp-Golomb)
    7       1     flags (bit 0: 256 code lengths follow the index)
    8       8     n_symbols
    16      4     chunk_symbols C (multiple of 256)
    20      4     n_chunks = ceil(n / C)
    24      8     payload_offset (multiple of 256)
    32      8     payload_bytes
    40      8     codebook_id (FNV-1a-64 of the codebook description)
    48      16    zero
    64            u64 chunk_off[n_chunks + 1]   byte offset of each chunk in the payload
                  u32 sub_end[n_chunks][C/256]  end bit of each 256-symbol sub-chunk,
                                                from its chunk's start
                  u8  code_len[256]             only if flags bit 0
                  zero bytes up to payload_offset
    payload_offset  payload (see csrc/oracle_codec.c for the bit order)

All integers are little-endian.
"""

from __future__ import annotations

import struct

import numpy as np

from . import _clib
from .codebooks import (EXP_GOLOMB, HUFFMAN, QLC, Codebook, huffman_codebook_from_lengths,
                        huffman_tree)

MAGIC = 0x53384345
VERSION = 1
HEADER = struct.Struct("<IHBBQIIQQQ16x")
assert HEADER.size == 64
FLAG_LENGTHS = 1


class CorruptStream(ValueError):
    pass


def layout(n: int, chunk_symbols: int, embed_lengths: bool = False):
    """(n_chunks, offset of sub_end, offset of code_len or None, payload_offset)."""
    assert chunk_symbols % 256 == 0 and chunk_symbols > 0
    n_chunks = -(-n // chunk_symbols)
    sub_at = 64 + 8 * (n_chunks + 1)
    end = sub_at + 4 * n_chunks * (chunk_symbols // 256)
    len_at = None
    if embed_lengths:
        len_at = end
        end += 256
    payload_offset = -(-end // 256) * 256
    return n_chunks, sub_at, len_at, payload_offset


def encode_payload(x: np.ndarray, cb: Codebook, chunk_symbols: int):
    """Bit-serial encode; returns (payload bytes, chunk_off, sub_end)."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    n = x.size
    n_chunks = -(-n // chunk_symbols)
    subs = chunk_symbols // 256
    code = np.array(cb.code, dtype=np.uint64)
    length = np.array(cb.length, dtype=np.uint8)
    cap = (n * int(max(cb.length)) + 7) // 8 + 16 * n_chunks + 16
    payload = np.zeros(cap, dtype=np.uint8)
    chunk_off = np.zeros(n_chunks + 1, dtype=np.uint64)
    sub_end = np.zeros(max(1, n_chunks * subs), dtype=np.uint32)
    L = _clib.lib()
    got = L.orc_encode(_clib.ptr(x, _clib.ctypes.c_uint8), n, chunk_symbols,
                       _clib.ptr(code, _clib.ctypes.c_uint64), _clib.ptr(length, _clib.ctypes.c_uint8),
                       _clib.ptr(payload, _clib.ctypes.c_uint8), cap,
                       _clib.ptr(chunk_off, _clib.ctypes.c_uint64), _clib.ptr(sub_end, _clib.ctypes.c_uint32))
    assert got != 2 ** 64 - 1
    return payload[:got].copy(), chunk_off, sub_end[: n_chunks * subs]


def encode_stream(x: np.ndarray, cb: Codebook, chunk_symbols: int, embed_lengths: bool = False) -> bytes:
    """The full stream (header, index, payload) for x under codebook cb."""
    n = int(np.asarray(x).size)
    payload, chunk_off, sub_end = encode_payload(x, cb, chunk_symbols)
    n_chunks, sub_at, len_at, payload_offset = layout(n, chunk_symbols, embed_lengths)
    flags = FLAG_LENGTHS if embed_lengths else 0
    head = HEADER.pack(MAGIC, VERSION, cb.codec, flags, n, chunk_symbols, n_chunks,
                       payload_offset, int(payload.size), cb.codebook_id)
    out = bytearray(payload_offset + payload.size)
    out[0:64] = head
    out[64:sub_at] = chunk_off.astype("<u8").tobytes()
    out[sub_at:sub_at + 4 * sub_end.size] = sub_end.astype("<u4").tobytes()
    if embed_lengths:
        out[len_at:len_at + 256] = bytes(int(l) for l in cb.length)
    out[payload_offset:] = payload.tobytes()
    return bytes(out)


def parse_header(stream: bytes) -> dict:
    if len(stream) < 64:
        raise CorruptStream("short header")
    (magic, version, codec, flags, n, C, n_chunks, payload_offset, payload_bytes,
     cb_id) = HEADER.unpack_from(stream, 0)
    h = dict(magic=magic, version=version, codec=codec, flags=flags, n=n, chunk_symbols=C,
             n_chunks=n_chunks, payload_offset=payload_offset, payload_bytes=payload_bytes,
             codebook_id=cb_id)
    if magic != MAGIC or version != VERSION:
        raise CorruptStream("bad magic or version")
    if C == 0 or C % 256:
        raise CorruptStream("bad chunk size")
    nc, sub_at, len_at, po = layout(n, C, bool(flags & FLAG_LENGTHS))
    if nc != n_chunks or po != payload_offset or len(stream) < po + payload_bytes:
        raise CorruptStream("inconsistent header")
    h["chunk_off"] = np.frombuffer(stream, dtype="<u8", count=n_chunks + 1, offset=64).astype(np.uint64)
    h["sub_end"] = np.frombuffer(stream, dtype="<u4", count=n_chunks * (C // 256),
                                 offset=sub_at).astype(np.uint32)
    if flags & FLAG_LENGTHS:
        h["code_len"] = list(stream[len_at:len_at + 256])
    return h


def decode_stream(stream: bytes, cb: Codebook | None, n: int | None = None) -> np.ndarray:
    """Decode a stream with codebook cb (None: rebuild a Huffman codebook from
    the code lengths embedded in the stream)."""
    h = parse_header(stream)
    if cb is None:
        if "code_len" not in h or h["codec"] != HUFFMAN:
            raise CorruptStream("no embedded code lengths")
        cb = huffman_codebook_from_lengths(h["code_len"])
    if h["codec"] != cb.codec or h["codebook_id"] != cb.codebook_id:
        raise CorruptStream("codebook mismatch")
    if n is not None and n != h["n"]:
        raise CorruptStream("length mismatch")
    n = h["n"]
    C = h["chunk_symbols"]
    out = np.zeros(max(n, 1), dtype=np.uint8)
    payload = np.frombuffer(stream, dtype=np.uint8, count=h["payload_bytes"],
                            offset=h["payload_offset"]).copy()
    if payload.size == 0:
        payload = np.zeros(1, dtype=np.uint8)
    chunk_off = np.ascontiguousarray(h["chunk_off"])
    sub_end = np.ascontiguousarray(h["sub_end"]) if h["sub_end"].size else np.zeros(1, np.uint32)
    c = _clib.ctypes
    L = _clib.lib()
    args = (_clib.ptr(payload, c.c_uint8), int(h["payload_bytes"]), _clib.ptr(chunk_off, c.c_uint64),
            _clib.ptr(sub_end, c.c_uint32), n, C)
    if cb.codec == QLC:
        area = np.array(cb.area_size, dtype=np.uint16)
        bits = np.array(cb.suffix_bits, dtype=np.uint8)
        r2s = np.array(cb.rank_to_sym, dtype=np.uint8)
        rc = L.orc_decode_qlc(*args, _clib.ptr(area, c.c_uint16), _clib.ptr(bits, c.c_uint8),
                              _clib.ptr(r2s, c.c_uint8), _clib.ptr(out, c.c_uint8))
    elif cb.codec == HUFFMAN:
        child = np.array(huffman_tree(cb.code, cb.length), dtype=np.int32)
        rc = L.orc_decode_huffman(*args, _clib.ptr(child, c.c_int32), _clib.ptr(out, c.c_uint8))
    elif cb.codec == EXP_GOLOMB:
        r2s = np.array(cb.rank_to_sym, dtype=np.uint8)
        rc = L.orc_decode_eg(*args, cb.k, _clib.ptr(r2s, c.c_uint8), _clib.ptr(out, c.c_uint8))
    else:
        raise CorruptStream("unknown codec")
    if rc != 0:
        raise CorruptStream("payload does not decode")
    return out[:n]
