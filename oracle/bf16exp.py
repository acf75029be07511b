"""Oracle for exponent coding of BF16 tensors - TEST INFRASTRUCTURE.

Follows "ZipCCL: Efficient Lossless Data Compression of Communication
Collectives for Accelerating LLM Training" (the ZipCCL page), methodology
A and B:

* a BF16 value is split into its sign-and-mantissa bits and its 8-bit
  exponent (B, separation);
* the seven most frequent exponent values get the 3-bit codes 1..7; any
  other exponent gets code 0 and is stored whole, in order, in a separate
  escape ("zero-point") array (B, remapping);
* the seven values can be predicted from the standard deviation alone,
  since the tensors are close to Gaussian (A): here the seven exponents
  whose octaves hold the most Gaussian probability mass.

The container (chunking, bit planes for the codes, index of escape
offsets) is this repository's own format; the page only says that the
codes are kept as three separate 1-bit arrays (C) and that blocks are
padded for wide memory transactions.  Layout, little-endian:

    header, 64 bytes: magic "EB16", version 1, n (u64), chunk values (u32),
        n_chunks (u32), the seven table exponents (u8 x 7), 0, escape count
        (u64), offsets of the sign-mantissa, plane and escape sections (u64 x 3)
    esc_off[n_chunks + 1]  u64: escapes before each chunk (exclusive prefix)
    (zero fill to a multiple of 256)
    sm[n]                  sign << 7 | mantissa of each value
    (zero fill to a multiple of 16)
    plane 0, 1, 2          bit k of value i's code: bit i & 7 of byte i >> 3 of
                           plane k; each plane padded to a multiple of 16 bytes
    esc[escape count]      the exponents coded 0, in value order
"""

from __future__ import annotations

import math
import struct

import numpy as np

MAGIC = b"EB16"
VERSION = 1
HEADER_BYTES = 64
TABLE_SIZE = 7


def split(x_u16: np.ndarray):
    """BF16 bit patterns -> (exponent, sign << 7 | mantissa), as uint8.
    BF16: bit 15 sign, bits 14..7 exponent, bits 6..0 mantissa."""
    x = x_u16.astype(np.uint32)
    exp = ((x >> 7) & 0xFF).astype(np.uint8)
    sm = (((x >> 8) & 0x80) | (x & 0x7F)).astype(np.uint8)
    return exp, sm


def join(exp: np.ndarray, sm: np.ndarray) -> np.ndarray:
    e = exp.astype(np.uint32)
    s = sm.astype(np.uint32)
    return (((s & 0x80) << 8) | (e << 7) | (s & 0x7F)).astype(np.uint16)


def exponent_counts(x_u16: np.ndarray) -> np.ndarray:
    return np.bincount(split(x_u16)[0], minlength=256).astype(np.uint64)


def table_from_counts(counts) -> list:
    """The seven exponents with the largest counts, most frequent first;
    equal counts go to the smaller exponent."""
    order = sorted(range(256), key=lambda e: (-int(counts[e]), e))
    return order[:TABLE_SIZE]


def octave_mass(e: int, sigma: float) -> float:
    """Probability that |x| lies in the octave of BF16 exponent e for
    x ~ N(0, sigma^2): [2^(e-127), 2^(e-126)) for e >= 1, [0, 2^-126) for
    e = 0 (zero and subnormals).  Rounding at the octave edges is ignored."""
    lo = 0.0 if e == 0 else math.ldexp(1.0, e - 127)
    hi = math.ldexp(1.0, e - 126)
    s = sigma * math.sqrt(2.0)
    return math.erf(hi / s) - math.erf(lo / s)


def table_from_sigma(sigma: float) -> list:
    """The seven exponents of the largest Gaussian octave mass for this
    sigma, largest first; equal masses go to the smaller exponent."""
    assert sigma > 0
    order = sorted(range(255), key=lambda e: (-octave_mass(e, sigma), e))
    return order[:TABLE_SIZE]


def _pad(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def layout(n: int, chunk: int):
    """(n_chunks, sm_at, plane_at, plane_bytes, esc_at) of a stream of n values."""
    n_chunks = (n + chunk - 1) // chunk
    idx_end = HEADER_BYTES + 8 * (n_chunks + 1)
    sm_at = _pad(idx_end, 256)
    plane_at = _pad(sm_at + n, 16)
    plane_bytes = _pad((n + 7) // 8, 16)
    esc_at = plane_at + 3 * plane_bytes
    return n_chunks, sm_at, plane_at, plane_bytes, esc_at


def encode(x_u16: np.ndarray, table, chunk: int = 16384) -> bytes:
    """The stream of the values x_u16 (BF16 bit patterns) for this table."""
    table = [int(e) for e in table]
    assert len(table) == TABLE_SIZE and len(set(table)) == TABLE_SIZE
    assert chunk > 0 and chunk % 128 == 0
    x_u16 = np.ascontiguousarray(x_u16, dtype=np.uint16)
    n = int(x_u16.size)
    exp, sm = split(x_u16)
    code = np.zeros(n, dtype=np.uint8)
    for c, e in enumerate(table, start=1):
        code[exp == e] = c
    esc_mask = code == 0
    esc = exp[esc_mask]
    n_chunks, sm_at, plane_at, plane_bytes, esc_at = layout(n, chunk)
    per_chunk = [int(esc_mask[c * chunk:(c + 1) * chunk].sum()) for c in range(n_chunks)]
    esc_off = [0]
    for k in per_chunk:
        esc_off.append(esc_off[-1] + k)
    out = bytearray(esc_at + len(esc))
    struct.pack_into("<4sHHQIIBBBBBBBBQQQQ", out, 0, MAGIC, VERSION, 0, n, chunk, n_chunks,
                     *table, 0, len(esc), sm_at, plane_at, esc_at)
    struct.pack_into("<%dQ" % (n_chunks + 1), out, HEADER_BYTES, *esc_off)
    out[sm_at:sm_at + n] = sm.tobytes()
    for k in range(3):
        bits = ((code >> k) & 1).astype(np.uint8)
        packed = np.packbits(bits, bitorder="little")
        out[plane_at + k * plane_bytes:plane_at + k * plane_bytes + packed.size] = packed.tobytes()
    out[esc_at:] = esc.tobytes()
    return bytes(out)


def decode(stream: bytes) -> np.ndarray:
    """Inverse of encode: the BF16 bit patterns."""
    (magic, version, _, n, chunk, n_chunks, *rest) = struct.unpack_from("<4sHHQIIBBBBBBBBQQQQ", stream, 0)
    table = rest[:TABLE_SIZE]
    n_esc, sm_at, plane_at, esc_at = rest[TABLE_SIZE + 1:]
    assert magic == MAGIC and version == VERSION
    assert (n_chunks, sm_at, plane_at, esc_at) == tuple(layout(n, chunk)[i] for i in (0, 1, 2, 4))
    plane_bytes = layout(n, chunk)[3]
    sm = np.frombuffer(stream, np.uint8, n, sm_at)
    code = np.zeros(n, dtype=np.uint8)
    for k in range(3):
        packed = np.frombuffer(stream, np.uint8, plane_bytes, plane_at + k * plane_bytes)
        code |= np.unpackbits(packed, bitorder="little")[:n] << k
    lut = np.array([0] + list(table), dtype=np.uint8)
    exp = lut[code]
    esc = np.frombuffer(stream, np.uint8, n_esc, esc_at)
    esc_mask = code == 0
    assert int(esc_mask.sum()) == n_esc
    exp[esc_mask] = esc
    return join(exp, sm)


def payload_bits(x_u16: np.ndarray, table) -> int:
    """11 bits a value plus 8 per escape: the coded size without the
    container (sign-mantissa byte, 3-bit code, escaped exponents)."""
    exp, _ = split(np.asarray(x_u16, dtype=np.uint16))
    n_esc = int((~np.isin(exp, np.array(list(table), dtype=np.uint8))).sum())
    return 11 * exp.size + 8 * n_esc
