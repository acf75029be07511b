"""Small helpers shared by the tests (no codec arithmetic)."""

import numpy as np


def deep_counts(depth: int) -> np.ndarray:
    """Byte counts whose smoothed (+1) Huffman code has a longest code of
    exactly ``depth`` bits (checked by the tests that use it).

    Symbols 0..m-1 get Fibonacci-scaled counts (a chain in the tree), the
    other 256 - m symbols count 0 and form a balanced subtree of 8 levels
    under the chain's deepest node, so depth = m + 8.
    """
    m = depth - 8
    fib = [1, 1]
    while len(fib) < m + 2:
        fib.append(fib[-1] + fib[-2])
    counts = np.zeros(256, dtype=np.int64)
    for i in range(m):
        counts[i] = fib[i] * 256 - 1
    return counts


# Device codebook table layout (DevTables in csrc/ec_internal.h): byte
# offsets of the fields these tests read.
TABLE_BYTES = 25056
T_ENC64, T_HL1, T_LIMIT, T_SYM, T_CODE_LEN, T_ID = 0, 7168, 23552, 24512, 24768, 25024


def parse_table(b: bytes) -> dict:
    """Fields of a device codebook table (Huffman) as Python values."""
    enc64 = np.frombuffer(b, np.uint64, 256, T_ENC64)
    code_len = list(np.frombuffer(b, np.uint8, 256, T_CODE_LEN))
    codec, max_len = np.frombuffer(b, np.uint32, 2, T_ID + 8)
    return dict(
        code_len=[int(v) for v in code_len],
        code=[int(e) >> (64 - int(l)) if l else 0 for e, l in zip(enc64, code_len)],
        enc_len=[int(e) & 0xFF for e in enc64],
        hl1=np.frombuffer(b, np.uint16, 8192, T_HL1),
        limit=[int(v) for v in np.frombuffer(b, np.uint64, 48, T_LIMIT)],
        sym=list(np.frombuffer(b, np.uint8, 256, T_SYM)),
        codebook_id=int(np.frombuffer(b, np.uint64, 1, T_ID)[0]),
        codec=int(codec), max_len=int(max_len))


def padding_flips(stream: bytes):
    """Copies of a stream with one padding bit set: the first and the last
    padding bit of the first chunk that has padding and of the last chunk.
    Reads only the container's index (header offsets 16-24, chunk_off[],
    sub_end[]); bit p of the payload is bit 31 - p % 32 of 32-bit LE word
    p // 32."""
    n = int(np.frombuffer(stream, "<u8", 1, 8)[0])
    C, n_chunks = (int(v) for v in np.frombuffer(stream, "<u4", 2, 16))
    po = int(np.frombuffer(stream, "<u8", 1, 24)[0])
    spc = C // 256
    chunk_off = np.frombuffer(stream, "<u8", n_chunks + 1, 64).astype(np.int64)
    sub_end = np.frombuffer(stream, "<u4", n_chunks * spc, 64 + 8 * (n_chunks + 1)).astype(np.int64)
    assert n > 0
    out = []
    padded = [c for c in range(n_chunks) if chunk_off[c] * 8 + sub_end[c * spc + spc - 1] < chunk_off[c + 1] * 8]
    for c in sorted({padded[0], padded[-1]} if padded else set()):
        start = int(chunk_off[c] * 8 + sub_end[c * spc + spc - 1])
        for p in (start, int(chunk_off[c + 1] * 8) - 1):
            word, b = divmod(p, 32)
            bitw = 31 - b
            t = bytearray(stream)
            t[po + word * 4 + bitw // 8] ^= 1 << (bitw % 8)
            out.append(((c, p), bytes(t)))
    return out
