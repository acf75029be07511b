"""Oracle codebook builders: ranking, Quad Length Codes, Huffman, Exp-Golomb.

Test infrastructure (see the package docstring).  Written for a reader who
checks each step against the pages; speed is irrelevant (256 symbols).

A codebook here is a :class:`Codebook`: for every byte value s it gives the
code ``code[s]`` (an integer whose ``length[s]`` low bits are written MSB
first) plus what the matching decoder needs.
"""

from __future__ import annotations

import heapq
from dataclasses import dataclass, field

QLC, HUFFMAN, EXP_GOLOMB = 1, 2, 3

# Base scheme, "Quad Length Codes for Lossless Compression of e4m3",
# section 2 (Methodology): eight areas chosen by a 3-bit prefix; the first
# five hold 8 symbols with 3 suffix bits (6-bit codes), the sixth 16 symbols
# (7 bits), the seventh 32 symbols (8 bits) and the eighth the remaining 168
# symbols with 8 suffix bits (11 bits).
QLC_BASE_AREAS = (8, 8, 8, 8, 8, 16, 32, 168)
QLC_BASE_SUFFIX = (3, 3, 3, 3, 3, 4, 5, 8)

# Adapted scheme for the FFN2-like workload (same page, section 3, case 2:
# the first area shrinks to 2 symbols).  Sizes 2, 4x8, 16, 32 and 174 sum to
# 256; suffix widths 1, 3, 3, 3, 3, 4, 5, 8 give lengths 4/6/7/8/11.
QLC_ADAPTED_AREAS = (2, 8, 8, 8, 8, 16, 32, 174)
QLC_ADAPTED_SUFFIX = (1, 3, 3, 3, 3, 4, 5, 8)


@dataclass
class Codebook:
    codec: int
    code: list                     # [256] code values
    length: list                   # [256] code lengths in bits
    rank_to_sym: list | None = None  # QLC / EG: rank -> byte
    area_size: tuple | None = None   # QLC
    suffix_bits: tuple | None = None  # QLC
    k: int | None = None             # EG order
    codebook_id: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def max_len(self) -> int:
        return max(self.length)


# ---------------------------------------------------------------- utilities

def fnv1a64(data: bytes) -> int:
    """FNV-1a, 64-bit (offset basis 0xcbf29ce484222325, prime 0x100000001b3)."""
    h = 0xCBF29CE484222325
    for b in data:
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def rank_symbols(counts) -> list:
    """Symbols in decreasing probability; equal counts in increasing byte value.

    QLC page, section 2 (LUT implementation): symbols are sorted by decreasing
    probability and given an index 0..255.  The tie-break by byte value is
    the plain reading (the pages do not state one).
    Returns rank_to_sym (rank_to_sym[r] = byte with rank r).
    """
    assert len(counts) == 256
    return sorted(range(256), key=lambda s: (-int(counts[s]), s))


# ---------------------------------------------------------------------- QLC

def qlc_codebook(counts, area_size=QLC_BASE_AREAS, suffix_bits=QLC_BASE_SUFFIX) -> Codebook:
    """Quad Length Code (QLC page, section 2).

    Area a (selected by the 3-bit prefix a) holds area_size[a] consecutive
    ranks and codes them with suffix_bits[a] further bits, so every code in
    the area is 3 + suffix_bits[a] bits long.  The rank r of a symbol in area
    a is coded as prefix a followed by the offset r - first_rank(a) in natural
    binary.
    """
    area_size = tuple(int(v) for v in area_size)
    suffix_bits = tuple(int(v) for v in suffix_bits)
    assert len(area_size) == 8 and len(suffix_bits) == 8
    assert sum(area_size) == 256
    for n_a, b_a in zip(area_size, suffix_bits):
        assert 0 <= b_a <= 8 and n_a <= (1 << b_a)
    rank_to_sym = rank_symbols(counts)
    code = [0] * 256
    length = [0] * 256
    first = 0
    for a in range(8):
        for off in range(area_size[a]):
            s = rank_to_sym[first + off]
            code[s] = (a << suffix_bits[a]) | off
            length[s] = 3 + suffix_bits[a]
        first += area_size[a]
    desc = bytes([QLC])
    for n_a, b_a in zip(area_size, suffix_bits):
        desc += n_a.to_bytes(2, "little") + bytes([b_a])
    desc += bytes(rank_to_sym)
    return Codebook(QLC, code, length, rank_to_sym=rank_to_sym, area_size=area_size,
                    suffix_bits=suffix_bits, codebook_id=fnv1a64(desc))


def qlc_area_cost(sorted_counts, area_size, suffix_bits, prefix_bits=3) -> int:
    """Payload bits of a QLC layout: rank r in area a costs prefix_bits +
    suffix_bits[a] bits, areas taking consecutive ranks in prefix order."""
    bits, r = 0, 0
    for n_a, b_a in zip(area_size, suffix_bits):
        bits += (prefix_bits + b_a) * sum(int(c) for c in sorted_counts[r:r + n_a])
        r += n_a
    return bits


def qlc_optimal_areas(counts, max_lengths=4, n_areas=8, prefix_bits=3, max_suffix=8):
    """QLC layout with the fewest payload bits for these counts.

    The QLC page (section 2) lets the number of symbols per area and the code
    lengths change with the distribution while at most four distinct code
    lengths remain; its closing outlook names a mathematical optimisation of
    exactly these choices as the next step.  Reading taken: with the 3-bit
    prefix (n_areas = 8 areas), choose a suffix width b_a in 0..max_suffix
    and a size n_a <= 2^b_a for every area, sizes summing to the alphabet,
    at most ``max_lengths`` distinct lengths among non-empty areas, to
    minimise sum over ranks of count x (prefix_bits + b_area).

    Ranks sorted by decreasing count make two moves free of cost: putting
    areas in order of increasing length, and filling an area before any rank
    goes to a longer one.  So some optimum has non-decreasing widths, every
    non-empty area but the last full, and the unused areas (size 0, width 0)
    at the end; this function tries every such layout (the brute-force tests
    over all layouts on small alphabets check the argument) and keeps the
    cheapest, equal costs going to the lexicographically smallest width
    sequence.  Returns (area_size, suffix_bits) as tuples of n_areas values.
    """
    M = len(counts)
    ranked = sorted(range(M), key=lambda s: (-int(counts[s]), s))
    sc = [int(counts[s]) for s in ranked]
    best = None

    def walk(widths, used):
        nonlocal best
        if used >= M:
            sizes = [1 << b for b in widths]
            sizes[-1] = M - sum(sizes[:-1])
            cost = qlc_area_cost(sc, sizes, widths, prefix_bits)
            key = (cost, tuple(widths))
            if best is None or key < best[0]:
                pad = n_areas - len(widths)
                best = (key, tuple(sizes) + (0,) * pad, tuple(widths) + (0,) * pad)
            return
        if len(widths) == n_areas:
            return
        lo = widths[-1] if widths else 0
        for b in range(lo, max_suffix + 1):
            if len(set(widths + [b])) <= max_lengths:
                walk(widths + [b], used + (1 << b))

    walk([], 0)
    assert best is not None, "no layout covers the alphabet"
    return best[1], best[2]


# ------------------------------------------------------------------ Huffman

def huffman_lengths(weights) -> list:
    """Huffman code lengths for positive weights (QLC page, section 1;
    single-stage Huffman page, abstract: the codebook is a Huffman code).

    Repeatedly merge the two lightest nodes.  Ties follow one fixed rule so
    that the result is reproducible: the key is (weight, kind, index) with
    leaves (kind 0, index = symbol) before internal nodes (kind 1, index =
    creation order).  The length of a symbol is the depth of its leaf.
    """
    n = len(weights)
    assert n >= 2 and all(int(w) >= 1 for w in weights)
    heap = [(int(w), 0, s, s) for s, w in enumerate(weights)]  # (w, kind, idx, node)
    heapq.heapify(heap)
    parent = {}
    next_node = n
    created = 0
    while len(heap) > 1:
        w1, _, _, a = heapq.heappop(heap)
        w2, _, _, b = heapq.heappop(heap)
        node = next_node
        next_node += 1
        parent[a] = node
        parent[b] = node
        heapq.heappush(heap, (w1 + w2, 1, created, node))
        created += 1
    lengths = []
    for s in range(n):
        d, v = 0, s
        while v in parent:
            v = parent[v]
            d += 1
        lengths.append(d)
    return lengths


def canonical_codes(lengths) -> list:
    """Canonical prefix code for the given lengths: symbols ordered by
    (length, symbol); the first gets all zeros and each next code is the
    previous one plus one, shifted left by the growth in length."""
    order = sorted((l, s) for s, l in enumerate(lengths) if l > 0)
    codes = [0] * len(lengths)
    code = 0
    prev = None
    for l, s in order:
        if prev is None:
            code = 0
        else:
            code = (code + 1) << (l - prev)
        codes[s] = code
        prev = l
    return codes


def huffman_codebook(counts, smoothing: int = 1) -> Codebook:
    """Huffman codebook over all 256 byte values.

    Every symbol gets weight counts[s] + smoothing (the pages are silent on
    symbols that never occurred; a fixed codebook must still code every later
    shard losslessly, so each symbol needs a codeword).  Codes are canonical.
    """
    weights = [int(c) + smoothing for c in counts]
    lengths = huffman_lengths(weights)
    codes = canonical_codes(lengths)
    cb = Codebook(HUFFMAN, codes, lengths, codebook_id=fnv1a64(bytes([HUFFMAN]) + bytes(lengths)))
    cb.extra["weights"] = weights
    return cb


def huffman_codebook_from_lengths(lengths) -> Codebook:
    codes = canonical_codes(lengths)
    return Codebook(HUFFMAN, codes, list(lengths),
                    codebook_id=fnv1a64(bytes([HUFFMAN]) + bytes(lengths)))


def huffman_tree(code, length):
    """Explicit binary tree of a prefix code, for the bit-serial decoder.

    Returns a flat child array: child[2*node + bit] is the next node, a value
    < 0 is the leaf of symbol -(value+1), and 0 marks a missing branch.
    """
    child = [0, 0]
    nodes = 1
    for s in range(len(length)):
        l = length[s]
        if l == 0:
            continue
        node = 0
        for i in range(l - 1, -1, -1):
            bit = (code[s] >> i) & 1
            if i == 0:
                assert child[2 * node + bit] == 0, "not a prefix code"
                child[2 * node + bit] = -(s + 1)
            else:
                nxt = child[2 * node + bit]
                assert nxt >= 0, "not a prefix code"
                if nxt == 0:
                    nxt = nodes
                    nodes += 1
                    child += [0, 0]
                    child[2 * node + bit] = nxt
                node = nxt
    return child


# -------------------------------------------------------------- Exp-Golomb

def eg_code(rank: int, k: int):
    """Order-k Exp-Golomb codeword of a non-negative integer (the universal
    code the QLC page, section 1, uses as its example).  With v = rank + 2^k
    and m = floor(log2 v): m - k zeros, then v in m + 1 bits.  Returns
    (value, length); the leading zeros are implicit in the length."""
    v = rank + (1 << k)
    m = v.bit_length() - 1
    return v, 2 * m - k + 1


def eg_best_order(counts, rank_to_sym=None, orders=range(0, 9)) -> int:
    """Order k in 0..8 with the fewest coded bits for these counts when
    symbols are coded by rank; ties go to the smaller k."""
    if rank_to_sym is None:
        rank_to_sym = rank_symbols(counts)
    best = None
    for k in orders:
        bits = sum(int(counts[s]) * eg_code(r, k)[1] for r, s in enumerate(rank_to_sym))
        if best is None or bits < best[0]:
            best = (bits, k)
    return best[1]


def eg_codebook(counts, k: int | None = None) -> Codebook:
    """Exp-Golomb on rank: symbols ranked as for QLC, rank coded with order k
    (k = None: the order that minimises the coded size of ``counts``)."""
    rank_to_sym = rank_symbols(counts)
    if k is None:
        k = eg_best_order(counts, rank_to_sym)
    assert 0 <= k <= 8
    code = [0] * 256
    length = [0] * 256
    for r, s in enumerate(rank_to_sym):
        code[s], length[s] = eg_code(r, k)
    desc = bytes([EXP_GOLOMB, k]) + bytes(rank_to_sym)
    return Codebook(EXP_GOLOMB, code, length, rank_to_sym=rank_to_sym, k=k,
                    codebook_id=fnv1a64(desc))


# ---------------------------------------------------------- code properties

def kraft_sum(lengths):
    """Sum of 2^-l over the lengths, exactly, as (numerator, 2^max_len)."""
    L = max(lengths)
    return sum(1 << (L - l) for l in lengths if l > 0), 1 << L


def coded_bits(counts, lengths) -> int:
    """Payload bits of data with these counts: sum over s of count * length."""
    return sum(int(c) * int(l) for c, l in zip(counts, lengths))
