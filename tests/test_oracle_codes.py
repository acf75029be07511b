"""Pins for the oracle's codebook builders (QLC, Huffman, Exp-Golomb).

Each test checks the oracle against something other than itself: the
scheme the QLC page prints, exact Kraft sums, brute-force optimal code
lengths, the textbook Exp-Golomb table, or an independent second Huffman
construction with a different tie rule.
"""

import itertools
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest

from oracle import codebooks as cbm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _schemes():
    rows = {}
    for line in open(os.path.join(GOLDEN, "qlc_schemes.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, a, n_a, b_a, total = line.split()
        rows.setdefault(name, []).append((int(a), int(n_a), int(b_a), int(total)))
    return rows


def _random_counts(seed, zeros=0):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 10000, 256)
    if zeros:
        c[rng.choice(256, zeros, replace=False)] = 0
    return c


def _is_prefix_free(code, length):
    words = sorted(format(c, "0%db" % l) for c, l in zip(code, length) if l > 0)
    return all(not words[i + 1].startswith(words[i]) for i in range(len(words) - 1))


# --------------------------------------------------------------------- QLC

@pytest.mark.parametrize("scheme", ["base", "adapted"])
def test_qlc_scheme_matches_page(scheme):
    rows = _schemes()[scheme]
    areas = tuple(r[1] for r in rows)
    bits = tuple(r[2] for r in rows)
    want_areas, want_bits = ((cbm.QLC_BASE_AREAS, cbm.QLC_BASE_SUFFIX) if scheme == "base"
                             else (cbm.QLC_ADAPTED_AREAS, cbm.QLC_ADAPTED_SUFFIX))
    assert areas == want_areas and bits == want_bits
    assert sum(areas) == 256
    cb = cbm.qlc_codebook(_random_counts(1), areas, bits)
    # every rank in area a gets the page's total length 3 + suffix bits
    r = 0
    for a, n_a, b_a, total in rows:
        assert total == 3 + b_a
        for off in range(n_a):
            s = cb.rank_to_sym[r]
            assert cb.length[s] == total
            assert cb.code[s] >> b_a == a           # the prefix is the area code
            assert cb.code[s] & ((1 << b_a) - 1) == off
            r += 1
    if scheme == "base":
        assert sorted(set(cb.length)) == [6, 7, 8, 11]   # four distinct lengths


def test_qlc_kraft_sums_exact():
    base = cbm.qlc_codebook(_random_counts(2))
    adapted = cbm.qlc_codebook(_random_counts(2), cbm.QLC_ADAPTED_AREAS, cbm.QLC_ADAPTED_SUFFIX)
    num, den = cbm.kraft_sum(base.length)
    assert Fraction(num, den) == Fraction(40, 64) + Fraction(16, 128) + Fraction(32, 256) + Fraction(168, 2048)
    assert float(Fraction(num, den)) == 0.95703125
    num, den = cbm.kraft_sum(adapted.length)
    assert float(Fraction(num, den)) == 0.9599609375
    assert _is_prefix_free(base.code, base.length)
    assert _is_prefix_free(adapted.code, adapted.length)


def test_rank_order_and_ties():
    counts = [0] * 256
    counts[7] = 50
    counts[3] = 50          # tie with 7: smaller byte first
    counts[200] = 99
    r2s = cbm.rank_symbols(counts)
    assert r2s[:3] == [200, 3, 7]
    assert r2s[3:] == [s for s in range(256) if s not in (200, 3, 7)]   # zero counts by byte
    cb = cbm.qlc_codebook(counts)
    assert cb.code[200] == 0 and cb.length[200] == 6       # most probable: 000 000


def test_qlc_cost_is_sum_count_times_length():
    counts = _random_counts(3, zeros=40)
    cb = cbm.qlc_codebook(counts)
    by_rank = [int(counts[s]) for s in cb.rank_to_sym]
    lens = [6] * 40 + [7] * 16 + [8] * 32 + [11] * 168
    assert cbm.coded_bits(counts, cb.length) == sum(c * l for c, l in zip(by_rank, lens))


def test_qlc_rejects_bad_layouts():
    with pytest.raises(AssertionError):
        cbm.qlc_codebook(_random_counts(4), (8, 8, 8, 8, 8, 16, 32, 167), cbm.QLC_BASE_SUFFIX)
    with pytest.raises(AssertionError):
        cbm.qlc_codebook(_random_counts(4), (9, 8, 8, 8, 7, 16, 32, 168), cbm.QLC_BASE_SUFFIX)


# ----------------------------------------------------------------- Huffman

def _brute_force_min_cost(w):
    """Minimum sum w_i * l_i over every prefix code on n symbols.

    Every length multiset with Kraft sum <= 1 (lengths 1..n-1 suffice for an
    optimal code) is enumerated; for a fixed multiset the cheapest assignment
    gives the shortest lengths to the largest weights (rearrangement
    inequality), so the minimum over multisets is the optimum over codes.
    """
    n = len(w)
    top = n - 1
    ws = sorted(w, reverse=True)
    best = None
    for ls in itertools.combinations_with_replacement(range(1, n), n):
        if sum(1 << (top - l) for l in ls) <= (1 << top):
            c = sum(a * b for a, b in zip(ws, ls))   # ls ascending, ws descending
            best = c if best is None or c < best else best
    return best


def _other_huffman_cost(w, seed):
    """A second Huffman construction: sorted list, random tie order."""
    rnd = random.Random(seed)
    items = [(x, rnd.random()) for x in w]
    cost = 0
    while len(items) > 1:
        items.sort()
        (a, _), (b, _) = items[0], items[1]
        cost += a + b                 # each merge adds one bit to every leaf below
        items = items[2:] + [(a + b, rnd.random())]
    return cost


@pytest.mark.parametrize("n", [2, 3, 4, 5, 6, 7, 8])
def test_huffman_is_optimal_by_brute_force(n):
    rng = np.random.default_rng(n)
    for trial in range(6):
        w = [int(v) for v in rng.integers(1, 20, n)]
        if trial == 5:
            w = [int(v) for v in rng.geometric(0.4, n)]
        lens = cbm.huffman_lengths(w)
        assert sum(a * b for a, b in zip(w, lens)) == _brute_force_min_cost(w)


def test_huffman_n8_special_weights():
    for w in ([1] * 8, [1, 1, 2, 3, 5, 8, 13, 21], [100, 1, 1, 1, 1, 1, 1, 1]):
        lens = cbm.huffman_lengths(w)
        assert sum(a * b for a, b in zip(w, lens)) == _brute_force_min_cost(w)


@pytest.mark.parametrize("seed", range(6))
def test_huffman_kraft_equality_and_cost_invariant(seed):
    rng = np.random.default_rng(seed)
    w = [int(v) for v in rng.integers(1, 1 << 20, 256)]
    if seed % 2:
        w = [int(v) for v in (rng.geometric(0.05, 256))]
    lens = cbm.huffman_lengths(w)
    num, den = cbm.kraft_sum(lens)
    assert num == den                           # complete code: sum 2^-l == 1 exactly
    cost = sum(a * b for a, b in zip(w, lens))
    for s in range(3):
        assert cost == _other_huffman_cost(w, s)


def test_huffman_entropy_bounds():
    rng = np.random.default_rng(9)
    w = [int(v) for v in rng.integers(1, 1000, 256)]
    lens = cbm.huffman_lengths(w)
    W = sum(w)
    H = -math.fsum(x / W * math.log2(x / W) for x in w)
    mean = sum(a * b for a, b in zip(w, lens)) / W
    assert H <= mean < H + 1


def test_huffman_tie_rule_is_fixed():
    # four equal weights: the leaves-first rule gives a balanced tree
    assert cbm.huffman_lengths([5, 5, 5, 5]) == [2, 2, 2, 2]
    # leaf wins a tie against the internal node of equal weight
    assert cbm.huffman_lengths([1, 1, 2]) == [2, 2, 1]


@pytest.mark.parametrize("depth", [39, 40, 41])
def test_huffman_fibonacci_chain_depth(depth):
    fib = [1, 1]
    while len(fib) < depth + 1:
        fib.append(fib[-1] + fib[-2])
    lens = cbm.huffman_lengths(fib[: depth + 1])
    assert max(lens) == depth
    num, den = cbm.kraft_sum(lens)
    assert num == den


def test_canonical_codes_are_prefix_free_and_ordered():
    rng = np.random.default_rng(11)
    cb = cbm.huffman_codebook(rng.integers(0, 5000, 256))
    assert _is_prefix_free(cb.code, cb.length)
    order = sorted(range(256), key=lambda s: (cb.length[s], s))
    left = [cb.code[s] << (64 - cb.length[s]) for s in order]   # left-justified
    assert left == sorted(left) and len(set(left)) == 256
    assert cb.code[order[0]] == 0


def test_canonical_codes_textbook_example():
    # lengths (2, 1, 3, 3) -> B=0, A=10, C=110, D=111 (the usual DEFLATE-style example)
    assert cbm.canonical_codes([2, 1, 3, 3]) == [0b10, 0b0, 0b110, 0b111]


def test_huffman_codebook_smooths_zero_counts():
    counts = [0] * 256
    counts[0x38] = 1000
    cb = cbm.huffman_codebook(counts)
    assert all(l > 0 for l in cb.length)
    assert cb.length[0x38] == 1


# -------------------------------------------------------------- Exp-Golomb

def _bits(v, l):
    return format(v, "0%db" % l)


def test_exp_golomb_k0_textbook_table():
    want = ["1", "010", "011", "00100", "00101", "00110", "00111", "0001000", "0001001"]
    assert [_bits(*cbm.eg_code(r, 0)) for r in range(9)] == want


def test_exp_golomb_k1_and_k2():
    assert [_bits(*cbm.eg_code(r, 1)) for r in range(6)] == ["10", "11", "0100", "0101", "0110", "0111"]
    assert [_bits(*cbm.eg_code(r, 2)) for r in range(6)] == ["100", "101", "110", "111", "01000", "01001"]


def test_exp_golomb_lengths_closed_form():
    for k in range(9):
        for r in range(256):
            v, l = cbm.eg_code(r, k)
            m = int(math.floor(math.log2(r + 2 ** k)))
            assert l == 2 * m - k + 1 and v == r + 2 ** k
    assert {cbm.eg_code(r, 8)[1] for r in range(256)} == {9}
    k4 = [cbm.eg_code(r, 4)[1] for r in range(256)]
    assert k4[:16] == [5] * 16 and k4[16:48] == [7] * 32 and k4[48:112] == [9] * 64
    assert k4[112:240] == [11] * 128 and k4[240:] == [13] * 16


def test_exp_golomb_best_order_is_argmin():
    for seed in range(5):
        counts = _random_counts(20 + seed) ** (seed + 1)
        cb = cbm.eg_codebook(counts)
        sizes = []
        for k in range(9):
            sizes.append(sum(int(counts[s]) * cbm.eg_code(r, k)[1] for r, s in enumerate(cb.rank_to_sym)))
        assert cb.k == sizes.index(min(sizes))
        assert _is_prefix_free(cb.code, cb.length)


# Closed-form cases for the best Exp-Golomb order, summed by hand from the
# codeword lengths 2m - k + 1 (m = floor(log2(rank + 2^k))):
#  - 256 equal counts: k = 8 gives 256 x 9 bits; k = 7 gives 128 x 8 + 128 x 10;
#    k = 6 gives 64 x 7 + 128 x 9 + 64 x 11; all 2304, while k = 5 gives
#    32 x 6 + 64 x 8 + 128 x 10 + 32 x 12 = 2368 and k = 4 gives 2496: the
#    three-way tie goes to the smallest order, 6;
#  - one symbol only: its rank-0 codeword has k + 1 bits, so k = 0;
#  - counts 2^(10 - r) on ranks 0..10 (geometric): k = 0 costs
#    1024 + 3 x 768 + 5 x 240 + 7 x 15 = 4633, k = 1 costs
#    2 x 1536 + 4 x 480 + 6 x 31 = 5178, k = 2 costs 3 x 1920 + 5 x 127 = 6395;
#  - equal counts on ranks 0..15: k = 2, 3, 4 all cost 80 per count (k = 1
#    costs 84, k = 5 costs 96): the tie goes to 2;
#  - equal counts on ranks 0..7: k = 1, 2, 3 cost 32 (k = 0 costs 34): 1;
#  - weight 3 on ranks 0..3 and 1 on ranks 4..11: k = 0, 1, 2, 3, 4 cost
#    86, 80, 76, 88, 100: 2, strictly.
EG_CLOSED_FORM = [
    ([5] * 256, 6),
    ([0] * 77 + [1000] + [0] * 178, 0),
    ([2 ** (10 - r) for r in range(11)] + [0] * 245, 0),
    ([1] * 16 + [0] * 240, 2),
    ([1] * 8 + [0] * 248, 1),
    ([3] * 4 + [1] * 8 + [0] * 244, 2),
]


@pytest.mark.parametrize("counts,k", EG_CLOSED_FORM)
def test_exp_golomb_best_order_closed_forms(counts, k):
    assert cbm.eg_best_order(counts) == k
    assert cbm.eg_codebook(counts).k == k


def test_codebook_ids_differ_and_are_stable():
    counts = _random_counts(30)
    a = cbm.qlc_codebook(counts)
    b = cbm.qlc_codebook(counts, cbm.QLC_ADAPTED_AREAS, cbm.QLC_ADAPTED_SUFFIX)
    c = cbm.huffman_codebook(counts)
    d = cbm.eg_codebook(counts, 3)
    ids = {a.codebook_id, b.codebook_id, c.codebook_id, d.codebook_id}
    assert len(ids) == 4
    assert a.codebook_id == cbm.qlc_codebook(counts).codebook_id
    # FNV-1a-64 published test vectors
    assert cbm.fnv1a64(b"") == 0xCBF29CE484222325
    assert cbm.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert cbm.fnv1a64(b"foobar") == 0x85944171F73967E8
