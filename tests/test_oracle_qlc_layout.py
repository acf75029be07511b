"""Pins for the oracle's QLC area-layout search.

The oracle enumerates only layouts of a canonical shape (widths that never
decrease, every non-empty area but the last full); the brute-force tests
here search every layout on small alphabets and must find nothing cheaper,
so a wrong shape argument, a dropped layout or a wrong cost fails them.
Closed forms cover the uniform distribution, a single symbol and the
one-length case; the search can never lose to the page's base and adapted
layouts, which lie inside its space.
"""

import itertools

import numpy as np
import pytest

import synth
from oracle import codebooks as cbm
from oracle import stats


def _brute_force(counts, n_areas, max_suffix, max_lengths, prefix_bits):
    """Cheapest cost over every layout: any widths in any area order, any
    sizes up to 2^width, consecutive ranks per area in prefix order."""
    M = len(counts)
    sc = sorted((int(c) for c in counts), reverse=True)
    best = None
    for widths in itertools.product(range(max_suffix + 1), repeat=n_areas):
        caps = [1 << b for b in widths]

        def sizes(a, left):
            if a == n_areas - 1:
                if left <= caps[a]:
                    yield (left,)
                return
            for n in range(min(caps[a], left) + 1):
                for rest in sizes(a + 1, left - n):
                    yield (n,) + rest

        for sz in sizes(0, M):
            if len({b for b, n in zip(widths, sz) if n}) > max_lengths:
                continue
            cost = cbm.qlc_area_cost(sc, sz, widths, prefix_bits)
            if best is None or cost < best:
                best = cost
    return best


def _check_layout(counts, layout, n_areas, max_suffix, max_lengths):
    sizes, widths = layout
    assert len(sizes) == len(widths) == n_areas
    assert sum(sizes) == len(counts)
    for n, b in zip(sizes, widths):
        assert 0 <= b <= max_suffix and 0 <= n <= (1 << b)
    assert len({b for b, n in zip(widths, sizes) if n}) <= max_lengths


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("max_lengths", [1, 2, 4])
def test_layout_search_matches_brute_force(seed, max_lengths):
    rng = np.random.default_rng(seed)
    M = 10
    counts = [int(v) for v in rng.integers(0, 50, M)]
    if seed % 3 == 0:
        counts[rng.integers(0, M)] = 0      # zero counts and ties
        counts[1] = counts[2]
    layout = cbm.qlc_optimal_areas(counts, max_lengths, n_areas=4, prefix_bits=2, max_suffix=3)
    _check_layout(counts, layout, 4, 3, max_lengths)
    got = cbm.qlc_area_cost(sorted(counts, reverse=True), *layout, prefix_bits=2)
    assert got == _brute_force(counts, 4, 3, max_lengths, 2)


def test_layout_search_matches_brute_force_skewed():
    counts = [1000, 300, 299, 60, 50, 9, 8, 2, 1, 1, 0]
    for L in (1, 2, 3, 4):
        layout = cbm.qlc_optimal_areas(counts, L, n_areas=4, prefix_bits=2, max_suffix=3)
        got = cbm.qlc_area_cost(sorted(counts, reverse=True), *layout, prefix_bits=2)
        assert got == _brute_force(counts, 4, 3, L, 2)


def test_uniform_counts_give_eight_areas_of_32():
    # every layout averages at least 5 suffix bits per symbol here (each area
    # holds at most 2^width symbols), and 8 x 32 reaches it
    assert cbm.qlc_optimal_areas([7] * 256, 4) == ((32,) * 8, (5,) * 8)
    assert cbm.qlc_optimal_areas([7] * 256, 8) == ((32,) * 8, (5,) * 8)


def test_single_symbol_costs_three_bits():
    counts = [0] * 256
    counts[0x42] = 12345
    sizes, widths = cbm.qlc_optimal_areas(counts, 4)
    # the symbol alone in a 3-bit area; the cheapest tie in lexicographic
    # order keeps widths 0 while seven areas cannot yet hold 256 symbols
    assert (sizes, widths) == ((1,) * 7 + (249,), (0,) * 7 + (8,))
    cb = cbm.qlc_codebook(counts, sizes, widths)
    assert cb.length[0x42] == 3


def test_one_length_is_eight_bits():
    rng = np.random.default_rng(5)
    counts = [int(v) for v in rng.integers(0, 1000, 256)]
    assert cbm.qlc_optimal_areas(counts, 1) == ((32,) * 8, (5,) * 8)


@pytest.mark.parametrize("recipe", ["normal", "ffn1", "ffn2", "grad"])
def test_search_never_loses_to_the_page_layouts(recipe):
    counts = [int(c) for c in stats.histogram(synth.draw(recipe, 11, 1 << 18))]
    sc = sorted(counts, reverse=True)
    base = cbm.qlc_area_cost(sc, cbm.QLC_BASE_AREAS, cbm.QLC_BASE_SUFFIX)
    adapted = cbm.qlc_area_cost(sc, cbm.QLC_ADAPTED_AREAS, cbm.QLC_ADAPTED_SUFFIX)
    quad = cbm.qlc_area_cost(sc, *cbm.qlc_optimal_areas(counts, 4))
    free = cbm.qlc_area_cost(sc, *cbm.qlc_optimal_areas(counts, 8))
    assert quad <= base                      # base has four lengths
    assert free <= min(quad, adapted)        # adapted has five
    # the layout's cost is the coded size of its codebook
    cb = cbm.qlc_codebook(counts, *cbm.qlc_optimal_areas(counts, 4))
    assert cbm.coded_bits(counts, cb.length) == quad
