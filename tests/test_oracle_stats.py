"""Pins for the oracle's statistics: histogram, PMF average, entropy, KL."""

import math
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import synth
from oracle import codebooks as cbm
from oracle import stats


@pytest.mark.parametrize("n", [0, 1, 1000, 123457])
def test_histogram_matches_bincount(n):
    x = synth.draw("ffn2", 11, n)
    h = stats.histogram(x)
    assert h.dtype == np.uint64 and int(h.sum()) == n
    assert (h == np.bincount(x, minlength=256)).all()


def test_average_pmf_of_equal_shards_is_pooled():
    rows = [stats.histogram(synth.draw("ffn1", s, 4096)) for s in range(8)]
    avg = stats.average_pmf(rows)
    pooled = sum(r.astype(np.int64) for r in rows)
    for s in range(256):
        assert avg[s] == pytest.approx(pooled[s] / pooled.sum(), rel=1e-15, abs=1e-18)
    assert math.fsum(avg) == pytest.approx(1.0, abs=1e-15)


def test_average_pmf_unequal_shards_is_mean_of_pmfs():
    a = [0] * 256
    b = [0] * 256
    a[0] = 1           # P_a = delta_0
    b[1] = 3           # P_b = delta_1, three times the samples
    avg = stats.average_pmf([a, b])
    assert avg[0] == 0.5 and avg[1] == 0.5     # mean of PMFs, not pooled counts (0.25/0.75)


def test_entropy_closed_forms():
    assert stats.entropy_bits([1] * 256) == pytest.approx(8.0, abs=1e-12)
    one = [0] * 256
    one[5] = 77
    assert stats.entropy_bits(one) == 0.0
    two = [0] * 256
    two[0], two[1] = 1, 3
    H = -(0.25 * math.log2(0.25) + 0.75 * math.log2(0.75))
    assert stats.entropy_bits(two) == pytest.approx(H, rel=1e-15)
    assert stats.ideal_compression_pct([1] * 256) == pytest.approx(0.0, abs=1e-10)


def test_huffman_mean_length_within_one_bit_of_entropy():
    counts = stats.histogram(synth.draw("ffn1", 2, 1 << 16))
    cb = cbm.huffman_codebook(counts)
    w = cb.extra["weights"]            # the code is optimal for these weights
    W = sum(w)
    H = stats.entropy_bits(w)
    mean = sum(a * b for a, b in zip(w, cb.length)) / W
    assert H <= mean < H + 1


def test_kl_zero_for_equal_and_nonnegative():
    p = stats.histogram(synth.draw("ffn1", 3, 1 << 16))
    assert stats.kl_bits(p, p) == pytest.approx(0.0, abs=1e-15)
    assert stats.kl_bits(p, 4 * p) == pytest.approx(0.0, abs=1e-15)
    rng = np.random.default_rng(1)
    for _ in range(20):
        a = rng.integers(0, 100, 256)
        b = rng.integers(1, 100, 256)
        assert stats.kl_bits(a, b) >= 0.0


def test_kl_two_point_closed_form():
    for p, q in [(0.3, 0.4), (0.01, 0.02), (0.5, 0.5 + 1e-3), (0.9, 0.1)]:
        Pn = 10 ** 6
        pc = [0] * 256
        qc = [0] * 256
        pc[0], pc[1] = round(p * Pn), Pn - round(p * Pn)
        qc[0], qc[1] = round(q * Pn), Pn - round(q * Pn)
        P0, Q0 = pc[0] / Pn, qc[0] / Pn
        want = P0 * math.log2(P0 / Q0) + (1 - P0) * math.log2((1 - P0) / (1 - Q0))
        assert stats.kl_bits(pc, qc) == pytest.approx(want, rel=1e-10)


def test_kl_exact_rational_inputs_high_precision():
    mpmath.mp.dps = 50
    rng = np.random.default_rng(7)
    for trial in range(5):
        p = [int(v) for v in rng.integers(0, 50, 256)]
        q = [int(v) for v in rng.integers(0, 50, 256)]
        Np = sum(p)
        Nq = sum(q) + 256
        want = mpmath.mpf(0)
        for s in range(256):
            if p[s]:
                P = Fraction(p[s], Np)
                Q = Fraction(q[s] + 1, Nq)
                want += mpmath.mpf(P.numerator) / P.denominator * mpmath.log(
                    mpmath.mpf((P / Q).numerator) / (P / Q).denominator, 2)
        assert stats.kl_bits(p, q, q_add=1) == pytest.approx(float(want), rel=1e-12)


def test_kl_exact_with_counts_beyond_2_to_31():
    # totals past 2^31 (the device kernel takes another branch there)
    mpmath.mp.dps = 60
    rng = np.random.default_rng(8)
    for trial in range(3):
        q = [int(v) for v in rng.integers(1 << 30, 1 << 34, 256)]
        p = [int(v + rng.integers(-(1 << 20), 1 << 20)) for v in q]
        Np, Nq = sum(p), sum(q)
        assert Np >= 1 << 31 and Nq >= 1 << 31
        want = mpmath.mpf(0)
        for s in range(256):
            want += mpmath.mpf(p[s]) / Np * mpmath.log((mpmath.mpf(p[s]) * Nq) / (mpmath.mpf(q[s]) * Np), 2)
        assert want > 0
        # (fp64 rounding of the plain sum limits the agreement at such small divergences)
        assert stats.kl_bits(p, q) == pytest.approx(float(want), rel=1e-7)


def test_kl_infinite_when_q_has_a_hole():
    p = [1] * 256
    q = [1] * 256
    q[9] = 0
    assert math.isinf(stats.kl_bits(p, q))
    assert math.isfinite(stats.kl_bits(p, q, q_add=1))


def test_compression_pct():
    assert stats.compression_pct(8 * 100, 100) == 0.0
    assert stats.compression_pct(6 * 100, 100) == 25.0
