"""Pins for the BF16 exponent-coding oracle (ZipCCL page, methodology A-C).

The bit split is checked exhaustively against torch's own bfloat16 values;
the exponent octave masses against their closed-form sum and a Monte Carlo
draw binned by numpy.frexp; the table rule against a lexsort; the page's
"top seven exponents hold over 97%" against the exact Gaussian masses; the
stream against a hand-derived four-value example, round trips and its size
formula.
"""

import math

import numpy as np
import pytest

import synth
from oracle import bf16exp as bx

torch = pytest.importorskip("torch")


def test_split_join_exhaustive_and_matches_bfloat16_values():
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp, sm = bx.split(x)
    assert np.array_equal(bx.join(exp, sm), x)
    # value of every finite, normal pattern from its fields vs torch's bfloat16
    vals = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    e = exp.astype(np.int64)
    s = (sm >> 7).astype(np.int64)
    m = (sm & 0x7F).astype(np.int64)
    normal = (e > 0) & (e < 255)
    want = (-1.0) ** s * np.ldexp(1.0 + m / 128.0, e - 127)
    assert np.array_equal(vals[normal], want[normal])
    sub = e == 0
    assert np.array_equal(vals[sub], ((-1.0) ** s * np.ldexp(m / 128.0, -126))[sub])


def test_table_from_counts_is_a_stable_top_seven():
    rng = np.random.default_rng(3)
    for trial in range(20):
        c = rng.integers(0, 50, 256)
        c[rng.choice(256, 30, replace=False)] = c.max()      # ties at the top
        got = bx.table_from_counts(c)
        want = list(np.lexsort((np.arange(256), -c))[:7])
        assert got == want


def test_octave_masses_sum_to_one_and_match_sampling():
    sigma = 0.37
    total = sum(bx.octave_mass(e, sigma) for e in range(255))
    assert abs(total - 1.0) < 1e-12
    rng = np.random.default_rng(11)
    x = np.abs(rng.standard_normal(1 << 22) * sigma)
    _, k = np.frexp(x)          # x = f * 2^k, f in [0.5, 1): octave [2^(k-1), 2^k)
    e = k - 1 + 127
    freq = np.bincount(e[x > 0], minlength=256) / x.size
    for b in range(110, 130):
        p = bx.octave_mass(b, sigma)
        se = math.sqrt(p * (1 - p) / x.size) + 1e-9
        assert abs(freq[b] - p) < 6 * se, b


def test_top_seven_gaussian_mass_is_about_97_percent():
    # the page: the seven most frequent exponents hold over 97 % of the
    # values; for an exact Gaussian the mass of the best seven octaves
    # depends on log2(sigma) modulo 1 and lies between 96.97 % and 97.88 %
    masses = []
    for f in np.linspace(0, 1, 41)[:-1]:
        for k in (-8, -3, 0, 2):
            s = 2.0 ** (k + f)
            t = bx.table_from_sigma(s)
            assert t == sorted(t, key=lambda e: -bx.octave_mass(e, s))
            assert max(t) - min(t) == 6              # seven adjacent octaves
            masses.append(sum(bx.octave_mass(e, s) for e in t))
    assert 0.9695 < min(masses) < 0.970 and 0.978 < max(masses) < 0.9790
    assert np.mean(masses) > 0.97


def test_sigma_table_equals_counted_table_on_a_gaussian_draw():
    x = synth.bf16_draw(5, 1 << 20, 0.02)
    assert bx.table_from_sigma(0.02) == bx.table_from_counts(bx.exponent_counts(x))


def test_hand_derived_stream():
    # 1.0, -1.0, +0, 3.140625 with exponents 127 and 128 coded 1 and 2
    x = np.array([0x3F80, 0xBF80, 0x0000, 0x4049], dtype=np.uint16)
    table = [127, 128, 126, 125, 124, 123, 122]
    s = bx.encode(x, table, chunk=128)
    n_chunks, sm_at, plane_at, plane_bytes, esc_at = bx.layout(4, 128)
    assert (n_chunks, sm_at, plane_at, plane_bytes, esc_at) == (1, 256, 272, 16, 320)
    assert s[:4] == b"EB16" and len(s) == 321
    assert list(s[sm_at:sm_at + 4]) == [0x00, 0x80, 0x00, 0x49]
    assert s[plane_at] == 0b0011 and s[plane_at + 16] == 0b1000 and s[plane_at + 32] == 0
    assert s[esc_at] == 0x00                      # the zero's exponent, escaped
    assert int.from_bytes(s[32:40], "little") == 1
    assert int.from_bytes(s[72:80], "little") == 1  # esc_off[1]
    assert np.array_equal(bx.decode(s), x)


@pytest.mark.parametrize("n", [0, 1, 127, 128, 16383, 16384, 16385, 50_000])
def test_round_trip_and_size(n):
    rng = np.random.default_rng(n)
    x = synth.bf16_draw(7 + n, n, 0.05)
    if n > 10:
        x[rng.choice(n, n // 10, replace=False)] = rng.integers(0, 1 << 16, n // 10, dtype=np.uint16)
    table = bx.table_from_sigma(0.05)
    s = bx.encode(x, table, chunk=16384)
    exp, _ = bx.split(x)
    n_esc = int((~np.isin(exp, table)).sum())
    assert len(s) == bx.layout(n, 16384)[4] + n_esc
    assert bx.payload_bits(x, table) == 11 * n + 8 * n_esc
    assert np.array_equal(bx.decode(s), x)
