"""Host side of the library's BF16 exponent coding: its table rules and
stream bound equal the oracle's (no GPU needed)."""

import numpy as np
import pytest

import synth
from oracle import bf16exp as bx


@pytest.fixture(scope="module")
def ec():
    import lossless_entropy_coding_amd as ec
    ec.lib()
    return ec


def test_table_from_sigma_equals_oracle(ec):
    for k in range(-12, 6):
        for f in (0.0, 0.13, 0.5, 0.72, 0.9):
            s = 2.0 ** (k + f)
            assert list(ec.bf16_exp_table_from_sigma(s)) == bx.table_from_sigma(s), s


def test_table_from_counts_equals_oracle(ec):
    rng = np.random.default_rng(4)
    for trial in range(10):
        c = rng.integers(0, 100, 256)
        c[rng.choice(256, 20, replace=False)] = 100
        assert list(ec.bf16_exp_table_from_counts([int(v) for v in c])) == bx.table_from_counts(c)
    x = synth.bf16_draw(9, 1 << 18, 0.3)
    c = bx.exponent_counts(x)
    assert list(ec.bf16_exp_table_from_counts([int(v) for v in c])) == bx.table_from_counts(c)


def test_max_encoded_bytes_is_the_all_escaped_stream(ec):
    for n in (0, 1, 2048, 16385, 1 << 20):
        for chunk in (2048, 16384):
            assert ec.bf16_exp_max_encoded_bytes(n, chunk) == bx.layout(n, chunk)[4] + n
    assert ec.bf16_exp_max_encoded_bytes(100, 1000) == 0      # chunk not a multiple of 2048


def test_bad_arguments(ec):
    with pytest.raises(ec.ECError):
        ec.bf16_exp_table_from_sigma(0.0)
    with pytest.raises(ec.ECError):
        ec.bf16_exp_table_from_sigma(float("nan"))
