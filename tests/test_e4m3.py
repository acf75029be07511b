"""Pins for the e4m3 cast used to build every input (synth.cast_e4m3)."""

import numpy as np
import pytest

import synth


def test_every_finite_code_round_trips():
    b = np.array([v for v in range(256) if (v & 0x7F) != 0x7F], dtype=np.uint8)
    assert b.size == 254
    assert (synth.cast_e4m3(synth.e4m3_value(b)) == b).all()


def test_value_table_spot_checks():
    v = synth.e4m3_value(np.array([0x00, 0x80, 0x01, 0x08, 0x38, 0x7E, 0xFE, 0x7F], dtype=np.uint8))
    assert v[0] == 0.0 and np.signbit(v[1])
    assert v[2] == 2.0 ** -9          # smallest subnormal
    assert v[3] == 2.0 ** -6          # smallest normal
    assert v[4] == 1.0
    assert v[5] == 448.0 and v[6] == -448.0
    assert np.isnan(v[7])


def test_midpoints_round_to_even_mantissa():
    codes = np.arange(0, 0x7E, dtype=np.uint8)          # 0x00..0x7D and their successor
    lo = synth.e4m3_value(codes)
    hi = synth.e4m3_value(codes + 1)
    mid = (lo + hi) / 2                                   # exact in fp64
    got = synth.cast_e4m3(mid)
    want = np.where((codes & 1) == 0, codes, codes + 1).astype(np.uint8)
    assert (got == want).all()
    got_neg = synth.cast_e4m3(-mid)
    assert (got_neg == (want | 0x80)).all()


def test_known_ties():
    x = np.array([1.0625, 3 * 2.0 ** -10, 2.0 ** -10])
    assert list(synth.cast_e4m3(x)) == [0x38, 0x02, 0x00]


def test_saturation_and_signed_zero():
    x = np.array([448.0, 449.0, 464.0, 1e4, np.inf, -470.0, -np.inf, 0.0, -0.0, -1e-12, 1e-12])
    assert list(synth.cast_e4m3(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80, 0x80, 0x00]


def test_matches_torch_on_clamped_fp32():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(123)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 30, 20000), rng.normal(0, 1e-3, 20000)])
    x = np.clip(x.astype(np.float32), -448, 448).astype(np.float64)  # fp32-exact, in range
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (synth.cast_e4m3(x) == ref).all()


def test_generators_are_seeded_and_shaped():
    a = synth.draw("ffn1", 2, 4096)
    b = synth.draw("ffn1", 2, 4096)
    assert a.dtype == np.uint8 and a.shape == (4096,)
    assert (a == b).all()
    g = synth.draw("grad", 4, 1000)   # ragged 128-block tail
    assert g.shape == (1000,)
    s = synth.batch_shards(2, 1024)
    assert s.shape == (2, 1024) and not (s[0] == s[1]).all()
