"""Seeded synthetic e4m3 workloads.

This module is the only code shared by the CPU oracle and the GPU path, and it
holds none of the codec arithmetic: it draws fp64 samples with numpy's PCG64
generator, casts them to 8-bit e4m3 bytes and hands the bytes to whoever asks.
Both sides then see identical input bytes.

The pages measure on Gemma-2B e4m3 activation and gradient tensors (QLC page,
section 3; single-stage Huffman page, TL;DR and abstract), which are not
available here.  The recipes below stand in for them:

* ``normal``    - N(0, 1) samples (the tiny base-scheme workload).
* ``ffn1``      - N(0, sigma^2) with a 1 % mixture of N(0, 8^2) outliers,
                  standing in for FFN1 activations.
* ``ffn2``      - 0.25 * GELU(N(0, 1)) (exact erf form), standing in for the
                  FFN2 input with its spike near zero.
* ``grad``      - Laplace(0, 0.02) scaled by 2^(6+e) per 128-element block,
                  e uniform in {-2..2}, standing in for gradients.

For the BF16 exponent codec (ZipCCL page: near-Gaussian training tensors in
BF16), ``bf16_draw`` gives N(0, sigma^2) samples as BF16 bit patterns.

numpy does not promise stream stability across versions, so callers that
record results also record ``numpy.__version__`` and a SHA-256 of the bytes.
"""

from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "E4M3_MAX",
    "cast_e4m3",
    "e4m3_value",
    "draw",
    "workload",
    "calibration_shards",
    "batch_shards",
    "sha256",
    "WORKLOADS",
    "bf16_bits",
    "bf16_draw",
    "BF16_WORKLOAD",
]

E4M3_MAX = 448.0


def cast_e4m3(x: np.ndarray) -> np.ndarray:
    """Cast fp64 values to OCP FP8 E4M3FN bytes, round-half-to-even, saturating.

    Byte layout s.eeee.mmm, exponent bias 7, no infinities, 0x7F/0xFF are NaN,
    largest finite value 448 (0x7E).  Magnitudes >= 448 saturate to +-448.
    The sign of a value that rounds to zero is kept (-tiny -> 0x80).  The cast
    is done straight from fp64: scaling by a power of two is exact there, so
    ``np.rint`` (ties to even) performs the only rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    out = np.zeros(x.shape, dtype=np.uint8)

    sub = a < 2.0 ** -6
    # subnormal grid: multiples of 2^-9; q == 8 lands exactly on 0x08 (2^-6)
    q_sub = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    out[sub] = q_sub.astype(np.uint8)

    norm = (~sub) & (a < E4M3_MAX) & ~np.isnan(a)
    an = a[norm]
    _, ex = np.frexp(an)          # an = f * 2^ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1   # an in [2^e, 2^(e+1))
    q = np.rint(np.ldexp(an, 3 - e)).astype(np.int64)  # in [8, 16]
    carry = q == 16
    q[carry] = 8
    e[carry] += 1
    out[norm] = ((e + 7) * 8 + (q - 8)).astype(np.uint8)

    out[(a >= E4M3_MAX) & ~np.isnan(a)] = 0x7E
    out |= sign
    out[np.isnan(a)] = 0x7F
    return out


def e4m3_value(b: np.ndarray) -> np.ndarray:
    """fp64 value of e4m3 bytes (NaN for 0x7F / 0xFF)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    v = s * v
    v = np.where((b & 0x7F) == 0x7F, np.nan, v)
    return v


# ----------------------------------------------------------------------------
# sample recipes (fp64), in exact draw order
# ----------------------------------------------------------------------------

def _normal(rng: np.random.Generator, n: int, sigma: float = 1.0) -> np.ndarray:
    return rng.normal(0.0, sigma, n)


def _ffn1(rng: np.random.Generator, n: int, sigma: float = 0.5) -> np.ndarray:
    x = rng.normal(0.0, sigma, n)
    m = rng.random(n) < 0.01
    x[m] = rng.normal(0.0, 8.0, int(m.sum()))
    return x


def _erf(x: np.ndarray) -> np.ndarray:
    try:
        from scipy.special import erf
        return erf(x)
    except ImportError:  # pragma: no cover - scipy is present in this image
        return np.vectorize(math.erf, otypes=[np.float64])(x)


def _ffn2(rng: np.random.Generator, n: int) -> np.ndarray:
    x = rng.normal(0.0, 1.0, n)
    return 0.25 * x * 0.5 * (1.0 + _erf(x / math.sqrt(2.0)))


def _grad(rng: np.random.Generator, n: int) -> np.ndarray:
    g = rng.laplace(0.0, 0.02, n)
    nb = (n + 127) // 128
    e = rng.integers(-2, 3, nb)
    g *= np.repeat(2.0 ** (6 + e), 128)[:n]
    return g


_RECIPES = {
    "normal": _normal,
    "ffn1": _ffn1,
    "ffn2": _ffn2,
    "grad": _grad,
}


def draw(recipe: str, seed: int, n: int, **kw) -> np.ndarray:
    """Draw ``n`` e4m3 bytes from ``recipe`` with ``np.random.default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    return cast_e4m3(_RECIPES[recipe](rng, n, **kw))


@dataclass(frozen=True)
class Workload:
    name: str
    recipe: str
    n: int
    seed: int
    calib_recipe: str
    calib_seeds: tuple
    calib_n: int
    chunk_symbols: int
    shape: tuple


# The five workloads, smallest first.  Sizes are bytes (= e4m3 symbols).
WORKLOADS = {
    "tiny_qlc": Workload("tiny_qlc", "normal", 1 << 20, 0, "normal", (1,), 1 << 20, 4096, (1 << 20,)),
    "ffn1": Workload("ffn1", "ffn1", 1 << 26, 2, "ffn1", tuple(range(100, 108)), 1 << 22, 16384, (4096, 16384)),
    "ffn2": Workload("ffn2", "ffn2", 1 << 26, 3, "ffn2", tuple(range(100, 108)), 1 << 22, 16384, (4096, 16384)),
    "grad": Workload("grad", "grad", 1 << 25, 4, "grad", tuple(range(100, 108)), 1 << 22, 16384, (2048, 16384)),
    "batch": Workload("batch", "ffn1", 64 << 22, 1000, "ffn1", tuple(range(100, 108)), 1 << 22, 16384, (64, 1 << 22)),
}


def workload(name: str, n: int | None = None) -> np.ndarray:
    """Data bytes of a named workload (optionally only its first ``n`` draws
    of the same recipe and seed - a smaller stand-in, not a prefix of the
    full draw)."""
    w = WORKLOADS[name]
    if name == "batch":
        return batch_shards(64 if n is None else max(1, n // (1 << 22)), 1 << 22).reshape(-1)
    return draw(w.recipe, w.seed, w.n if n is None else n)


def calibration_shards(name: str, n: int | None = None) -> np.ndarray:
    """Calibration shards of a workload, shape (len(seeds), calib_n)."""
    w = WORKLOADS[name]
    cn = w.calib_n if n is None else n
    return np.stack([draw(w.calib_recipe, s, cn) for s in w.calib_seeds])


def batch_shards(count: int = 64, shard_n: int = 1 << 22, first_seed: int = 1000) -> np.ndarray:
    """Multi-shard batch: shard i uses seed first_seed+i, sigma ~ U(0.4, 0.6)
    drawn first from that shard's generator, then the ffn1 recipe."""
    out = np.empty((count, shard_n), dtype=np.uint8)
    for i in range(count):
        rng = np.random.default_rng(first_seed + i)
        sigma = rng.uniform(0.4, 0.6)
        out[i] = cast_e4m3(_ffn1(rng, shard_n, sigma))
    return out


def sha256(b: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(b).tobytes()).hexdigest()


# ------------------------------------------------------------------- BF16

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 values -> BF16 bit patterns (uint16): to fp32 with numpy's
    round-to-nearest-even cast, then to the upper 16 bits with round half to
    even (finite inputs only)."""
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_draw(seed: int, n: int, sigma: float = 0.02) -> np.ndarray:
    """n BF16 bit patterns of N(0, sigma^2) samples (numpy PCG64, ``seed``)."""
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal(n) * sigma)


# BF16 workload: a 64 MiB weight-like tensor (2^25 values), N(0, 0.02^2),
# seed 5, chunks of 16384 values.
BF16_WORKLOAD = dict(n=1 << 25, seed=5, sigma=0.02, chunk=16384)
