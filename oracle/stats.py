"""Oracle statistics: byte histogram, PMF, average PMF, entropy, KL divergence.

Test infrastructure (see the package docstring).  Floating point is fp64,
sums use ``math.fsum``.
"""

from __future__ import annotations

import math

import numpy as np

from . import _clib


def histogram(x: np.ndarray) -> np.ndarray:
    """counts[s] = number of bytes equal to s (plain C loop), as uint64."""
    x = np.ascontiguousarray(x, dtype=np.uint8).reshape(-1)
    counts = np.zeros(256, dtype=np.uint64)
    buf = x if x.size else np.zeros(1, dtype=np.uint8)
    _clib.lib().orc_histogram(_clib.ptr(buf, _clib.ctypes.c_uint8), x.size,
                              _clib.ptr(counts, _clib.ctypes.c_uint64))
    return counts


def pmf(counts) -> list:
    """P_s = counts[s] / n."""
    n = sum(int(c) for c in counts)
    return [int(c) / n for c in counts]


def average_pmf(count_rows) -> list:
    """Average distribution over shards (single-stage Huffman page, TL;DR and
    method step 2): the mean of the shards' PMFs."""
    rows = [pmf(r) for r in count_rows]
    S = len(rows)
    return [math.fsum(r[s] for r in rows) / S for s in range(256)]


def entropy_bits(counts) -> float:
    """Shannon entropy H = -sum P log2 P in bits per symbol."""
    p = pmf(counts)
    return -math.fsum(v * math.log2(v) for v in p if v > 0)


def ideal_compression_pct(counts) -> float:
    """Shannon-bound compressibility 100 * (1 - H / 8) (single-stage Huffman
    page, TL;DR: compressibility relative to the ideal Shannon bound)."""
    return 100.0 * (1.0 - entropy_bits(counts) / 8.0)


def kl_bits(p_counts, q_counts, q_add: int = 0) -> float:
    """KL divergence D(P || Q) = sum_{P_s > 0} P_s log2(P_s / Q_s), in bits.

    P is the shard's distribution, Q the average the codebook was built from
    (single-stage Huffman page, figure 3: KL divergence of shards from the
    average PMF).  Q_s = (q_s + q_add) / sum(q + q_add).  Infinite when some
    Q_s = 0 < P_s.
    """
    np_ = sum(int(c) for c in p_counts)
    q = [int(c) + q_add for c in q_counts]
    nq = sum(q)
    terms = []
    for s in range(256):
        ps = int(p_counts[s])
        if ps == 0:
            continue
        if q[s] == 0:
            return math.inf
        P = ps / np_
        Q = q[s] / nq
        terms.append(P * math.log2(P / Q))
    return math.fsum(terms)


def compression_pct(coded_bits: int, n: int) -> float:
    """Compression as the pages quote it: 100 * (1 - coded bits / (8 n))."""
    return 100.0 * (1.0 - coded_bits / (8.0 * n))
