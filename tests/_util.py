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
