"""CPU oracle for lossless e4m3 entropy coding - TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import or run anything in this package.  The product (the
HIP library under ``lossless_entropy_coding_amd/`` and its binding) never
does; the oracle shares no code, header, table or constant generator with it.

What it computes, each part citing the passage it follows:

* ``codebooks``  rank by decreasing probability, Quad Length Codes (QLC page,
  section 2), Huffman (QLC page section 1; single-stage Huffman page,
  abstract), order-k Exp-Golomb on rank (QLC page section 1).
* ``stream``     the chunked container and the bit-serial encoder/decoders
  (plain C in ``csrc/oracle_codec.c``, driven from Python).
* ``stats``      histogram, PMF, average PMF, entropy and KL divergence
  (single-stage Huffman page, TL;DR, method steps 1-2, figure 3), in fp64.
* ``bf16exp``    exponent coding of BF16 tensors: seven frequent exponents
  in 3-bit codes, the rest escaped (ZipCCL page, methodology A-C).

Every function is pinned by tests in ``tests/test_oracle_*.py`` against
closed forms, brute force, invariants or library routines.  Parity is
unpinned only for the pages' own compression figures, which come from Gemma
tensors that are not available.
"""

from . import bf16exp, codebooks, stats, stream  # noqa: F401
from ._clib import build  # noqa: F401
