"""Plain CPU oracle for the E8-lattice-codebook linear layer.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package. The library under
dequant_e8_codebook_amd/ never imports it and shares no code with it.

Everything here is deliberately slow and literal: float64 unless a step is
defined at a lower precision, numpy/scipy primitives as single steps, no
blocking or fusion. Each function names the passage of the pages it
follows:

  [glq] "glq 0.1.1" (PyPI project page), sections "How it works" (E8 codebook
        of 65536 vectors from the first 7 shells, 16-bit index per 8 weights,
        residual codebook of 8 or 16 more bits, RHT = random sign flips +
        fast Walsh-Hadamard transform), "Bit widths" (table: 16 / 16+8 /
        16+16 bits per 8 weights, global scale only), "Results" (sizes that
        equal the nominal rate), "Acknowledgments" (Conway & Sloane).
  [entropack] the EntroPack news item: storage rate separate from compute
        precision; GPU fused decode + weight reconstruction; actual_bpp
        includes metadata.

nearest_bf.c (loaded by cnative.py) is the brute-force nearest-entry
search written out as a plain C loop, used to check the faster numpy search
on large samples.

Readings of points the pages leave open are stated, each under a label
(R1, R2, ...), in the docstring of the module that uses them. Functions
whose result has no independent pin say "parity unpinned" in their
docstring.
"""
from . import e8, rht, glq, ldlq, entropack  # noqa: F401
