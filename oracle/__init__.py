"""Plain CPU oracle for the FP8 scaled-GEMM path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it. The
GPU library never calls it and shares no code, table or constant with it.

Everything here is slow on purpose: it is the definition of each step written
out in numpy/float64 so that a reader can check it against the pages by eye.

* ``e4m3``  -- the OCP E4M3FN format: decode from bit fields, and the
  saturating round-to-nearest-even cast from fp32.
* ``quant`` -- the per-row (per-token / per-channel) quantizer that turns fp32
  into E4M3 codes plus one fp32 scale per row, and the MXFP8 block quantizer
  (one UE8M0 scale per 32 consecutive K elements) used to build mode-(b) inputs.
* ``gemm``  -- the two GEMM definitions (per-token x per-channel scales, and
  MXFP8 block scales) accumulated in float64, their error bound, and the
  element-by-element parity check.
* ``concat`` -- concat_mla_k, the MLA key assembly (128 nope + 64 rope
  elements per row) on raw 1- or 2-byte elements.

Pins: ``tests/test_oracle_*.py`` hold every check that ties these functions to
something other than themselves (the format definition, torch's own E4M3 cast,
exact rational arithmetic, closed forms, brute force).
"""

from . import e4m3, quant, gemm, concat  # noqa: F401
