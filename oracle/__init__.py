"""Plain CPU oracle for the FP8 scaled-GEMM path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it. The
GPU library never calls it and shares no code, table or constant with it.

Everything here is slow on purpose: it is the definition of each step written
out in numpy/float64 so that a reader can check it against the pages by eye.

* ``e4m3``, ``e5m2`` -- the OCP E4M3FN and E5M2 formats: decode from bit
  fields, and the saturating round-to-nearest-even cast from fp32.
* ``quant`` -- the per-row (per-token / per-channel) and per-tensor quantizers
  that turn fp32 (or bf16) into E4M3 or E5M2 codes plus fp32 scales, and the
  MXFP8 block quantizer (one UE8M0 scale per 32 consecutive K elements).
* ``gemm``  -- the two GEMM definitions (per-token x per-channel scales, and
  MXFP8 block scales) accumulated in float64, their error bound, and the
  element-by-element parity check.
* ``concat`` -- concat_mla_k, the MLA key assembly (128 nope + 64 rope
  elements per row) on raw 1- or 2-byte elements.
* ``cpp_oracle`` (import explicitly; builds with g++) -- the same definitions
  restated in plain C++ (``cpp/fp8_oracle.cpp``), used to check the cast on
  every fp32 pattern and to cross-check the numpy oracle.

Pins: ``tests/test_oracle_*.py`` hold every check that ties these functions to
something other than themselves (the format definition, torch's own E4M3 cast,
exact rational arithmetic, closed forms, brute force).
"""

from . import e4m3, e5m2, quant, gemm, concat  # noqa: F401
