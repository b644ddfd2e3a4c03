"""CPU oracle for blockwise-scaled FP8 quantization and GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
header, table or constant with the HIP library: every function here is
written from the definitions in the source pages (and, where the pages are
silent, from the OCP FP8 and IEEE-754 definitions), in plain numpy/Python,
float64 unless a step fixes a narrower precision.

Sources, cited by page title and section:
  [REPRO]  pytorch/ao PR "add repro for blockwise _scaled_mm investigation"
           (What Changed; Findings So Far; review comments).
  [INTEG]  pytorch/ao PR "integrate torch._scaled_mm into Float8BlockwiseLinear
           and add bench script" (Summary; Benchmarks).
  [GENERIC] pytorch/ao PR "add more generic kernel for fp8 blockwise scaling"
           (bullets; Performance table; review thread).
  [AITER]  ROCm/aiter issue "Does gemm_a8w8 support per-tensor quant?"
           (Steps to Reproduce; printed comparison).
  [INDUCT] pytorch/pytorch issue on the inductor FP8 tensorwise test
           (Describe the bug).
  [OCP]    OCP 8-bit Floating Point Specification (OFP8), E4M3 encoding.

Pinning status (what each function is checked against, in tests/):
  e4m3.decode / encode_rne  brute-force nearest-code search, torch CPU
                            float8_e4m3fn cast, OCP special values.
  quant.*                   exact-rational (Fraction) brute force, block
                            invariants, transposition identities.
  gemm.*                    Fraction brute force on tiny shapes, integer
                            arithmetic for block partials, dequant identity,
                            reduction to the tensorwise case, SQNR band.
  metrics.sqnr_db           the collapse SQNRs printed in [REPRO] Findings.
  Absolute output norms printed in [REPRO] are parity unpinned (the page does
  not state M or N).
"""

from . import e4m3, quant, gemm, linear, metrics  # noqa: F401
