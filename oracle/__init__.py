"""CPU oracle for the block-scaled FP4 (E2M1) hot path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the smoke entry
point and the benchmark's CPU-baseline leg may import anything in this
package.  The GPU library never calls it and shares no code with it: the
two sides meet only through the seeded input generators, which hold none of
the method's arithmetic.

Layout of the oracle:
  formats.py -- E2M1 / E4M3 / E8M0 / BF16 decode tables and the
                round-to-nearest-even encoders onto those grids.
  quant.py   -- the NVFP4 and MXFP4 block quantisers and their dequantisers.
  gemm.py    -- NVFP4, MXFP4 and W4A16 GEMMs as the plain definition
                D = bf16(alpha * dequant(A) @ dequant(B)^T) in float64.
  moe.py     -- the MXFP4 and NVFP4 W4A4 mixture-of-experts layers, stage by
                stage.
  layout.py  -- block-scale layout interchange: row-major <-> the pages' padded
                128x4 swizzled layouts.
  tolerance.py -- the acceptance rule for floating-point outputs.

Floating point: every step of the quantisers is an IEEE-754 binary32
operation (numpy float32 ufuncs are correctly rounded, and numpy does not
contract a*b+c into a fused multiply-add); every GEMM is float64.
"""
