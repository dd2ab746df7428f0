"""CPU oracle for the fused MoE grouped MLP with MXFP8 and NVFP4 group quantization.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
anything in this package: only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library (no kernels, helpers, tables or constants), and the library never
imports it.

What it computes and where that is defined:

* ``formats``  -- the E4M3, E8M0 and E2M1 codecs and the bf16 / fp32 roundings
  (OCP 8-bit Floating Point v1.0; OCP Microscaling Formats (MX) v1.0).
* ``quant``    -- MXFP8 and NVFP4 group quantization with their row-wise and
  column-wise layouts ("GEMM + Swiglu fused Grouped MLP for MXFP8", Greptile
  summary and sequence diagram; "Reduce NVFP4 quantization work for the fused
  GroupedMLP fc2 input ...", Description and Changes).
* ``rht``      -- the 16x16 randomized Hadamard transform with a sign mask and
  the per-group pre-/post-RHT amax (same NVFP4 page, Changes and the commit
  "Pass the RHT sign mask to the Hadamard-fused GEMM kernel").
* ``mlp``      -- the grouped GEMMs and the unfused forward and backward of
  fc1 -> activation * prob -> fc2 (the MXFP8 page's sequence diagram).

Everything is plain numpy: fp64 arithmetic, with each step that the encodings
define in fp32 emulated by rounding the fp64 result of that single operation to
fp32 (exact emulation, since 53 >= 2*24 + 2).  Every reading of a point the
pages leave open is listed in the module that takes it.
"""
