"""CPU oracle for the NVFP4 block-scaled GEMM (W4A4 and W4A16) and its quantizer.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (the HIP library and its Python binding) never imports it, and
this package imports nothing from the product path: the two share no code, no
tables and no helpers. The only module both sides use is ``synth`` (seeded raw
random inputs), which holds none of the method's arithmetic.

What is computed, with the passage each part follows:

* ``formats``  -- E2M1 and E4M3 decode/encode, nibble packing, BF16 rounding.
  The pages never print the E2M1 table, the E4M3 bit layout or the nibble
  order; the readings taken are the OCP E2M1 / E4M3 ("fn") encodings and
  low-nibble-first packing (Colfax article, "Version 2" input-footprint
  paragraph: 4-bit elements, 8-bit scales per 16 elements; TileLang PR #3290,
  "Design: Weight layout": E2M1 codes as fp4 times a power of two).
* ``quantize`` -- BF16 -> NVFP4 block quantizer: per-tensor global scale,
  per-16 E4M3 scale, E2M1 codes, in a fixed IEEE binary32 order.
* ``gemm``     -- D = alpha * (A . SFA)(B . SFB)^T with FP32-or-better
  accumulation (Colfax article, introduction and "Version 3" epilogue: alpha
  applied in FP32 before the output convert); W4A16 y = alpha * x W~^T
  (TileLang PR #3290, "Summary").
* ``prepared`` -- the byte map of the prepared-weight layout used by the
  library, with the sign and zero folding of the block scales (TileLang PR
  #3290, "Design: Weight layout": zero scales zero their codes, negative
  scales flip code signs, prepared size N*K/2 + N*K/16).

Everything here is deliberately slow and plain: numpy, float64 or exact
integers, no blocking or fusion beyond what the definitions state.
"""
