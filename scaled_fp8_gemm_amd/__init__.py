"""MI355X-native FP8 scaled GEMM: quantise BF16 to OCP FP8 under a scaling
recipe, then the fprop / dgrad / wgrad GEMMs of a linear layer on gfx950 MFMA.

The compute path lives in the C-ABI library ``libfp8sg.so`` (HIP kernels for
gfx950); ``scaled_fp8_gemm_amd.fp8sg`` is its thin Python binding.  Importing
this package does not load the library; ``gen`` holds the seeded input
generators.
"""
