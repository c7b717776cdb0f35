"""Block-scaled (MX / tensor-wise / groupwise) FP8 and FP4 GEMM for MI355X.

The compute path lives in the HIP library ``libmxgemm.so`` (C ABI declared in
``include/mxgemm.h``); ``block_scaled_precision_03_amd.mxgemm`` is its thin
Python binding.  ``synth`` builds seeded synthetic inputs.
"""
