"""bsgemm: block-scaled low-precision GEMM (NVFP4, MXFP8) for AMD MI355X (gfx950).

The computation lives in the HIP library ``libbsgemm.so`` (C ABI in
``include/bsgemm.h``); ``lib`` is its thin ctypes binding and ``synth`` the
seeded synthetic input generators.  Build with
``python -m block_scaled_precision_bsgemm_amd.build``.
"""

__all__ = ["lib", "synth", "build"]
