"""Block-scaled FP8 quantization and GEMMs for AMD MI355X (gfx950).

The computation lives in the HIP library ``libfp8bs.so`` (C ABI declared in
``include/fp8bs.h``); this package is its thin Python binding.  Importing
``fp8_fine_grained_act_amd.lib`` loads the library and fails if it is not built.
"""

__all__ = ["lib"]
