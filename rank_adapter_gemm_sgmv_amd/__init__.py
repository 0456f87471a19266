"""MI355X (gfx950) multi-LoRA batched linear: y = x W + (x A_i) B_i * alpha_i / r_i.

The library is liblora_mi355x.so (C ABI in include/lora.h, HIP kernels in csrc/); the
binding with the same function names is ``rank_adapter_gemm_sgmv_amd.lora``.  Importing the
binding loads the library and raises if it has not been built
(``python -m rank_adapter_gemm_sgmv_amd.build``).
"""

__all__ = ["lora", "build"]
