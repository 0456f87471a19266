"""CPU oracle for the multi-LoRA batched linear -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The GPU library and its Python binding never import it.
"""

from .oracle import (  # noqa: F401
    OracleError,
    build,
    build_segments,
    fp8_e4m3_decode,
    library_path,
    lora_expand,
    lora_linear,
    lora_linear_fp8w,
    lora_shrink,
    moe_lora_linear,
)
