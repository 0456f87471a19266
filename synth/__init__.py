"""Seeded synthetic inputs for the multi-LoRA batched linear.

This package only draws inputs. It holds none of the layer's arithmetic, and both the
CPU oracle and the GPU library receive what it produces. See ``synth.workloads``.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    Projection,
    Workload,
    bf16_bits_to_f32,
    compact_pool,
    f32_to_bf16_bits,
    fp8_base,
    make_workload,
    MoeWorkload,
    make_moe_workload,
    moe_case,
    pool_param_count,
    random_alpha,
    random_case,
    zipf_probs,
)
