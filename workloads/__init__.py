"""Seeded synthetic inputs for paged decode attention (shared by the oracle tests, the GPU
parity tests and the benchmark). No attention arithmetic lives here."""
from .block_manager import AppendPlan, BlockManager, PoolExhausted, check_plan  # noqa: F401
from .configs import (  # noqa: F401
    SEEDS,
    DecodeCase,
    PrefillCase,
    StepInputs,
    by_name,
    eight_b,
    kv_head_shard,
    normal_f16,
    prefill_8b,
    prefill_case,
    prefix_groups,
    random_case,
    shared_prefix,
    softmax_scale,
    sweep,
    tiny,
    variant,
)
from .quant import quantize_pool, quantize_tile  # noqa: F401
