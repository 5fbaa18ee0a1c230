"""CPU oracle for the single-GPU MoE expert-layer forward (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import anything from this package. The product path (the HIP library and its
Python binding) never imports it, and it never imports the product path: the
two share no code. Inputs come from the seeded generators in `workloads`.

Pages cited in this package (titles as they appear on the pages):
  [MoE-vLLM]  "LLM 分布式推理基础（一）— MoE 分布式推理基础（基于 vLLM）",
              cnblogs.com/paitsai (OLMoE-1B-7B shapes, Algorithm 2 and the
              Hugging Face router/experts source it annotates).
  [goin]      "0. goin", obnotes DModel/learn (torchtitan token dispatchers
              and the MinimalAsyncEP kernel table).
  [Domino]    "XTuner Domino EP", icarus.shaojiemike.top.
  [Fusion]    "大模型系统中的通算融合：从 overlap 到 tile-level operator",
              aigcage.com.
"""

from . import fp8  # noqa: F401
from .moe_oracle import (  # noqa: F401
    backward,
    combine_backward,
    combine_slot_order,
    dispatch_backward,
    ep_share_forward,
    expert_counts,
    expert_ffn,
    forward,
    gate_up_preactivations,
    grouped_data_grad,
    grouped_swiglu,
    grouped_weight_grad,
    offsets_from_counts,
    permutation,
    round_to_f32,
    route_from_logits,
    router_backward,
    router_logits,
    splits_by_rank,
    splits_from_offsets,
    swiglu_backward,
    topk_margin,
    weighted_rows_token_order,
)
