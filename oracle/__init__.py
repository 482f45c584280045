"""CPU oracle for the latent-MoE layer forward (test infrastructure).

This package is a plain, slow, obviously-correct numpy implementation of what
the layer computes. It exists to check the HIP path: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it. The product path never imports it, and it imports nothing from the
product path.

Every function cites the passage of the pages it follows:

* Hugging Face model card "Edge0-145B . Q3_K", section "Architecture" (the
  paragraph under the architecture table): attention works at width 2560; D
  projects each token down to the latent width; the router picks 10 of 512
  experts; each expert runs latent -> 640 -> latent; a shared expert runs
  alongside; U projects the combined result back to 2560; D and U are shared,
  one copy per layer.
* Same card, architecture table: 512 experts per layer, 10 routed + 1 shared
  active per token, SwiGLU width 640, expert pool at latent width 1792.
* agentspulse tutorial "Edge0-145B hardware requirements", section "latent MoE
  architecture": tokens are projected to 1,792 dimensions before the experts
  and back afterwards; 512 routed experts plus one shared expert; the router
  picks 10 per token.
* alphasignal news page, table "Released model variants": latent width 1792
  (145B) and 1280 (120B).

The pages name the weight format (NVFP4, 4-bit floating point) but do not
define it, and do not fix the gating function. The readings taken here: gating
is a softmax over all expert logits, the top-k experts by logit (ties to the
lower index), weights renormalised over the chosen k; experts hold e2m1 codes
with E4M3 per-16 block scales and one fp32 scale per matrix (the OCP formats).

Arithmetic is float64 throughout. The one decision taken in another
precision is the top-k choice, made on router logits rounded to float32, the
precision in which the GPU kernel makes the same choice.
"""
from .formats import bf16_value, dequant_e1m1, dequant_fp4, e1m1_value, e2m1_value, e4m3fn_value, unpack_e1m1
from .latent_moe import (
    OracleResult,
    block_forward,
    expert_record_bytes,
    forward,
    gate_topk,
    param_counts,
    rmsnorm,
    route_bookkeeping,
    silu,
    stack_forward,
    swiglu_expert,
)

__all__ = [
    "bf16_value", "e2m1_value", "e4m3fn_value", "dequant_fp4", "e1m1_value", "unpack_e1m1",
    "dequant_e1m1", "OracleResult",
    "forward", "gate_topk", "route_bookkeeping", "swiglu_expert", "silu", "rmsnorm",
    "block_forward", "stack_forward", "expert_record_bytes", "param_counts",
]
