"""Model shapes and workloads for the denoising step.

The method (DiffusionGemma technical report, as summarised on the arXiv
abstract page and the laozijiushiniubi.cn article, sections 2 and 4): a
mixture-of-experts transformer with 128 experts and top-8 routing refines a
256-token canvas in parallel, with causal attention over an encoded prompt
prefix and bidirectional attention inside the canvas.  The pages do not give
the layer dimensions, so the full-size shapes below are synthetic: 30 layers
at d_model 2816 land near the pages' 25.2B total / 3.8B active parameters.

This module holds plain data only (no arithmetic of the method).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    d_expert: int
    d_shared: int          # 0 = no shared FFN
    vocab: int             # 0 = no embedding / LM head (hidden-state workload)
    self_cond: int         # 1 = gated self-conditioning projection present
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6

    @property
    def qkv_dim(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    def param_counts(self) -> dict:
        """Total / active / self-conditioning parameter counts."""
        d, hd = self.d_model, self.head_dim
        attn = d + self.qkv_dim * d + 2 * hd + d * self.n_heads * hd
        ffn_dense = d + self.n_experts * d + 3 * d * self.d_shared
        expert = 3 * d * self.d_expert
        per_layer_total = attn + ffn_dense + self.n_experts * expert
        per_layer_active = attn + ffn_dense + self.top_k * expert
        emb = self.vocab * d + (d if self.vocab else 0)      # tied table + final norm
        sc = (d * d + d) if self.self_cond else 0
        return {
            "total": self.n_layers * per_layer_total + emb + sc,
            "active": self.n_layers * per_layer_active + emb + sc,
            "self_cond": sc,
        }


@dataclass(frozen=True)
class SamplerParams:
    tau_start: float = 0.8
    tau_end: float = 0.4
    max_steps: int = 48
    lock_rule: int = 0          # 0: H_i < lock_thresh ; 1: sorted cumulative entropy <= lock_thresh
    lock_thresh: float = 0.5
    stop_rule: int = 0          # 0: mean H < stop_thresh ; 1: mean H < stop_thresh and argmax unchanged
    stop_thresh: float = 0.1


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    batch: int          # canvases B
    prefix_batch: int   # prefixes Bp (1 = shared by every canvas, or == batch)
    prefix_len: int     # P
    canvas_len: int     # T
    steps: int          # denoising steps run by the workload (1 = single step)
    hidden_input: bool  # True: canvas/prefix given as hidden states (no embedding, no head)
    sampler: SamplerParams = SamplerParams()
    hidden_common: float = 0.0  # hidden-state inputs: weight of a direction shared by every canvas row

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


TINY = ModelShape(n_layers=2, d_model=256, n_heads=4, n_kv_heads=2, head_dim=64,
                  n_experts=8, top_k=2, d_expert=512, d_shared=0, vocab=2048, self_cond=0)

# the tiny model with a shared FFN two expert widths wide: decoding runs it as
# two extra experts of the grouped products
TINY_SHARED = dataclasses.replace(TINY, d_shared=1024)

# the tiny model with the gated self-conditioning projection (the block tests
# follow the soft-prediction state from step to step)
TINY_SELF_COND = dataclasses.replace(TINY, self_cond=1)

FULL_LAYER = ModelShape(n_layers=1, d_model=2816, n_heads=16, n_kv_heads=8, head_dim=256,
                        n_experts=128, top_k=8, d_expert=704, d_shared=2112, vocab=0,
                        self_cond=0)

FULL = ModelShape(n_layers=30, d_model=2816, n_heads=16, n_kv_heads=8, head_dim=256,
                  n_experts=128, top_k=8, d_expert=704, d_shared=2112, vocab=262144,
                  self_cond=1)

WORKLOADS = {
    # 2-layer model, 64-token prefix, 32-token canvas, one step.
    "tiny_step": Workload("tiny_step", TINY, batch=1, prefix_batch=1, prefix_len=64,
                          canvas_len=32, steps=1, hidden_input=False),
    # one full-width layer over a 2048-token prefix; canvas hidden states in, out.
    "layer_step": Workload("layer_step", FULL_LAYER, batch=1, prefix_batch=1,
                           prefix_len=2048, canvas_len=256, steps=1, hidden_input=True),
    # layer_step with canvas rows that share a common direction (weight 0.95):
    # the router then picks about 84 distinct experts over the 256 rows (84 at
    # seed 2024, 93 at seed 1234: the count depends on the draw), the count the
    # article's section 5 gives for the trained model; iid rows pick all 128,
    # and the 30-layer random model averages 57.
    "layer_step_routed": Workload("layer_step_routed", FULL_LAYER, batch=1, prefix_batch=1,
                                  prefix_len=2048, canvas_len=256, steps=1, hidden_input=True,
                                  hidden_common=0.95),
    # full 30-layer model, one steady-state denoising step.
    "full_step": Workload("full_step", FULL, batch=1, prefix_batch=1, prefix_len=2048,
                          canvas_len=256, steps=1, hidden_input=False),
    # full model, block of up to 48 steps with the entropy lock / stop rule.
    "full_block": Workload("full_block", FULL, batch=1, prefix_batch=1, prefix_len=2048,
                           canvas_len=256, steps=48, hidden_input=False),
    # full model, 32768-token shared prefix, 4 canvases, up to 48 steps.
    "long_block": Workload("long_block", FULL, batch=4, prefix_batch=1, prefix_len=32768,
                           canvas_len=256, steps=48, hidden_input=False),
    # long_block with one 32768-token prompt per canvas (4 prompts, 4x the KV)
    "long_block_bp4": Workload("long_block_bp4", FULL, batch=4, prefix_batch=4, prefix_len=32768,
                               canvas_len=256, steps=48, hidden_input=False),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]
