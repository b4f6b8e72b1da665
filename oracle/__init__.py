"""CPU oracle of the routed-expert MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or run anything in this package.  It imports
nothing from the product package, and the product never imports it.

Parity status per function (pins in tests/test_oracle_pins.py):
every function below, and those of ``oracle.mxfp8`` (MXFP8 dispatch), is pinned; the float outputs of the full-size layers have
no worked numeric example on the pages and are pinned only through the
brute-force, closed-form and special-case checks on small layers.
"""
from .moe_oracle import (decode, round_bf16, round_f32, gate_logits, router_scores, topk_ids,
                         routing_weights, routing_margins, expert_counts, segment_offsets,
                         permutation, gather_rows, dispatch_bytes, silu, expert_ffn_rows,
                         grouped_expert_ffn, shared_expert_ffn, combine, latent_down, latent_up,
                         route, layer_forward, token_outputs, load_skew, p95_nearest_rank)
from . import mxfp8

__all__ = ["decode", "round_bf16", "round_f32", "gate_logits", "router_scores", "topk_ids",
           "routing_weights", "routing_margins", "expert_counts", "segment_offsets",
           "permutation", "gather_rows", "dispatch_bytes", "silu", "expert_ffn_rows",
           "grouped_expert_ffn", "shared_expert_ffn", "combine", "latent_down", "latent_up", "route",
           "layer_forward", "token_outputs", "load_skew", "p95_nearest_rank", "mxfp8"]
