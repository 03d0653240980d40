"""fp64 CPU oracle of the sparse MoE layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.
"""
from .oracle import *  # noqa: F401,F403
from .oracle import (LayerShape, TOPK_THEN_SOFTMAX, SOFTMAX_THEN_TOPK,  # noqa: F401
                     capacity, router_logits, topk_select, softmax_all,
                     gate_weights, dispatch, silu, expert_ffn, routing_stats,
                     forward, brute_topk_set)
