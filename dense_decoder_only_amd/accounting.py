"""Parameter and FLOP accounting for the training step.

Convention (nano-series page "Karpathy 的 nano 諧系", section nanochat: the
d20 run's ~4e19 training FLOPs equal 6 x params x tokens): a matmul weight of
N entries costs 6 N FLOPs per token for forward plus backward; the embedding
table is a gather and costs nothing.  Causal attention adds, per token and
query head, 2 hd T forward FLOPs (QK^T and PV over T/2 keys on average) and
twice that backward: 6 L H hd T per token in total.
"""
from __future__ import annotations


def matmul_params(cfg) -> int:
    L, d, H, hd, F, V = cfg.n_layer, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.d_ff, cfg.vocab
    per_layer = cfg.qkv_dim * d + d * H * hd + F * d + d * F
    return L * per_layer + V * d


def total_params(cfg, kv_heads: int | None = None) -> int:
    """All parameters; ``kv_heads`` overrides the K/V head count (MHA check)."""
    kv = cfg.n_kv_head if kv_heads is None else kv_heads
    L, d, H, hd, F, V = cfg.n_layer, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.d_ff, cfg.vocab
    qkv = (H + 2 * kv) * hd
    per_layer = qkv * d + d * H * hd + F * d + d * F
    return L * per_layer + 2 * V * d


def flops_per_token(cfg) -> float:
    return 6.0 * matmul_params(cfg) + 6.0 * cfg.n_layer * cfg.n_head * cfg.head_dim * cfg.seq_len


def flops_per_step(cfg) -> float:
    return flops_per_token(cfg) * cfg.tokens


def flops_per_token_full_square(cfg) -> float:
    """PaLM-style count: attention over all T keys (no causal halving)."""
    return 6.0 * matmul_params(cfg) + 12.0 * cfg.n_layer * cfg.n_head * cfg.head_dim * cfg.seq_len
