"""Model-FLOP accounting for throughput and MFU reports.

The convention is the CS336 pretraining page's, section 4 (resource
accounting): only matrix products count, 2 FLOPs per multiply-add, and a
training step costs 3 x the forward (the backward is twice the forward).
Attention counts the causal pairs (j <= i) its kernels compute:
T (T + 1) / 2 per sequence and head.  The padded vocabulary is counted, since
the head's product runs over all of its rows.
"""
from __future__ import annotations


def causal_pairs(T: int) -> int:
    """Number of (query i, key j) pairs with j <= i in a sequence of T positions."""
    return T * (T + 1) // 2


def forward_flops_per_sequence(n_layer: int, n_embd: int, seq: int, vocab: int) -> int:
    """Forward matrix-product FLOPs of one sequence of `seq` tokens (GPT-2 block)."""
    C, L, T = n_embd, n_layer, seq
    proj = 2 * T * 12 * C * C * L           # qkv 3C^2, out C^2, fc 4C^2, mlp-proj 4C^2 per token
    attn = 2 * 2 * C * causal_pairs(T) * L  # q.k and p.v: C multiply-adds per pair over all heads
    head = 2 * T * C * vocab
    return proj + attn + head


def training_flops_per_token(n_layer: int, n_embd: int, seq: int, vocab: int) -> float:
    return 3.0 * forward_flops_per_sequence(n_layer, n_embd, seq, vocab) / seq


def lmhead_flops(N: int, V: int, C: int) -> float:
    """Forward logits, data gradient and weight gradient of the LM head: 6 N V C."""
    return 6.0 * N * V * C
