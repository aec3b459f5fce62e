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


def block_weights(n_embd: int, d_ff: int = 0) -> int:
    """Matrix weights of one block: GPT-2 (d_ff = 0) qkv 3C^2, out C^2, fc 4C^2, mlp-proj 4C^2;
    the RMSNorm / RoPE / SwiGLU variant qkv 3C^2, out C^2 and SwiGLU's three C x d_ff matrices."""
    C = n_embd
    return 12 * C * C if d_ff == 0 else 4 * C * C + 3 * C * d_ff


def forward_flops_per_sequence(n_layer: int, n_embd: int, seq: int, vocab: int, d_ff: int = 0) -> int:
    """Forward matrix-product FLOPs of one sequence of `seq` tokens."""
    C, L, T = n_embd, n_layer, seq
    proj = 2 * T * block_weights(C, d_ff) * L  # every block weight once per token
    attn = 2 * 2 * C * causal_pairs(T) * L     # q.k and p.v: C multiply-adds per pair over all heads
    head = 2 * T * C * vocab
    return proj + attn + head


def training_flops_per_token(n_layer: int, n_embd: int, seq: int, vocab: int, d_ff: int = 0) -> float:
    return 3.0 * forward_flops_per_sequence(n_layer, n_embd, seq, vocab, d_ff) / seq


def lmhead_flops(N: int, V: int, C: int) -> float:
    """Forward logits, data gradient and weight gradient of the LM head: 6 N V C."""
    return 6.0 * N * V * C
