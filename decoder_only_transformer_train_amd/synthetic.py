"""Seeded synthetic inputs shared by the HIP path, the oracle and the bench.

This module only draws random numbers and lays them out; it computes nothing
of the training step itself.  Both sides of every parity test receive the
arrays it returns.

Streams
  * uniform token IDs in [0, V) (the tiny fp32 model);
  * a finite Zipf(s) stream over ranks k = 1..V with ID = k - 1, drawn by
    inverse CDF, and an end-of-text ID written after every Geometric(p) gap
    of ordinary tokens (document separators in a concatenated token stream,
    as in the GPT-2 reproduction lecture's data section);
  * inputs of the isolated LM-head + cross-entropy problem.

Weights follow the GPT-2 reproduction lecture's initialisation section:
N(0, 0.02) for matrices and embeddings, N(0, 0.02/sqrt(2L)) for the two
residual-output projections of each block, zero biases and LayerNorm beta,
LayerNorm gamma one.  Values are drawn in float64 with numpy's default_rng
and rounded once to float32, the master-weight precision.
"""
from __future__ import annotations

import numpy as np

EOT_ID = 50256


def uniform_tokens(n: int, vocab: int, seed: int) -> np.ndarray:
    """n token IDs uniform in [0, vocab), int32."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def _zipf_cdf(vocab: int, s: float) -> np.ndarray:
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    w = ranks ** (-s)
    cdf = np.cumsum(w)
    return cdf / cdf[-1]


def zipf_ids(n: int, vocab: int, seed: int, s: float = 1.1,
             rng: np.random.Generator | None = None) -> np.ndarray:
    """n IDs from a finite Zipf(s) law over ranks 1..vocab, ID = rank - 1."""
    if rng is None:
        rng = np.random.default_rng(seed)
    cdf = _zipf_cdf(vocab, s)
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def zipf_eot_stream(n: int, vocab: int = 50257, seed: int = 0, s: float = 1.1,
                    eot: int = EOT_ID, p_gap: float = 1.0 / 600.0) -> np.ndarray:
    """Zipf(s) token stream of length n with `eot` after every Geometric(p_gap) gap."""
    rng = np.random.default_rng(seed)
    toks = zipf_ids(n, vocab, seed, s, rng=rng)
    # gaps g >= 1 of ordinary tokens, each followed by one separator
    n_gaps = int(n * p_gap * 2) + 16
    gaps = rng.geometric(p_gap, size=n_gaps)
    pos = np.cumsum(gaps + 1) - 1
    while pos[-1] < n:
        more = rng.geometric(p_gap, size=n_gaps)
        pos = np.concatenate([pos, pos[-1] + np.cumsum(more + 1)])
    pos = pos[pos < n]
    toks[pos] = eot
    return toks


def tensor_layout(n_layer: int, n_embd: int, vocab_padded: int, max_seq: int):
    """Ordered (name, shape, std_kind) list: embeddings, blocks, final norm.

    std_kind: "w" N(0,0.02), "wr" N(0,0.02/sqrt(2L)), "zero", "one".
    Matrices are row-major [out, in]; the attention input projection packs
    rows as [q | k | v].
    """
    C, L = n_embd, n_layer
    out = [("wte", (vocab_padded, C), "w"), ("wpe", (max_seq, C), "w")]
    for l in range(L):
        p = f"h{l}."
        out += [
            (p + "ln1.g", (C,), "one"), (p + "ln1.b", (C,), "zero"),
            (p + "attn.w", (3 * C, C), "w"), (p + "attn.b", (3 * C,), "zero"),
            (p + "proj.w", (C, C), "wr"), (p + "proj.b", (C,), "zero"),
            (p + "ln2.g", (C,), "one"), (p + "ln2.b", (C,), "zero"),
            (p + "fc.w", (4 * C, C), "w"), (p + "fc.b", (4 * C,), "zero"),
            (p + "mlp_proj.w", (C, 4 * C), "wr"), (p + "mlp_proj.b", (C,), "zero"),
        ]
    out += [("lnf.g", (C,), "one"), ("lnf.b", (C,), "zero")]
    return out


def init_params(n_layer: int, n_embd: int, vocab_padded: int, max_seq: int,
                seed: int = 0) -> dict[str, np.ndarray]:
    """Initial weights as float32 arrays, drawn in layout order from one generator."""
    rng = np.random.default_rng(seed)
    std = 0.02
    std_r = 0.02 / np.sqrt(2.0 * n_layer)
    params: dict[str, np.ndarray] = {}
    for name, shape, kind in tensor_layout(n_layer, n_embd, vocab_padded, max_seq):
        if kind == "w":
            a = rng.standard_normal(shape) * std
        elif kind == "wr":
            a = rng.standard_normal(shape) * std_r
        elif kind == "zero":
            a = np.zeros(shape)
        else:
            a = np.ones(shape)
        params[name] = a.astype(np.float32)
    return params


def tensor_layout_cs336(n_layer: int, n_embd: int, d_ff: int, vocab_padded: int):
    """Ordered (name, shape, std_kind) list of the RMSNorm / RoPE / SwiGLU block variant.

    No biases and no position table; w1 (gate) and w3 (up) are [d_ff, C], w2 is
    [C, d_ff]; lm_head [V_pad, C] is the output projection, separate from wte.
    """
    C, L, F = n_embd, n_layer, d_ff
    out = [("wte", (vocab_padded, C), "w")]
    for l in range(L):
        p = f"h{l}."
        out += [
            (p + "rms1.g", (C,), "one"), (p + "attn.w", (3 * C, C), "w"), (p + "proj.w", (C, C), "wr"),
            (p + "rms2.g", (C,), "one"), (p + "w1", (F, C), "w"), (p + "w3", (F, C), "w"),
            (p + "w2", (C, F), "wr"),
        ]
    out += [("rmsf.g", (C,), "one"), ("lm_head", (vocab_padded, C), "w")]
    return out


def init_params_cs336(n_layer: int, n_embd: int, d_ff: int, vocab_padded: int, seed: int = 0,
                      gain_jitter: float = 0.0) -> dict[str, np.ndarray]:
    """Initial weights of the variant as float32 arrays (same scheme as init_params);
    gain_jitter > 0 draws the RMSNorm gains as 1 + gain_jitter * N(0, 1)."""
    rng = np.random.default_rng(seed)
    std = 0.02
    std_r = 0.02 / np.sqrt(2.0 * n_layer)
    params: dict[str, np.ndarray] = {}
    for name, shape, kind in tensor_layout_cs336(n_layer, n_embd, d_ff, vocab_padded):
        if kind == "w":
            a = rng.standard_normal(shape) * std
        elif kind == "wr":
            a = rng.standard_normal(shape) * std_r
        else:
            a = 1.0 + gain_jitter * rng.standard_normal(shape) if gain_jitter else np.ones(shape)
        params[name] = a.astype(np.float32)
    return params


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(np.shape(a))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exactly bfloat16."""
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def lmhead_inputs(n: int, vocab: int, n_embd: int, seed: int = 1):
    """Inputs of the isolated LM-head + CE problem.

    X [n, C] ~ N(0, 1) per element (the scale of LayerNorm output with unit
    gain), W [vocab, C] ~ N(0, 0.02), both rounded to bf16; targets drawn
    Zipf(1.1) over the vocabulary.  Returned as float32 arrays holding
    bf16-exact values, plus int32 targets.
    """
    rng = np.random.default_rng(seed)
    X = round_bf16(rng.standard_normal((n, n_embd)).astype(np.float32))
    W = round_bf16((rng.standard_normal((vocab, n_embd)) * 0.02).astype(np.float32))
    y = zipf_ids(n, vocab, seed, 1.1, rng=rng)
    return X, W, y
