"""Named model / batch configurations of the GPT-2 training step."""
from __future__ import annotations

from dataclasses import dataclass, replace

from . import binding


@dataclass(frozen=True)
class GPTConfig:
    n_layer: int
    n_embd: int
    n_head: int
    vocab: int
    padded_vocab: int
    max_seq: int
    batch: int
    seq: int
    dtype: int = binding.GPT_BF16
    accum: int = 1  # micro-steps per optimiser step
    block: int = binding.GPT_BLOCK_GPT2
    d_ff: int = 0            # SwiGLU width (block GPT_BLOCK_RMS_ROPE_SWIGLU)
    rope_theta: float = 10000.0

    def to_c(self) -> binding.GPTConfigC:
        return binding.GPTConfigC(self.n_layer, self.n_embd, self.n_head, self.vocab, self.padded_vocab,
                                  self.max_seq, self.batch, self.seq, self.dtype, self.block, self.d_ff,
                                  self.rope_theta)

    def with_(self, **kw) -> "GPTConfig":
        return replace(self, **kw)

    @property
    def tokens_per_step(self) -> int:
        return self.batch * self.seq * self.accum


# the lecture's GPT-2 small: 12 layers, width 768, 12 heads, 50257 tokens padded to 50304, 1024 positions
TINY_F32 = GPTConfig(2, 64, 4, 256, 256, 32, 4, 32, binding.GPT_F32)
GPT2_124M = GPTConfig(12, 768, 12, 50257, 50304, 1024, 16, 1024, binding.GPT_BF16)
GPT2_350M = GPTConfig(24, 1024, 16, 50257, 50304, 1024, 8, 1024, binding.GPT_BF16)
GPT2_1P5B = GPTConfig(48, 1600, 25, 50257, 50304, 1024, 4, 1024, binding.GPT_BF16, accum=4)

# the second block variant (RMSNorm, RoPE, SwiGLU, untied head; CS336 pretraining page): the page's
# TinyStories model (V = 10000, context 256, d_model 512, d_ff 1344, 4 layers, 16 heads, RoPE theta
# 10000) in fp32 with its batch of 32, a tiny fp32 one for parity, and a bf16 one with head size 64
CS336_TINYSTORIES = GPTConfig(4, 512, 16, 10000, 10000, 256, 32, 256, binding.GPT_F32,
                              block=binding.GPT_BLOCK_RMS_ROPE_SWIGLU, d_ff=1344)
CS336_TINY_F32 = GPTConfig(2, 64, 4, 256, 256, 32, 4, 32, binding.GPT_F32,
                           block=binding.GPT_BLOCK_RMS_ROPE_SWIGLU, d_ff=192)
CS336_TINYSTORIES_BF16 = CS336_TINYSTORIES.with_(n_head=8, dtype=binding.GPT_BF16)

PRESETS = {"tiny": TINY_F32, "gpt2-124m": GPT2_124M, "gpt2-350m": GPT2_350M, "gpt2-1.5b": GPT2_1P5B,
           "cs336-tinystories": CS336_TINYSTORIES, "cs336-tinystories-bf16": CS336_TINYSTORIES_BF16}

# AdamW settings of the step (lecture: GPT-3 small peak lr 6e-4; betas (0.9, 0.95), eps 1e-8, wd 0.1)
ADAMW = dict(lr=6e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
