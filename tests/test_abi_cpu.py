"""The C ABI without a GPU: the library loads, exports what include/gpt.h
declares, validates configurations and implements the host cursor rule."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from decoder_only_transformer_train_amd import binding, configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gpt.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_are_exported():
    lib = binding.load()
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.EXPORTS)


def test_exports_in_dynamic_symbol_table():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    syms = set(re.findall(r"\bT (gpt_\w+)", out))
    assert set(declared_functions()) <= syms


@pytest.mark.parametrize("name", list(configs.PRESETS))
def test_arena_bytes_presets(name):
    n = binding.arena_bytes(configs.PRESETS[name])
    assert n > 0 and n % 256 == 0


def test_arena_scales_with_model():
    a = binding.arena_bytes(configs.GPT2_124M)
    b = binding.arena_bytes(configs.GPT2_350M)
    # 124M: 16 B/param fp32 state + 2 B/param shadow is at least 2.2 GB
    assert a > 124e6 * 18 and b > a


@pytest.mark.parametrize("bad", [
    dict(n_embd=100), dict(n_head=5), dict(padded_vocab=100), dict(seq=2048), dict(dtype=7),
    dict(batch=0), dict(n_layer=0), dict(n_embd=4096, n_head=64),
])
def test_invalid_configs_rejected(bad):
    cfg = configs.GPT2_124M.with_(**bad)
    assert binding.arena_bytes(cfg) == 0
    lib = binding.load()
    out = ctypes.c_void_p()
    rc = lib.gpt_init(ctypes.byref(cfg.to_c()), ctypes.c_void_p(4096), 1 << 40, None, 0, ctypes.byref(out))
    assert rc == binding.GPT_EINVAL
    assert lib.gpt_last_error()


def test_init_rejects_small_arena_before_touching_it():
    lib = binding.load()
    cfg = configs.TINY_F32.to_c()
    out = ctypes.c_void_p()
    need = lib.gpt_arena_bytes(ctypes.byref(cfg))
    rc = lib.gpt_init(ctypes.byref(cfg), ctypes.c_void_p(1 << 20), need - 256, None, 0, ctypes.byref(out))
    assert rc == binding.GPT_ENOMEM
    assert b"arena too small" in lib.gpt_last_error()
    rc = lib.gpt_init(ctypes.byref(cfg), ctypes.c_void_p((1 << 20) + 4), need, None, 0, ctypes.byref(out))
    assert rc == binding.GPT_EINVAL


def test_next_start_matches_oracle_cursor():
    rng = np.random.default_rng(0)
    for _ in range(200):
        B, T = int(rng.integers(1, 5)), int(rng.integers(1, 9))
        R = int(rng.integers(1, 4))
        r = int(rng.integers(0, R))
        n = int(rng.integers(B * T * R + 1, 400))
        pos = B * T * r
        for _ in range(6):
            want = oracle.next_start(pos, n, B, T, r, R)
            got = binding.next_start(pos, n, B, T, r, R)
            assert got == want
            pos = got


def test_next_start_pages_example():
    # 28.3: B=2, T=3, R=2: next windows at 12 and 18
    assert [binding.next_start(6 * r, 100, 2, 3, r, 2) for r in range(2)] == [12, 18]
    with pytest.raises(binding.GPTError):
        binding.next_start(0, 100, 2, 3, 2, 2)


def test_lmhead_ws_bytes():
    lib = binding.load()
    assert lib.gpt_lmhead_ce_ws_bytes(65536, 50257, 768, 1) > 0
    assert lib.gpt_lmhead_ce_ws_bytes(65536, 50257, 100, 1) == 0


def test_block_variant_config_checks():
    # the RMSNorm / RoPE / SwiGLU variant: valid presets size an arena; bad widths and bases do not
    lib = binding.load()
    for cfg in (configs.CS336_TINY_F32, configs.CS336_TINYSTORIES, configs.CS336_TINYSTORIES_BF16):
        assert lib.gpt_arena_bytes(ctypes.byref(cfg.to_c())) > 0, cfg
    base = configs.CS336_TINY_F32
    for bad in (base.with_(d_ff=0), base.with_(d_ff=100), base.with_(rope_theta=0.0), base.with_(block=7)):
        assert lib.gpt_arena_bytes(ctypes.byref(bad.to_c())) == 0, bad
    # the GPT-2 block ignores d_ff and rope_theta
    assert lib.gpt_arena_bytes(ctypes.byref(configs.TINY_F32.with_(d_ff=3, rope_theta=-1.0).to_c())) > 0
    # the variant holds no biases and no position table: fewer bytes than GPT-2 at the same sizes
    g2 = configs.TINY_F32
    v = configs.CS336_TINY_F32.with_(d_ff=4 * g2.n_embd)
    assert lib.gpt_arena_bytes(ctypes.byref(v.to_c())) != lib.gpt_arena_bytes(ctypes.byref(g2.to_c()))


def test_batch_token_limit():
    """B*T up to 262144 (the chunked token sort); one more sequence is rejected."""
    ok = configs.TINY_F32.with_(batch=262144 // configs.TINY_F32.seq)
    assert binding.arena_bytes(ok) > 0
    assert binding.arena_bytes(ok.with_(batch=ok.batch + 1)) == 0


def test_operand_4gib_limit():
    """GEMM operands use 32-bit buffer offsets: a config whose widest activation
    ([N, 4C], or [N, 2 d_ff] for the variant block) or embedding reaches 4 GiB
    is rejected; one just below is accepted."""
    # fp32, N = 262144, C = 1024: [N, 4C] is exactly 4 GiB
    big = configs.TINY_F32.with_(n_embd=1024, n_head=16, batch=262144 // configs.TINY_F32.seq)
    assert binding.arena_bytes(big) == 0
    assert binding.arena_bytes(big.with_(n_embd=960, n_head=15)) > 0
    # variant block: [N, 2 d_ff] in bf16 at N = 65536
    v = configs.CS336_TINY_F32.with_(dtype=binding.GPT_BF16, n_embd=64, n_head=1, batch=65536 // 32)
    assert binding.arena_bytes(v.with_(d_ff=16384)) == 0
    assert binding.arena_bytes(v.with_(d_ff=16384 - 64)) > 0

