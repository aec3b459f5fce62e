"""The fused LM head + cross-entropy (gpt_lmhead_ce) against the oracle.

The isolated-kernel workload: X [N, 768] ~ N(0,1), W [V, 768] ~ N(0, 0.02),
both bf16, Zipf(1.1) targets (seed 1), compared in full at smaller sizes here
(the full N=65536, V=50257 size is in test_gpu_stated.py), plus ragged row
chunks at wide rows and out-of-range targets.
"""
import numpy as np
import pytest

import oracle
from decoder_only_transformer_train_amd import binding, synthetic
from gpu_util import announce, cosine, rel_err

pytestmark = pytest.mark.gpu


def to_dev(X, W, y, dtype):
    import torch
    if dtype == binding.GPT_BF16:
        Xd = torch.from_numpy(synthetic.bf16_bits(X).view(np.int16)).cuda()
        Wd = torch.from_numpy(synthetic.bf16_bits(W).view(np.int16)).cuda()
    else:
        Xd = torch.from_numpy(np.ascontiguousarray(X, np.float32)).cuda()
        Wd = torch.from_numpy(np.ascontiguousarray(W, np.float32)).cuda()
    return Xd, Wd, torch.from_numpy(np.ascontiguousarray(y, np.int32)).cuda()


@pytest.mark.parametrize("N,V", [(2048, 50257), (384, 1000), (128, 64)])
def test_head_bf16_vs_oracle(N, V):
    announce(f"head bf16 N={N} V={V}")
    X, W, y = synthetic.lmhead_inputs(N, V, 768, seed=1)
    loss, dX, dW = binding.lmhead_ce(*to_dev(X, W, y, binding.GPT_BF16), binding.GPT_BF16)
    rl, _, rdX, rdW = oracle.lmhead_ce(X, W, y)
    assert abs(loss.item() - rl) <= 2e-2
    assert cosine(dX.cpu().numpy(), rdX) >= 0.999
    assert cosine(dW.cpu().numpy(), rdW) >= 0.999


@pytest.mark.parametrize("N,V,dtype", [(2048, 50257, binding.GPT_BF16), (333, 1000, binding.GPT_BF16),
                                       (256, 1000, binding.GPT_F32)])
def test_head_gemm_form_vs_oracle_and_single_kernel(N, V, dtype, monkeypatch):
    # dW by column-block GEMMs (GPT_HEAD_DW=gemm: 13 blocks with a ragged last one at V=50257)
    announce(f"head GEMM-form dW dtype={dtype} N={N} V={V}")
    C = 768 if dtype == binding.GPT_BF16 else 64
    if dtype == binding.GPT_BF16:
        X, W, y = synthetic.lmhead_inputs(N, V, C, seed=4)
    else:
        rng = np.random.default_rng(4)
        X = rng.standard_normal((N, C)).astype(np.float32)
        W = (rng.standard_normal((V, C)) * 0.3).astype(np.float32)
        y = rng.integers(0, V, N).astype(np.int32)
    dev = to_dev(X, W, y, dtype)
    _, _, dW1 = binding.lmhead_ce(*dev, dtype)
    monkeypatch.setenv("GPT_HEAD_DW", "gemm")
    loss, dX, dW = binding.lmhead_ce(*dev, dtype)
    rl, _, rdX, rdW = oracle.lmhead_ce(X, W, y)
    if dtype == binding.GPT_BF16:
        assert abs(loss.item() - rl) <= 2e-2
        assert cosine(dW.cpu().numpy(), rdW) >= 0.999
        assert rel_err(dW.cpu().numpy(), dW1.cpu().numpy()) <= 1e-2
    else:
        assert rel_err(dW.cpu().numpy(), rdW) <= 1e-4
        assert rel_err(dW.cpu().numpy(), dW1.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("N,V,C", [(256, 1000, 64), (200, 77, 128)])
def test_head_fp32_vs_oracle(N, V, C):
    announce(f"head fp32 N={N} V={V} C={C}")
    rng = np.random.default_rng(5)
    X = rng.standard_normal((N, C)).astype(np.float32)
    W = (rng.standard_normal((V, C)) * 0.3).astype(np.float32)
    y = rng.integers(0, V, N).astype(np.int32)
    loss, dX, dW = binding.lmhead_ce(*to_dev(X, W, y, binding.GPT_F32), binding.GPT_F32)
    rl, _, rdX, rdW = oracle.lmhead_ce(X, W, y)
    assert abs(loss.item() - rl) <= 1e-4 * rl
    assert rel_err(dX.cpu().numpy(), rdX) <= 1e-4
    assert rel_err(dW.cpu().numpy(), rdW) <= 1e-4


@pytest.mark.parametrize("N,V,C", [(4352, 300, 1600), (4352, 300, 1280), (4100, 257, 1792), (333, 129, 1024),
                                   (97, 33, 192)])
def test_head_ragged_rows_wide_rows(N, V, C):
    # row counts and vocabularies that are not multiples of the 32- or 64-row blocks, at every
    # register/LDS shape of the kernel (64-column groups per wave: 1, 3, 4, 5, 7)
    announce(f"head bf16 N={N} V={V} C={C}")
    X, W, y = synthetic.lmhead_inputs(N, V, C, seed=2)
    loss, dX, dW = binding.lmhead_ce(*to_dev(X, W, y, binding.GPT_BF16), binding.GPT_BF16)
    rl, _, rdX, rdW = oracle.lmhead_ce(X, W, y)
    assert abs(loss.item() - rl) <= 2e-2
    assert cosine(dX.cpu().numpy(), rdX) >= 0.999
    assert cosine(dW.cpu().numpy(), rdW) >= 0.999


def test_head_target_out_of_range_is_erange():
    import torch
    N, V, C = 256, 100, 64
    X, W, y = synthetic.lmhead_inputs(N, V, C, seed=3)
    for bad in (V, -1, 1 << 30):
        yb = y.copy()
        yb[37] = bad
        with pytest.raises(binding.GPTError) as e:
            binding.lmhead_ce(*to_dev(X, W, yb, binding.GPT_BF16), binding.GPT_BF16)
        assert e.value.code == binding.GPT_ERANGE
    # a valid call on the same buffers afterwards is clean
    loss, _, _ = binding.lmhead_ce(*to_dev(X, W, y, binding.GPT_BF16), binding.GPT_BF16)
    rl, _, _, _ = oracle.lmhead_ce(X, W, y)
    assert abs(loss.item() - rl) <= 2e-2
    torch.cuda.synchronize()


@pytest.mark.parametrize("N,V,C", [(2048, 50257, 768), (333, 1000, 768), (200, 32, 768), (130, 64, 768),
                                   (97, 95, 768), (333, 129, 1024), (4352, 300, 1024)])
def test_head_pipelined_sweep_matches_sequential(N, V, C, monkeypatch):
    # C = 768 and 1024 run the software-pipelined sweep (GPT_HEAD_PIPE=0: the sequential one); it
    # forms the same products and sums in the same order, so every output has the same bits.
    # Streamed blocks per sweep: V / 32 = 1, 2, 3, 5, 32, 1571 (pass 1), N / 32 = 4 .. 136 (pass 2).
    import torch
    announce(f"head pipelined vs sequential N={N} V={V} C={C}")
    X, W, y = synthetic.lmhead_inputs(N, V, C, seed=6)
    dev = to_dev(X, W, y, binding.GPT_BF16)
    loss1, dX1, dW1 = binding.lmhead_ce(*dev, binding.GPT_BF16)
    monkeypatch.setenv("GPT_HEAD_PIPE", "0")
    loss0, dX0, dW0 = binding.lmhead_ce(*dev, binding.GPT_BF16)
    assert loss1.item() == loss0.item()
    assert torch.equal(dX1, dX0)
    assert torch.equal(dW1, dW0)
    rl, _, rdX, rdW = oracle.lmhead_ce(X, W, y)
    assert abs(loss1.item() - rl) <= 2e-2
    assert cosine(dX1.cpu().numpy(), rdX) >= 0.999
    assert cosine(dW1.cpu().numpy(), rdW) >= 0.999


@pytest.mark.parametrize("C", [768, 1024, 64])
def test_head_softmax_reference_redo(C, monkeypatch):
    # rows whose largest logit (about 0.13 |x|^2, 100 at C = 768) lies in a W block after the
    # first and exceeds that block's maximum by far more than 2^64 in exp2 units: their sweep
    # is redone with the larger reference; the loss and gradients still match the oracle
    import torch
    announce(f"head softmax reference redo C={C}")
    N, V = 256, 1000
    X, W, y = synthetic.lmhead_inputs(N, V, C, seed=7)
    s = 100.0 / C
    for r, v in [(0, 500), (77, 999), (200, 40), (201, 33)]:
        W[v] = synthetic.round_bf16((s * X[r]).astype(np.float32))
    y[0] = 500  # one peaked row whose target is its peak, one whose target is elsewhere
    dev = to_dev(X, W, y, binding.GPT_BF16)
    loss, dX, dW = binding.lmhead_ce(*dev, binding.GPT_BF16)
    rl, per, rdX, rdW = oracle.lmhead_ce(X, W, y)
    assert np.isfinite(loss.item())
    assert abs(loss.item() - rl) <= 2e-2
    assert cosine(dX.cpu().numpy(), rdX) >= 0.999
    assert cosine(dW.cpu().numpy(), rdW) >= 0.999
    monkeypatch.setenv("GPT_HEAD_PIPE", "0")
    loss0, dX0, dW0 = binding.lmhead_ce(*dev, binding.GPT_BF16)
    assert loss.item() == loss0.item() and torch.equal(dX, dX0) and torch.equal(dW, dW0)
