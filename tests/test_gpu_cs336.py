"""The second block variant (RMSNorm, RoPE on Q and K, SwiGLU, untied head; CS336
pretraining page, sections 4 and 6) on the GPU against the fp64 oracle.

fp32: the tiny variant and the page's TinyStories model (V = 10000, context 256,
d_model 512, d_ff 1344, 4 layers, 16 heads of 32) at its batch of 32, 1e-4
relative on the loss and on every gradient, then one AdamW update; bf16 (head
size 64, 8 heads): |loss - oracle| <= 2e-2 and gradient cosine >= 0.999.
Gains are drawn around 1 (not all ones) so that a dropped gain fails.
"""
import numpy as np
import pytest

import oracle
from decoder_only_transformer_train_amd import binding, configs, synthetic
from gpu_util import announce, context, cosine, init_for, rel_err

pytestmark = pytest.mark.gpu

ADAM = dict(lr=6e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def run_step(cfg, p, toks, accum=1):
    g = context(cfg, p)
    N = cfg.batch * cfg.seq
    losses = []
    for i in range(accum):
        g.make_batch(toks, i * N)
        losses.append(g.forward_loss(1.0 / accum))
        g.backward()
    return g, float(np.mean(losses))


@pytest.mark.parametrize("cfg", [configs.CS336_TINY_F32, configs.CS336_TINYSTORIES],
                         ids=["tiny", "tinystories-b32"])
def test_fp32_step_and_update_match_oracle(cfg):
    announce(f"cs336 fp32 step {cfg.n_layer}L C={cfg.n_embd} F={cfg.d_ff} B={cfg.batch}")
    p = init_for(cfg, seed=1, gain_jitter=0.1)
    toks = synthetic.uniform_tokens(cfg.batch * cfg.seq + 1, cfg.vocab, seed=1)
    g, loss = run_step(cfg, p, toks)
    grads = g.get_all(binding.GRAD)
    x, y = oracle.make_batch(toks, 0, cfg.batch, cfg.seq)
    rl, rows, G = oracle.cs336_loss_and_grads(p, x, y, cfg.n_head, cfg.rope_theta)
    assert abs(loss - rl) <= 1e-4 * rl, (loss, rl)
    np.testing.assert_allclose(g.token_losses(), rows, rtol=1e-4, atol=1e-5)
    assert set(g.names) == set(p)
    for k in g.names:
        assert rel_err(grads[k], G[k]) <= 1e-4, (k, rel_err(grads[k], G[k]))
    gn = g.adamw_step(**ADAM)
    P2, m, v = oracle.adamw_step({k: np.asarray(a, np.float64) for k, a in p.items()}, G,
                                 {k: np.zeros(a.shape) for k, a in p.items()},
                                 {k: np.zeros(a.shape) for k, a in p.items()}, 1, **{k: ADAM[k] for k in ADAM})
    assert abs(gn - oracle.grad_norm(G)) <= 1e-4 * gn
    for k in g.names:
        assert rel_err(g.get(k) - p[k], P2[k] - p[k]) <= 1e-3, k


def test_bf16_step_matches_oracle():
    cfg = configs.CS336_TINYSTORIES_BF16.with_(batch=2)
    announce("cs336 bf16 step (TinyStories shapes, 8 heads of 64)")
    p = init_for(cfg, seed=2, gain_jitter=0.1)
    toks = synthetic.uniform_tokens(cfg.batch * cfg.seq + 1, cfg.vocab, seed=2)
    g, loss = run_step(cfg, p, toks)
    grads = g.get_all(binding.GRAD)
    x, y = oracle.make_batch(toks, 0, cfg.batch, cfg.seq)
    rl, _, G = oracle.cs336_loss_and_grads(p, x, y, cfg.n_head, cfg.rope_theta)
    assert abs(loss - rl) <= 2e-2, (loss, rl)
    for k in g.names:
        c = cosine(grads[k], G[k])
        assert c >= 0.999, (k, c)
        na, nb = np.linalg.norm(grads[k]), np.linalg.norm(G[k])
        assert abs(na - nb) <= 0.02 * nb + 1e-6, (k, na, nb)


def test_accumulation_and_determinism():
    cfg = configs.CS336_TINY_F32
    announce("cs336 accumulation and determinism")
    p = init_for(cfg, seed=3, gain_jitter=0.1)
    N = cfg.batch * cfg.seq
    toks = synthetic.uniform_tokens(2 * N + 1, cfg.vocab, seed=3)
    g2, l2 = run_step(cfg, p, toks, accum=2)
    ga, la = run_step(cfg, p, toks, accum=2)
    A, Bv = g2.get_all(binding.GRAD), ga.get_all(binding.GRAD)
    for k in A:
        assert np.array_equal(A[k], Bv[k]), k
    # two micro-steps of B rows each against the oracle's 2B-row batch
    x = np.concatenate([oracle.make_batch(toks, 0, cfg.batch, cfg.seq)[0],
                        oracle.make_batch(toks, N, cfg.batch, cfg.seq)[0]])
    y = np.concatenate([oracle.make_batch(toks, 0, cfg.batch, cfg.seq)[1],
                        oracle.make_batch(toks, N, cfg.batch, cfg.seq)[1]])
    rl, _, G = oracle.cs336_loss_and_grads(p, x, y, cfg.n_head, cfg.rope_theta)
    assert abs(l2 - rl) <= 1e-4 * rl
    for k in A:
        assert rel_err(A[k], G[k]) <= 1e-4, k
