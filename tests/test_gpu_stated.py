"""Parity at the stated configurations, at their full sizes, against the fp64 oracle.

bf16 tolerances: |loss - oracle| <= 2e-2 and per-tensor gradient cosine >= 0.999
after one step (all micro-steps summed), norms within 2%.

  * GPT-2 124M at the bench's shape, B=16, T=1024, every gradient; and two
    identical steps give bit-identical gradients at this shape (two streams,
    split-K weight gradients, the 16384-key token sort);
  * GPT-2 350M, L=24, C=1024, H=16, B=8, T=1024;
  * GPT-2 1.5B, L=48, C=1600, H=25, B=4 x 4 accumulation micro-steps, T=1024,
    on a token stream that repeats every 5 rows: the 16 rows of the 4
    micro-batches are 5 distinct rows (each micro-batch differs from the one
    before), so the oracle runs 5 rows and weights each by how often it occurs;
  * the isolated LM head + cross-entropy at N=65536, V=50257, C=768 (loss, dX, dW).

The oracle's rows run in worker processes (tests/oracle_pool.py).
"""
import numpy as np
import pytest

import oracle
import oracle_pool
from decoder_only_transformer_train_amd import binding, configs, synthetic
from gpu_util import announce, context, cosine, init_for

pytestmark = pytest.mark.gpu


def _workers(per_proc_gb, want):
    """How many oracle workers the host's free memory allows (at least 1)."""
    try:
        import psutil
        avail = psutil.virtual_memory().available / 2**30
    except Exception:
        avail = 64
    return max(1, min(want, int(avail * 0.7 // per_proc_gb)))


def check_bf16(names, grads, G, loss, ref_loss, label):
    worst = min((cosine(grads[k], G[k]), k) for k in names)
    announce(f"{label}: loss {loss:.5f} vs oracle {ref_loss:.5f}; worst gradient cosine {worst}")
    assert abs(loss - ref_loss) <= 2e-2, (loss, ref_loss)
    for k in names:
        c = cosine(grads[k], G[k])
        assert c >= 0.999, (k, c)
        na, nb = np.linalg.norm(grads[k]), np.linalg.norm(G[k])
        assert abs(na - nb) <= 0.02 * nb + 1e-6, (k, na, nb)


def gpu_step(cfg, p, stream, starts):
    g = context(cfg, p)
    losses = []
    for s in starts:
        g.make_batch(stream, s)
        losses.append(g.forward_loss(1.0 / len(starts)))
        g.backward()
    grads = g.get_all(binding.GRAD)
    names = list(g.names)
    g.close()
    return float(np.mean(losses)), grads, names


@pytest.mark.timeout(900)
def test_gpt2_124m_b16_full_gradients_and_determinism():
    cfg = configs.GPT2_124M
    N = cfg.batch * cfg.seq
    stream = synthetic.zipf_eot_stream(N + 1, cfg.vocab, seed=0)
    p = init_for(cfg)
    announce("124M B=16: two identical steps")
    loss, grads, names = gpu_step(cfg, p, stream, [0])
    loss2, grads2, _ = gpu_step(cfg, p, stream, [0])
    assert loss2 == loss
    for k in names:
        np.testing.assert_array_equal(grads2[k], grads[k], err_msg=k)
    del grads2
    x, y = oracle.make_batch(stream, 0, cfg.batch, cfg.seq)
    announce("124M B=16: oracle, 16 rows")
    ref_loss, G = oracle_pool.batch_loss_and_grads(p, x, y, cfg.n_head, [1.0 / cfg.batch] * cfg.batch,
                                                   procs=_workers(8, 4), threads=4, label="124M B=16")
    check_bf16(names, grads, G, loss, ref_loss, "124M B=16")


@pytest.mark.timeout(900)
def test_gpt2_350m_full_depth_b8():
    cfg = configs.GPT2_350M
    N = cfg.batch * cfg.seq
    stream = synthetic.zipf_eot_stream(N + 1, cfg.vocab, seed=0)
    p = init_for(cfg)
    announce("350M L=24 B=8 step")
    loss, grads, names = gpu_step(cfg, p, stream, [0])
    x, y = oracle.make_batch(stream, 0, cfg.batch, cfg.seq)
    announce("350M: oracle, 8 rows")
    ref_loss, G = oracle_pool.batch_loss_and_grads(p, x, y, cfg.n_head, [1.0 / cfg.batch] * cfg.batch,
                                                   procs=_workers(16, 4), threads=4, label="350M B=8")
    check_bf16(names, grads, G, loss, ref_loss, "350M B=8")


@pytest.mark.timeout(1200)
def test_gpt2_1p5b_full_depth_b4_accum4():
    cfg = configs.GPT2_1P5B
    B, T, A = cfg.batch, cfg.seq, cfg.accum
    period = 5
    base = synthetic.zipf_eot_stream(period * T, cfg.vocab, seed=0)
    reps = (A * B + period) // period + 1
    stream = np.tile(base, reps)[:A * B * T + 1]  # row i of the stream is base row i mod 5
    p = init_for(cfg)
    announce("1.5B L=48 B=4 x 4 micro-steps")
    loss, grads, names = gpu_step(cfg, p, stream, [k * B * T for k in range(A)])
    counts = np.bincount([(k * B + b) % period for k in range(A) for b in range(B)], minlength=period)
    assert counts.tolist() == [4, 3, 3, 3, 3]
    ext = np.concatenate([base, base[:1]])  # the last row's extra target wraps to the first token
    x, y = oracle.make_batch(ext, 0, period, T)
    announce("1.5B: oracle, 5 distinct rows")
    ref_loss, G = oracle_pool.batch_loss_and_grads(p, x, y, cfg.n_head, counts / (A * B),
                                                   procs=_workers(60, 3), threads=5, label="1.5B")
    check_bf16(names, grads, G, loss, ref_loss, "1.5B B=4x4")


@pytest.mark.timeout(900)
def test_lmhead_full_size_vs_oracle():
    import torch
    N, V, C = 65536, 50257, 768
    X, W, y = synthetic.lmhead_inputs(N, V, C, seed=1)
    announce("LM head N=65536 V=50257 C=768")
    Xd = torch.from_numpy(synthetic.bf16_bits(X).view(np.int16)).cuda()
    Wd = torch.from_numpy(synthetic.bf16_bits(W).view(np.int16)).cuda()
    yd = torch.from_numpy(np.ascontiguousarray(y, np.int32)).cuda()
    loss, dX, dW = binding.lmhead_ce(Xd, Wd, yd, binding.GPT_BF16)
    loss, dX, dW = loss.item(), dX.cpu().numpy(), dW.cpu().numpy()
    del Xd, Wd, yd
    announce("LM head: oracle, 16 chunks of 4096 rows")
    rl, rdX, rdW = oracle_pool.lmhead_loss_and_grads(X, W, y, chunk=4096, procs=_workers(10, 4), threads=4)
    announce(f"LM head: loss {loss:.5f} vs {rl:.5f}; cos dX {cosine(dX, rdX):.6f} dW {cosine(dW, rdW):.6f}")
    assert abs(loss - rl) <= 2e-2
    assert cosine(dX, rdX) >= 0.999
    assert cosine(dW, rdW) >= 0.999
    for a, b in ((dX, rdX), (dW, rdW)):
        assert abs(np.linalg.norm(a) - np.linalg.norm(b)) <= 0.02 * np.linalg.norm(b)
    # every row's gradient: a dropped or doubled chunk of rows would show here
    rc = np.einsum("ij,ij->i", dX.astype(np.float64), rdX) / (
        np.linalg.norm(dX, axis=1) * np.linalg.norm(rdX, axis=1) + 1e-300)
    assert rc.min() >= 0.99, rc.min()
