"""Tiny fp32 model on the GPU against the fp64 oracle (1e-4 relative), plus
batch construction, causality, determinism, accumulation, clipping and the
error paths of the C ABI."""
import math

import numpy as np
import pytest

import oracle
from decoder_only_transformer_train_amd import binding, configs, synthetic
from gpu_util import announce, context, cosine, init_for, rel_err

pytestmark = pytest.mark.gpu

CFG = configs.TINY_F32
ADAM = dict(lr=6e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def tiny_inputs(seed=0, n_extra=0):
    p = init_for(CFG, seed)
    toks = synthetic.uniform_tokens(CFG.batch * CFG.seq + 1 + n_extra, CFG.vocab, seed=seed)
    return p, toks


def test_tiny_fp32_full_step_matches_oracle():
    announce("tiny fp32 step vs oracle")
    p, toks = tiny_inputs()
    g = context(CFG, p)
    g.make_batch(toks, 0)
    loss = g.forward_loss(1.0)
    g.backward()
    grads = g.get_all(binding.GRAD)
    x, y = oracle.make_batch(toks, 0, CFG.batch, CFG.seq)
    ref = oracle.train_step(p, x, y, CFG.n_head, **{"lr": 6e-4, "betas": (0.9, 0.95), "eps": 1e-8,
                                                     "weight_decay": 0.1})
    assert abs(loss - ref["loss"]) <= 1e-4 * abs(ref["loss"])
    np.testing.assert_allclose(g.token_losses(), ref["per_row"], rtol=1e-4, atol=1e-5)
    for k in g.names:
        assert rel_err(grads[k], ref["grads"][k]) <= 1e-4, (k, rel_err(grads[k], ref["grads"][k]))
    gn = g.adamw_step(**ADAM)
    assert abs(gn - oracle.grad_norm(ref["grads"])) <= 1e-4 * gn
    for k in g.names:
        new = g.get(k)
        assert rel_err(new - p[k], ref["params"][k] - p[k]) <= 1e-3, k
        assert rel_err(g.get(k, binding.ADAM_M), ref["m"][k]) <= 1e-4, k
        assert rel_err(g.get(k, binding.ADAM_V), ref["v"][k]) <= 2e-4, k
    assert g.step_count() == 1
    # gradients read as cleared after the update
    assert not np.any(g.get("h0.fc.w", binding.GRAD))


def test_fp32_head_forms_agree_with_oracle(monkeypatch):
    """fp32 contexts run the LM head as column-block fp32 MFMA products (the
    default); the fused plain-FMA kernels stay selectable with GPT_HEAD_DW=kernel
    (read when the context is laid out and at each step).  Both match the oracle
    and each other."""
    announce("tiny fp32 step, both forms of the LM head")
    p, toks = tiny_inputs(seed=3)
    x, y = oracle.make_batch(toks, 0, CFG.batch, CFG.seq)
    ref_loss, _, ref = oracle.loss_and_grads(p, x, y, CFG.n_head)
    out = {}
    for form in ("gemm", "kernel"):
        if form == "kernel":
            monkeypatch.setenv("GPT_HEAD_DW", "kernel")
        g = context(CFG, p)
        g.make_batch(toks, 0)
        loss = g.forward_loss(1.0)
        g.backward()
        out[form] = (loss, g.token_losses(), g.get_all(binding.GRAD))
        g.close()
        assert abs(loss - ref_loss) <= 1e-4 * abs(ref_loss), form
        for k in ref:
            assert rel_err(out[form][2][k], ref[k]) <= 1e-4, (form, k)
    np.testing.assert_allclose(out["gemm"][1], out["kernel"][1], rtol=1e-5, atol=1e-6)
    assert rel_err(out["gemm"][2]["wte"], out["kernel"][2]["wte"]) <= 1e-5


def test_two_steps_match_oracle():
    announce("tiny two steps")
    p, toks = tiny_inputs(seed=3, n_extra=CFG.batch * CFG.seq)
    g = context(CFG, p)
    x0, y0 = oracle.make_batch(toks, 0, CFG.batch, CFG.seq)
    r1 = oracle.train_step(p, x0, y0, CFG.n_head)
    start = binding.next_start(0, len(toks), CFG.batch, CFG.seq)
    x1, y1 = oracle.make_batch(toks, start, CFG.batch, CFG.seq)
    r2 = oracle.train_step(r1["params"], x1, y1, CFG.n_head, m=r1["m"], v=r1["v"], t=2)
    for s in (0, start):
        g.make_batch(toks, s)
        g.forward_loss(1.0)
        g.backward()
        g.adamw_step(**ADAM)
    for k in g.names:
        assert rel_err(g.get(k) - r1["params"][k], r2["params"][k] - r1["params"][k]) <= 2e-3, k
    losses = g.read_losses()
    assert len(losses) == 2
    assert abs(losses[1] - r2["loss"]) <= 1e-4 * r2["loss"]


def test_make_batch_bit_exact_and_errors():
    announce("make_batch")
    p, _ = tiny_inputs()
    g = context(CFG, p)
    stream = synthetic.uniform_tokens(5000, CFG.vocab, seed=9)
    rng = np.random.default_rng(1)
    for start in [0, 1, 17] + list(rng.integers(0, len(stream) - CFG.batch * CFG.seq - 1, 5)):
        g.make_batch(stream, int(start))
        x, y = g.get_batch()
        ex, ey = oracle.make_batch(stream, int(start), CFG.batch, CFG.seq)
        np.testing.assert_array_equal(x, ex)
        np.testing.assert_array_equal(y, ey)
    with pytest.raises(binding.GPTError) as e:
        g.make_batch(stream, len(stream) - CFG.batch * CFG.seq)
    assert e.value.code == binding.GPT_ERANGE
    bad = stream.copy()
    bad[40] = CFG.vocab
    with pytest.raises(binding.GPTError) as e:
        g.make_batch(bad, 0)
    assert e.value.code == binding.GPT_ERANGE
    bad[40] = -1
    with pytest.raises(binding.GPTError):
        g.make_batch(bad, 0)


def test_make_batch_copies_before_returning():
    """make_batch returns without waiting for the GPU (the window goes through a pinned
    staging buffer), yet the caller may overwrite its tokens at once: batches queued
    back to back, each followed by an overwrite of the caller's array, are the
    windows that were passed, and a forward queued behind them sees the last one."""
    announce("make_batch staging")
    p, _ = tiny_inputs()
    g = context(CFG, p)
    stream = synthetic.uniform_tokens(3000, CFG.vocab, seed=11)
    n = CFG.batch * CFG.seq + 1
    for start in (0, 5, 333):
        buf = stream.copy()
        g.make_batch(buf, start)
        buf[:] = (buf + 1) % CFG.vocab  # the caller reuses its array straight away
        x, y = g.get_batch()
        ex, ey = oracle.make_batch(stream, start, CFG.batch, CFG.seq)
        np.testing.assert_array_equal(x, ex)
        np.testing.assert_array_equal(y, ey)
    # three windows queued without a synchronisation in between (two staging buffers
    # alternate), the last one feeds the forward
    for start in (7, 70, 700):
        buf = stream[start:start + n].copy()
        g.make_batch(buf, 0)
        buf[:] = 0
    loss = g.forward_loss(1.0)
    x, y = oracle.make_batch(stream, 700, CFG.batch, CFG.seq)
    ref_loss, _, _ = oracle.loss_and_grads(p, x, y, CFG.n_head)
    assert abs(loss - ref_loss) <= 1e-4 * ref_loss, (loss, ref_loss)


def test_causality_on_gpu():
    announce("causality")
    p, toks = tiny_inputs()
    g = context(CFG, p)
    g.make_batch(toks, 0)
    g.forward_loss(0.0)
    base = g.token_losses()
    t0 = 11
    toks2 = toks.copy()
    b = 2
    toks2[b * CFG.seq + t0 + 1: (b + 1) * CFG.seq + 1] = (toks2[b * CFG.seq + t0 + 1:(b + 1) * CFG.seq + 1] + 5) % CFG.vocab
    g.make_batch(toks2, 0)
    g.forward_loss(0.0)
    pert = g.token_losses()
    # inputs x[b, t0+1:] and targets from t0 on changed; losses at t < t0 are unchanged bit for bit
    np.testing.assert_array_equal(pert[b, :t0], base[b, :t0])
    assert np.abs(pert[b, t0:] - base[b, t0:]).max() > 0
    for r in range(CFG.batch):
        if r != b and r != b + 1:
            np.testing.assert_array_equal(pert[r], base[r])


def test_determinism_bit_identical():
    announce("determinism")
    p, toks = tiny_inputs()
    out = []
    for _ in range(2):
        g = context(CFG, p)
        g.make_batch(toks, 0)
        g.forward_loss(1.0)
        g.backward()
        out.append(g.get_all(binding.GRAD))
        g.close()
    for k in out[0]:
        np.testing.assert_array_equal(out[0][k], out[1][k])


def test_accumulation_two_micro_steps():
    announce("accumulation")
    cfg = CFG.with_(batch=2)
    p, toks = tiny_inputs()
    g = context(cfg, p)
    ls = []
    for s in (0, 64):
        g.make_batch(toks, s)
        ls.append(g.forward_loss(0.5))
        g.backward()
    grads = g.get_all(binding.GRAD)
    x, y = oracle.make_batch(toks, 0, CFG.batch, CFG.seq)  # the same 4 rows in one batch
    loss, _, G = oracle.loss_and_grads(p, x, y, CFG.n_head)
    assert abs(np.mean(ls) - loss) <= 1e-4 * loss
    for k in g.names:
        assert rel_err(grads[k], G[k]) <= 1e-4, k


def test_clip_and_grad_norm():
    announce("clip")
    p, toks = tiny_inputs()
    x, y = oracle.make_batch(toks, 0, CFG.batch, CFG.seq)
    ref = oracle.train_step(p, x, y, CFG.n_head, grad_clip=0.05)
    assert ref["grad_norm"] > 0.05  # the clip is active
    g = context(CFG, p)
    g.make_batch(toks, 0)
    g.forward_loss(1.0)
    g.backward()
    gn = g.adamw_step(grad_clip=0.05, **ADAM)
    assert abs(gn - ref["grad_norm"]) <= 1e-4 * gn
    for k in g.names:
        assert rel_err(g.get(k, binding.ADAM_M), ref["m"][k]) <= 1e-4, k


def test_nonfinite_loss_and_grad_are_errors():
    announce("non-finite")
    p, toks = tiny_inputs()
    bad = dict(p)
    w = p["h1.fc.w"].copy()
    w[3, 5] = np.nan
    bad["h1.fc.w"] = w
    g = context(CFG, bad)
    g.make_batch(toks, 0)
    with pytest.raises(binding.GPTError) as e:
        g.forward_loss(1.0)
    assert e.value.code == binding.GPT_ENONFINITE
    g.backward()
    before = g.get("h0.attn.w")
    with pytest.raises(binding.GPTError) as e:
        g.adamw_step(**ADAM)
    assert e.value.code == binding.GPT_ENONFINITE
    np.testing.assert_array_equal(g.get("h0.attn.w"), before)
    assert g.step_count() == 0
    assert not np.all(np.isfinite(g.get("h1.fc.w", binding.GRAD)))


def test_backward_without_forward_is_einval():
    p, toks = tiny_inputs()
    g = context(CFG, p)
    with pytest.raises(binding.GPTError) as e:
        g.backward()
    assert e.value.code == binding.GPT_EINVAL
    g.make_batch(toks, 0)
    g.forward_loss(0.0)
    with pytest.raises(binding.GPTError):
        g.backward()


def test_device_init_statistics():
    announce("device init")
    g = binding.GPT(configs.TINY_F32.with_(n_layer=4, n_embd=256, padded_vocab=4096, vocab=4096), seed=7)
    w = g.get("wte")
    assert abs(w.mean()) < 1e-3 and abs(w.std() - 0.02) < 5e-4
    r = g.get("h2.mlp_proj.w")
    assert abs(r.std() - 0.02 / math.sqrt(8)) < 0.03 * 0.02 / math.sqrt(8)
    assert (g.get("h1.ln2.g") == 1).all() and (g.get("h3.fc.b") == 0).all()
    g2 = binding.GPT(configs.TINY_F32.with_(n_layer=4, n_embd=256, padded_vocab=4096, vocab=4096), seed=7)
    np.testing.assert_array_equal(g2.get("h2.attn.w"), g.get("h2.attn.w"))
    names = [n for n, _, _ in synthetic.tensor_layout(4, 256, 4096, 32)]
    assert g.names == names


def test_large_batch_chunked_token_sort():
    """B*T = 40960 tokens (three 16384-token sort chunks, the last one partial): the
    embedding gradient goes through the chunked sort and its merge; every gradient
    matches the oracle, and two identical steps give bit-identical gradients."""
    cfg = CFG.with_(batch=1280)
    announce(f"tiny fp32, B*T = {cfg.batch * cfg.seq}: chunked token sort")
    p = init_for(cfg, 0)
    toks = synthetic.uniform_tokens(cfg.batch * cfg.seq + 1, cfg.vocab, seed=5)
    runs = []
    for _ in range(2):
        g = context(cfg, p)
        g.make_batch(toks, 0)
        loss = g.forward_loss(1.0)
        g.backward()
        runs.append((loss, g.get_all(binding.GRAD)))
        g.close()
    (loss, grads), (loss2, grads2) = runs
    assert loss2 == loss
    for k in grads:
        np.testing.assert_array_equal(grads2[k], grads[k], err_msg=k)
    x, y = oracle.make_batch(toks, 0, cfg.batch, cfg.seq)
    ref_loss, _, ref = oracle.loss_and_grads(p, x, y, cfg.n_head)
    assert abs(loss - ref_loss) <= 1e-4 * ref_loss, (loss, ref_loss)
    for k in grads:
        assert rel_err(grads[k], ref[k]) <= 1e-4, (k, rel_err(grads[k], ref[k]))
