"""Host logic of the multi-step driver: schedule against the oracle's, checkpoint files,
and the oracle's own loop overfitting one batch (CS336 page, section 3: before a real run,
train one fixed small batch and the loss must go far down)."""
import numpy as np
import pytest

import oracle
from decoder_only_transformer_train_amd import configs, synthetic, train


@pytest.mark.parametrize("mx,mn,wu,tot", [(6e-4, 6e-5, 10, 100), (1e-3, 1e-4, 0, 7), (3e-3, 0.0, 5, 6),
                                          (6e-4, 6e-5, 715, 19073)])
def test_schedule_matches_oracle(mx, mn, wu, tot):
    for t in list(range(0, min(tot + 3, 400))) + [tot - 1, tot, tot + 1, 10 * tot]:
        assert train.cosine_lr(t, mx, mn, wu, tot) == pytest.approx(oracle.lr_schedule(t, mx, mn, wu, tot),
                                                                    rel=1e-14, abs=1e-20)
    with pytest.raises(ValueError):
        train.cosine_lr(0, mx, mn, tot, tot)


def test_checkpoint_file_roundtrip(tmp_path):
    rng = np.random.default_rng(0)
    arrays = {"param/wte": rng.standard_normal((5, 3)).astype(np.float32),
              "m/h0.ln1.g": rng.standard_normal(7).astype(np.float32)}
    meta = {"format": 1, "adam_t": 17, "pos": 4097, "schedule": {"max_lr": 6e-4, "warmup": 3}}
    p = str(tmp_path / "ck.npz")
    train.write_checkpoint(p, arrays, meta)
    a2, m2 = train.read_checkpoint(p)
    assert m2 == meta
    assert set(a2) == set(arrays)
    for k in arrays:
        assert a2[k].dtype == np.float32
        np.testing.assert_array_equal(a2[k], arrays[k])


def test_oracle_loop_overfits_one_batch():
    cfg = configs.TINY_F32
    p = synthetic.init_params(cfg.n_layer, cfg.n_embd, cfg.padded_vocab, cfg.max_seq, seed=0)
    toks = synthetic.uniform_tokens(cfg.batch * cfg.seq + 1, cfg.vocab, seed=0)
    x, y = oracle.make_batch(toks, 0, cfg.batch, cfg.seq)
    m = v = None
    losses = []
    for t in range(60):
        lr = oracle.lr_schedule(t, 3e-3, 3e-4, 5, 60)
        r = oracle.train_step(p, x, y, cfg.n_head, lr=lr, grad_clip=1.0, m=m, v=v, t=t + 1)
        p, m, v = r["params"], r["m"], r["v"]
        losses.append(r["loss"])
    assert losses[0] > 5.0
    assert losses[-1] < 0.5 * losses[0]
