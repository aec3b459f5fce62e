"""Helpers shared by the GPU tests (device contexts, comparison metrics)."""
import os
import time

import numpy as np

from decoder_only_transformer_train_amd import binding, synthetic


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def cosine(a, b):
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if nb == 0:
        return 1.0 if na <= 1e-6 else 0.0
    return float(a @ b / (na * nb + 1e-300))


def context(cfg, params=None, seed=0):
    g = binding.GPT(cfg, seed=seed)
    if params is not None:
        g.set_params(params)
    return g


def init_for(cfg, seed=0, gain_jitter=0.0):
    if cfg.block == binding.GPT_BLOCK_RMS_ROPE_SWIGLU:
        return synthetic.init_params_cs336(cfg.n_layer, cfg.n_embd, cfg.d_ff, cfg.padded_vocab, seed=seed,
                                           gain_jitter=gain_jitter)
    return synthetic.init_params(cfg.n_layer, cfg.n_embd, cfg.padded_vocab, cfg.max_seq, seed=seed)


_PROGRESS = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out",
                         "gpu_test_progress.log")


def announce(msg):
    """Print a progress line, and append it to a log that shows a long test is alive."""
    line = f"[gpu-test {time.strftime('%H:%M:%S')}] {msg}"
    print(line, flush=True)
    try:
        os.makedirs(os.path.dirname(_PROGRESS), exist_ok=True)
        with open(_PROGRESS, "a") as f:
            f.write(line + "\n")
    except OSError:
        pass
