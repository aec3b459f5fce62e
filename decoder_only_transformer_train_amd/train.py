"""Multi-step training on the library's step: schedule, clipping, validation, checkpoints.

The loop is the pages' (CS336 pretraining page, section 3, full loop; the
lecture's optimisation loop; "GPT training" (Zero), training loop):

    lr = schedule(step) -> per micro-step: batch, forward + loss, backward
    -> clip the global gradient norm -> AdamW -> (validate) -> (checkpoint)

  * learning rate: linear warm-up from 0, then a half cosine down to min_lr
    at `total` steps, constant after (CS336 page, section 2, learning-rate
    schedule; the lecture's schedule decays to about 10% of the 6e-4 peak);
    the schedule's step counts from 0, AdamW's bias-correction counter from 1;
  * gradient clipping at a global norm of 1.0 (lecture, gradient clipping);
    a non-finite loss or gradient norm raises (CS336 page, section 3);
  * validation: the same fixed windows from the start of the held-out stream
    every time (the loader is reset), forward only, mean loss over them
    ("Chapter 28", 28.4: a fixed set of validation batches; equal token
    counts per batch, so the mean of batch means is the token mean);
  * checkpoints hold everything the next update depends on ("Chapter 28",
    28.6): parameters, AdamW m and v, the update counter t, the index of the
    next schedule step, the schedule, the data cursor and a hash of the token
    stream.  No random numbers are drawn in a step (no dropout; the data
    cursor is deterministic), so there is no generator state to keep.  Files
    are .npz archives of plain arrays (the metadata is a JSON string stored
    as bytes) and load without unpickling anything.

Every number crunched here is a host scalar; the step itself runs in libgpt.so.
"""
from __future__ import annotations

import hashlib
import json
import math
import time
from dataclasses import asdict, dataclass

import numpy as np

from . import binding


def cosine_lr(step: int, max_lr: float, min_lr: float, warmup: int, total: int) -> float:
    """Warm-up then cosine decay; `step` counts from 0."""
    if not 0 <= warmup < total:
        raise ValueError("the schedule needs 0 <= warmup < total")
    if step >= total:
        return min_lr
    if step < warmup:
        return max_lr * step / warmup
    progress = (step - warmup) / (total - warmup)
    return min_lr + (max_lr - min_lr) * (1.0 + math.cos(math.pi * progress)) / 2.0


@dataclass
class Schedule:
    max_lr: float = 6e-4
    min_lr: float = 6e-5
    warmup: int = 10
    total: int = 100

    def lr(self, step: int) -> float:
        return cosine_lr(step, self.max_lr, self.min_lr, self.warmup, self.total)


@dataclass
class OptimConfig:
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    grad_clip: float = 1.0


def stream_digest(tokens: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(tokens, dtype=np.int32).tobytes()).hexdigest()


class Trainer:
    """Training loop over one GPT context and a token stream (see the module notes)."""

    def __init__(self, gpt: "binding.GPT", train_tokens: np.ndarray, val_tokens: np.ndarray | None = None,
                 schedule: Schedule | None = None, optim: OptimConfig | None = None, accum: int = 1,
                 val_batches: int = 20):
        if accum < 1 or val_batches < 0:
            raise ValueError("accum >= 1 and val_batches >= 0")
        self.gpt = gpt
        self.cfg = gpt.cfg
        self.train_tokens = np.ascontiguousarray(train_tokens, dtype=np.int32)
        self.val_tokens = None if val_tokens is None else np.ascontiguousarray(val_tokens, dtype=np.int32)
        self.schedule = schedule or Schedule()
        self.optim = optim or OptimConfig()
        self.accum = accum
        self.val_batches = val_batches
        self.next_step = 0  # index of the next schedule step
        self.pos = 0        # data cursor: start of the next training window
        self.t0 = time.perf_counter()

    @property
    def tokens_per_step(self) -> int:
        return self.accum * self.cfg.batch * self.cfg.seq

    def step(self) -> dict:
        """One optimiser step; returns its record."""
        g, B, T = self.gpt, self.cfg.batch, self.cfg.seq
        lr = self.schedule.lr(self.next_step)
        losses = []
        for _ in range(self.accum):
            g.make_batch(self.train_tokens, self.pos)
            losses.append(g.forward_loss(1.0 / self.accum))  # raises on a non-finite loss
            g.backward()
            self.pos = binding.next_start(self.pos, len(self.train_tokens), B, T)
        o = self.optim
        norm = g.adamw_step(lr=lr, beta1=o.beta1, beta2=o.beta2, eps=o.eps, weight_decay=o.weight_decay,
                            grad_clip=o.grad_clip)  # raises on a non-finite norm (update skipped)
        self.next_step += 1
        return {"step": self.next_step, "tokens": self.next_step * self.tokens_per_step,
                "seconds": time.perf_counter() - self.t0, "train_loss": float(np.mean(losses)), "lr": lr,
                "grad_norm": norm}

    def validate(self) -> float:
        """Mean loss over the first val_batches windows of the held-out stream (forward only)."""
        if self.val_tokens is None or self.val_batches == 0:
            raise ValueError("no validation stream")
        g, B, T = self.gpt, self.cfg.batch, self.cfg.seq
        pos, out = 0, []
        for _ in range(self.val_batches):
            g.make_batch(self.val_tokens, pos)
            out.append(g.forward_loss(0.0))
            pos = binding.next_start(pos, len(self.val_tokens), B, T)
        return float(np.mean(out))

    def run(self, steps: int, val_every: int = 0, log=None) -> list:
        """`steps` optimiser steps; validation every val_every steps and after the last one."""
        recs = []
        for i in range(steps):
            r = self.step()
            last = i == steps - 1
            if self.val_tokens is not None and self.val_batches and (last or (val_every and r["step"] % val_every == 0)):
                r["val_loss"] = self.validate()
            recs.append(r)
            if log is not None:
                log.write(json.dumps(r) + "\n")
                log.flush()
        return recs

    # ---- checkpoints ----
    def state(self) -> tuple[dict, dict]:
        """(arrays, metadata) of everything the next update depends on."""
        g = self.gpt
        arrays = {}
        for kind, tag in ((binding.PARAM, "param"), (binding.ADAM_M, "m"), (binding.ADAM_V, "v")):
            for n, a in g.get_all(kind).items():
                arrays[f"{tag}/{n}"] = a
        meta = {"format": 1, "config": asdict(self.cfg), "adam_t": g.step_count(), "next_step": self.next_step,
                "pos": self.pos, "accum": self.accum, "schedule": asdict(self.schedule),
                "optim": asdict(self.optim), "val_batches": self.val_batches,
                "train_stream": {"n": int(len(self.train_tokens)), "sha256": stream_digest(self.train_tokens)}}
        return arrays, meta

    def save(self, path: str):
        arrays, meta = self.state()
        write_checkpoint(path, arrays, meta)

    def load(self, path: str):
        arrays, meta = read_checkpoint(path)
        if meta.get("format") != 1:
            raise ValueError("unknown checkpoint format")
        if meta["config"] != asdict(self.cfg):
            raise ValueError("checkpoint was written for another model configuration")
        ts = meta["train_stream"]
        if ts["n"] != len(self.train_tokens) or ts["sha256"] != stream_digest(self.train_tokens):
            raise ValueError("checkpoint was written for another token stream")
        g = self.gpt
        for kind, tag in ((binding.PARAM, "param"), (binding.ADAM_M, "m"), (binding.ADAM_V, "v")):
            for n in g.names:
                g.set(n, arrays[f"{tag}/{n}"], kind)
        g.set_step_count(meta["adam_t"])
        self.next_step = meta["next_step"]
        self.pos = meta["pos"]
        self.accum = meta["accum"]
        self.schedule = Schedule(**meta["schedule"])
        self.optim = OptimConfig(**meta["optim"])
        self.val_batches = meta["val_batches"]
        return meta


def write_checkpoint(path: str, arrays: dict, meta: dict):
    """arrays (name -> ndarray) and JSON-able metadata into one .npz file."""
    if "__meta__" in arrays:
        raise ValueError("reserved array name")
    blob = np.frombuffer(json.dumps(meta, sort_keys=True).encode(), dtype=np.uint8)
    with open(path, "wb") as f:
        np.savez(f, __meta__=blob, **arrays)


def read_checkpoint(path: str) -> tuple[dict, dict]:
    with np.load(path, allow_pickle=False) as z:
        meta = json.loads(bytes(z["__meta__"]).decode())
        arrays = {k: z[k] for k in z.files if k != "__meta__"}
    return arrays, meta
