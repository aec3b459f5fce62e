"""ctypes binding of libgpt.so (include/gpt.h): argument marshalling only.

Every step of the training step runs in the library's HIP kernels; torch is
used here only to own the device arena / workspaces and to hand over the
current HIP stream.  Importing this module does not need a GPU; creating a
GPT context does.  A missing library raises instead of falling back.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_uint64, c_void_p

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgpt.so")

GPT_OK, GPT_EINVAL, GPT_ERANGE, GPT_ENOMEM, GPT_EHIP, GPT_ENONFINITE = 0, -1, -2, -3, -4, -5
GPT_F32, GPT_BF16 = 0, 1
PARAM, GRAD, ADAM_M, ADAM_V = 0, 1, 2, 3

EXPORTS = [
    "gpt_arena_bytes", "gpt_init", "gpt_destroy", "gpt_make_batch", "gpt_next_start",
    "gpt_forward_loss", "gpt_backward", "gpt_adamw_step", "gpt_lmhead_ce_ws_bytes", "gpt_lmhead_ce",
    "gpt_lmhead_ce_noalloc",
    "gpt_num_tensors", "gpt_tensor_info", "gpt_get_tensor", "gpt_set_tensor",
    "gpt_get_batch", "gpt_get_token_losses", "gpt_read_losses", "gpt_step_count", "gpt_set_step_count",
    "gpt_profile_begin",
    "gpt_profile_end", "gpt_last_error",
]


class GPTConfigC(ctypes.Structure):
    _fields_ = [("n_layer", c_int32), ("n_embd", c_int32), ("n_head", c_int32),
                ("vocab", c_int32), ("padded_vocab", c_int32),
                ("max_seq", c_int32), ("batch", c_int32), ("seq", c_int32), ("dtype", c_int32),
                ("block", c_int32), ("d_ff", c_int32), ("rope_theta", ctypes.c_float)]


GPT_BLOCK_GPT2, GPT_BLOCK_RMS_ROPE_SWIGLU = 0, 1


class GPTError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


_lib = None


def load():
    """Load libgpt.so and declare its signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P = POINTER
    sig = {
        "gpt_arena_bytes": (c_size_t, [P(GPTConfigC)]),
        "gpt_init": (c_int, [P(GPTConfigC), c_void_p, c_size_t, c_void_p, c_uint64, P(c_void_p)]),
        "gpt_destroy": (c_int, [c_void_p]),
        "gpt_make_batch": (c_int, [c_void_p, c_void_p, c_int64, c_int64]),
        "gpt_next_start": (c_int64, [c_int64, c_int64, c_int32, c_int32, c_int32, c_int32]),
        "gpt_forward_loss": (c_int, [c_void_p, c_float, P(c_float)]),
        "gpt_backward": (c_int, [c_void_p]),
        "gpt_adamw_step": (c_int, [c_void_p, c_float, c_float, c_float, c_float, c_float, c_float, P(c_float)]),
        "gpt_lmhead_ce_ws_bytes": (c_size_t, [c_int64, c_int64, c_int64, c_int32]),
        "gpt_lmhead_ce": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int32,
                                  c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "gpt_lmhead_ce_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int32,
                                          c_void_p, c_void_p, c_void_p, c_void_p]),
        "gpt_num_tensors": (c_int, [c_void_p]),
        "gpt_tensor_info": (c_int, [c_void_p, c_int, P(c_char_p), P(c_int64), P(c_int)]),
        "gpt_get_tensor": (c_int, [c_void_p, c_int, c_int, c_void_p, c_int64]),
        "gpt_set_tensor": (c_int, [c_void_p, c_int, c_int, c_void_p, c_int64]),
        "gpt_get_batch": (c_int, [c_void_p, c_void_p, c_void_p, c_int64]),
        "gpt_get_token_losses": (c_int, [c_void_p, c_void_p, c_int64]),
        "gpt_read_losses": (c_int, [c_void_p, c_void_p, c_int]),
        "gpt_step_count": (c_int64, [c_void_p]),
        "gpt_set_step_count": (c_int, [c_void_p, c_int64]),
        "gpt_profile_begin": (c_int, [c_void_p, c_char_p]),
        "gpt_profile_end": (c_int, [c_void_p, P(c_double), P(c_int64), P(c_double), P(c_double)]),
        "gpt_last_error": (c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(rc: int) -> int:
    if rc < 0:
        raise GPTError(rc, load().gpt_last_error().decode())
    return rc


def next_start(pos: int, n_tokens: int, B: int, T: int, rank: int = 0, world: int = 1) -> int:
    return _check(load().gpt_next_start(pos, n_tokens, B, T, rank, world))


def arena_bytes(cfg) -> int:
    return int(load().gpt_arena_bytes(byref(cfg.to_c())))


class GPT:
    """One training context: the caller-owned device arena plus the library handle."""

    def __init__(self, cfg, seed: int = 0, device: str = "cuda:0", stream=None):
        import torch
        lib = load()
        self.cfg = cfg
        self._c = cfg.to_c()
        n = int(lib.gpt_arena_bytes(byref(self._c)))
        if n == 0:
            _check(lib.gpt_init(byref(self._c), None, 0, None, 0, byref(c_void_p())))
        self.device = torch.device(device)
        self.arena = torch.empty(n, dtype=torch.uint8, device=self.device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        ctx = c_void_p()
        _check(lib.gpt_init(byref(self._c), c_void_p(self.arena.data_ptr()), n,
                            c_void_p(self.stream.cuda_stream), seed, byref(ctx)))
        self._ctx = ctx
        self.names = []
        self.shapes = {}
        self.decays = {}
        for i in range(_check(lib.gpt_num_tensors(ctx))):
            nm = c_char_p()
            shp = (c_int64 * 2)()
            dec = c_int()
            _check(lib.gpt_tensor_info(ctx, i, byref(nm), shp, byref(dec)))
            name = nm.value.decode()
            self.names.append(name)
            self.shapes[name] = (shp[0], shp[1]) if shp[1] else (shp[0],)
            self.decays[name] = bool(dec.value)
        self.ids = {n: i for i, n in enumerate(self.names)}

    def close(self):
        if getattr(self, "_ctx", None) is not None:
            load().gpt_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- the step ----
    def make_batch(self, tokens: np.ndarray, start: int):
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(load().gpt_make_batch(self._ctx, tokens.ctypes.data, len(tokens), start))

    def forward_loss(self, loss_scale: float = 1.0, sync: bool = True):
        out = c_float()
        _check(load().gpt_forward_loss(self._ctx, loss_scale, byref(out) if sync else None))
        return out.value if sync else None

    def backward(self):
        _check(load().gpt_backward(self._ctx))

    def adamw_step(self, lr=6e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_clip=0.0,
                   sync: bool = True):
        out = c_float()
        _check(load().gpt_adamw_step(self._ctx, lr, beta1, beta2, eps, weight_decay, grad_clip,
                                     byref(out) if sync else None))
        return out.value if sync else None

    # ---- tensors ----
    def get(self, name: str, kind: int = PARAM) -> np.ndarray:
        shape = self.shapes[name]
        a = np.empty(shape, dtype=np.float32)
        _check(load().gpt_get_tensor(self._ctx, kind, self.ids[name], a.ctypes.data, a.size))
        return a

    def set(self, name: str, value: np.ndarray, kind: int = PARAM):
        a = np.ascontiguousarray(value, dtype=np.float32)
        if a.shape != self.shapes[name]:
            raise ValueError(f"{name}: shape {a.shape} != {self.shapes[name]}")
        _check(load().gpt_set_tensor(self._ctx, kind, self.ids[name], a.ctypes.data, a.size))

    def set_params(self, params: dict):
        for k, v in params.items():
            self.set(k, v)

    def get_all(self, kind: int = PARAM) -> dict:
        return {n: self.get(n, kind) for n in self.names}

    def get_batch(self):
        x = np.empty((self.cfg.batch, self.cfg.seq), dtype=np.int32)
        y = np.empty_like(x)
        _check(load().gpt_get_batch(self._ctx, x.ctypes.data, y.ctypes.data, x.size))
        return x, y

    def token_losses(self) -> np.ndarray:
        a = np.empty((self.cfg.batch, self.cfg.seq), dtype=np.float32)
        _check(load().gpt_get_token_losses(self._ctx, a.ctypes.data, a.size))
        return a

    def read_losses(self, max_n: int = 4096) -> np.ndarray:
        a = np.empty(max_n, dtype=np.float32)
        k = _check(load().gpt_read_losses(self._ctx, a.ctypes.data, max_n))
        return a[:k]

    def step_count(self) -> int:
        return _check(load().gpt_step_count(self._ctx))

    def set_step_count(self, t: int):
        _check(load().gpt_set_step_count(self._ctx, int(t)))

    # ---- timing ----
    def profile_begin(self, cls: str):
        _check(load().gpt_profile_begin(self._ctx, cls.encode()))

    def profile_end(self):
        ms, n, fl, by = c_double(), c_int64(), c_double(), c_double()
        _check(load().gpt_profile_end(self._ctx, byref(ms), byref(n), byref(fl), byref(by)))
        return dict(ms=ms.value, launches=n.value, flops=fl.value, bytes=by.value)


class LMHead:
    """Buffers for repeated gpt_lmhead_ce calls of one shape: workspace, loss [1], dX [N, C], dW [V, C]."""

    def __init__(self, N: int, V: int, C: int, dtype: int, want_grads: bool = True, device="cuda:0"):
        import torch
        lib = load()
        self.N, self.V, self.C, self.dtype = N, V, C, dtype
        self.ws_n = int(lib.gpt_lmhead_ce_ws_bytes(N, V, C, dtype))
        if self.ws_n == 0:
            raise GPTError(GPT_EINVAL, "bad lmhead_ce shape")
        self.ws = torch.empty(self.ws_n, dtype=torch.uint8, device=device)
        self.loss = torch.empty(1, dtype=torch.float32, device=device)
        self.dX = torch.empty((N, C), dtype=torch.float32, device=device) if want_grads else None
        self.dW = torch.empty((V, C), dtype=torch.float32, device=device) if want_grads else None

    def __call__(self, X, W, y, stream=None):
        import torch
        if tuple(X.shape) != (self.N, self.C) or tuple(W.shape) != (self.V, self.C) or y.numel() != self.N:
            raise ValueError("lmhead_ce: shapes do not match the buffers")
        s = stream if stream is not None else torch.cuda.current_stream(X.device)
        ptr = lambda t: c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
        _check(load().gpt_lmhead_ce(ptr(X), ptr(W), ptr(y), self.N, self.V, self.C, self.dtype, ptr(self.loss),
                                    ptr(self.dX), ptr(self.dW), ptr(self.ws), self.ws_n, c_void_p(s.cuda_stream)))
        return self.loss, self.dX, self.dW


def lmhead_ce_noalloc(X, W, y, dtype: int, loss, dX=None, dW=None, stream=None):
    """gpt_lmhead_ce_noalloc on caller tensors: X [N, C], W [V, C], y int32 [N] and the
    fp32 outputs loss [1], dX [N, C] (or None), dW [V, C] (or None); nothing is allocated."""
    import torch
    N, C = X.shape
    V = W.shape[0]
    if y.numel() != N or loss.numel() < 1 or (dX is not None and tuple(dX.shape) != (N, C)) or \
            (dW is not None and tuple(dW.shape) != (V, C)):
        raise ValueError("lmhead_ce_noalloc: shapes do not match")
    s = stream if stream is not None else torch.cuda.current_stream(X.device)
    ptr = lambda t: c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    _check(load().gpt_lmhead_ce_noalloc(ptr(X), ptr(W), ptr(y), N, V, C, dtype, ptr(loss), ptr(dX), ptr(dW),
                                        c_void_p(s.cuda_stream)))
    return loss, dX, dW


def lmhead_ce(X, W, y, dtype: int, want_grads: bool = True, stream=None):
    """Fused LM head + CE on device tensors X [N, C], W [V, C] (fp32, or bf16 bits as int16/bf16), y int32 [N].

    Returns (loss tensor [1], dX [N, C] or None, dW [V, C] or None), all fp32 device tensors.
    """
    N, C = X.shape
    V = W.shape[0]
    return LMHead(N, V, C, dtype, want_grads, device=X.device)(X, W, y, stream)
