"""Plain fp64 CPU oracle of one GPT-2 training step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
bench's CPU-baseline leg may import this module.  It shares no code with the
HIP library and imports nothing from it.

Every function is the textbook definition written out in float64 NumPy, in
the order and notation the pages use; nothing is blocked, fused or reordered
beyond what that definition states.  Sources, by page title and section:

  [R]  "Andrej Karpathy: reproducing GPT-2 from scratch" (lecture summary),
       sections on the architecture, the data loader, initialisation,
       mixed precision, vocabulary padding, AdamW, weight decay groups,
       gradient accumulation and DDP.
  [D]  "Chapter 28 Data, evaluation and resume", section 28.3 (how B x T + 1
       tokens become one batch).
  [C]  "Implementing an LLM from scratch (CS336) - pretraining", section 1
       (training objective, cross-entropy), section 2 (AdamW, learning-rate
       schedule, gradient clipping), section 4 (resource accounting, FLOPs
       and MFU).
  [Z]  "GPT training" (Zero framework), sections autoregressive objective,
       Embedding, Attention, Transformer Block and output layer.

Readings where the pages are silent (each also listed in the design notes):
  * LayerNorm epsilon 1e-5 with the biased variance (no page states it).
  * GELU is the tanh approximation
      0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))
    (Hendrycks & Gimpel 2016); the lecture only says "approximate GELU".
  * The causal mask excludes j > i outright (the lecture's reading); the
    Zero page's -1e4 additive mask gives the same probabilities in fp64
    whenever |S| is far below 1e4.
  * Padded vocabulary rows are ordinary softmax classes (the lecture's
    vocabulary-padding section: the extra rows stay in the output
    distribution).
  * AdamW adds eps to sqrt(v) and folds bias correction into the step size,
    as in the CS336 page's optimiser code; weight decay applies to 2-D
    tensors only (the lecture's parameter-group section).
"""
from __future__ import annotations

import math

import numpy as np

LN_EPS = 1e-5
GELU_K = math.sqrt(2.0 / math.pi)
GELU_A = 0.044715


# --------------------------------------------------------------------------
# Batch construction  ([D] 28.3; [R] data loader; [Z] autoregressive objective)
# --------------------------------------------------------------------------

def make_batch(stream: np.ndarray, start: int, B: int, T: int):
    """x = window[:-1], y = window[1:] of the B*T+1 tokens at `start`, as [B, T].

    Raises ValueError when the window runs past the stream, as the data
    loader cannot serve a full batch there.
    """
    n = len(stream)
    if start < 0 or start + B * T + 1 > n:
        raise ValueError("window past the end of the token stream")
    w = np.asarray(stream[start:start + B * T + 1], dtype=np.int64)
    x = w[:-1].reshape(B, T)
    y = w[1:].reshape(B, T)
    return x, y


def next_start(pos: int, n: int, B: int, T: int, rank: int = 0, world: int = 1) -> int:
    """Cursor after one batch ([D] 28.3; [R] data loader and DDP sections).

    Rank r starts at B*T*r and advances by B*T*R; when the next full window
    (B*T*R tokens plus the one extra target) would not fit, it returns to
    its own starting offset.
    """
    step = B * T * world
    pos = pos + step
    if pos + step + 1 > n:
        pos = B * T * rank
    return pos


# --------------------------------------------------------------------------
# Layers ([Z] Embedding / Attention / Transformer Block / output layer; [R])
# --------------------------------------------------------------------------

def layernorm(h, g, b):
    """LN(z) = (z - mu) / sqrt(var + eps) * g + b over the last axis, biased var."""
    mu = h.mean(axis=-1, keepdims=True)
    var = ((h - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + LN_EPS)
    xhat = (h - mu) * rstd
    return xhat * g + b, (xhat, rstd)


def layernorm_backward(dout, xhat, rstd, g):
    """Chain rule of layernorm: returns dx, dg, db."""
    dxhat = dout * g
    dg = (dout * xhat).reshape(-1, xhat.shape[-1]).sum(axis=0)
    db = dout.reshape(-1, dout.shape[-1]).sum(axis=0)
    m1 = dxhat.mean(axis=-1, keepdims=True)
    m2 = (dxhat * xhat).mean(axis=-1, keepdims=True)
    dx = rstd * (dxhat - m1 - xhat * m2)
    return dx, dg, db


def gelu(u):
    return 0.5 * u * (1.0 + np.tanh(GELU_K * (u + GELU_A * u ** 3)))


def gelu_backward(du_out, u):
    t = np.tanh(GELU_K * (u + GELU_A * u ** 3))
    dt = GELU_K * (1.0 + 3.0 * GELU_A * u ** 2)
    return du_out * (0.5 * (1.0 + t) + 0.5 * u * (1.0 - t * t) * dt)


def causal_attention(q, k, v):
    """softmax(q k^T / sqrt(D) with j > i excluded) v for q, k, v [B, H, T, D]."""
    D = q.shape[-1]
    T = q.shape[-2]
    S = q @ np.swapaxes(k, -1, -2) / math.sqrt(D)
    future = np.triu(np.ones((T, T), dtype=bool), k=1)
    S = np.where(future, -np.inf, S)
    S = S - S.max(axis=-1, keepdims=True)
    E = np.exp(S)
    P = E / E.sum(axis=-1, keepdims=True)
    return P @ v, P


def causal_attention_backward(do, q, k, v, P):
    D = q.shape[-1]
    dv = np.swapaxes(P, -1, -2) @ do
    dP = do @ np.swapaxes(v, -1, -2)
    dS = P * (dP - (dP * P).sum(axis=-1, keepdims=True))
    dq = dS @ k / math.sqrt(D)
    dk = np.swapaxes(dS, -1, -2) @ q / math.sqrt(D)
    return dq, dk, dv


def cross_entropy_rows(z, y):
    """Per-row -log softmax(z)[y], with the row maximum subtracted first ([C] section 1)."""
    zmax = z.max(axis=-1, keepdims=True)
    lse = np.log(np.exp(z - zmax).sum(axis=-1)) + zmax[:, 0]
    return lse - z[np.arange(z.shape[0]), y], lse


def lmhead_ce(X, W, y, loss_scale: float = 1.0):
    """Tied LM head + mean cross-entropy, forward and backward.

    z = X W^T; loss = mean_n [logsumexp(z_n) - z_n[y_n]];
    dz = (softmax(z) - onehot(y)) * loss_scale / N; dX = dz W; dW = dz^T X.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    N = X.shape[0]
    z = X @ W.T
    per_row, lse = cross_entropy_rows(z, y)
    loss = per_row.mean()
    P = np.exp(z - lse[:, None])
    P[np.arange(N), y] -= 1.0
    dz = P * (loss_scale / N)
    return loss, per_row, dz @ W, dz.T @ X


# --------------------------------------------------------------------------
# Whole model
# --------------------------------------------------------------------------

def _n_layer(params):
    L = 0
    while f"h{L}.ln1.g" in params:
        L += 1
    return L


def forward(params, x, y, n_head: int, keep=True):
    """Forward pass and mean next-token loss ([Z] model; [R] architecture).

    params: name -> array (cast to float64 here); x, y int [B, T].
    Returns (loss, per_position_loss [B, T], cache).
    """
    P = {k: np.asarray(v, dtype=np.float64) for k, v in params.items()}
    L = _n_layer(P)
    B, T = x.shape
    C = P["wte"].shape[1]
    H = n_head
    D = C // H
    N = B * T
    cache = {"x": x, "y": y, "B": B, "T": T, "H": H, "L": L}
    # token + learned position embedding, positions restart at 0 in every row
    h = P["wte"][x] + P["wpe"][np.arange(T)][None, :, :]
    h = h.reshape(N, C)
    layers = []
    for l in range(L):
        p = f"h{l}."
        a, ln1 = layernorm(h, P[p + "ln1.g"], P[p + "ln1.b"])
        qkv = a @ P[p + "attn.w"].T + P[p + "attn.b"]
        q, k, v = (qkv[:, i * C:(i + 1) * C].reshape(B, T, H, D).transpose(0, 2, 1, 3)
                   for i in range(3))
        o, Pm = causal_attention(q, k, v)
        o = o.transpose(0, 2, 1, 3).reshape(N, C)
        h_mid = h + o @ P[p + "proj.w"].T + P[p + "proj.b"]
        m, ln2 = layernorm(h_mid, P[p + "ln2.g"], P[p + "ln2.b"])
        u = m @ P[p + "fc.w"].T + P[p + "fc.b"]
        gu = gelu(u)
        h_out = h_mid + gu @ P[p + "mlp_proj.w"].T + P[p + "mlp_proj.b"]
        if keep:
            layers.append(dict(a=a, ln1=ln1, q=q, k=k, v=v, P=Pm, o=o,
                               m=m, ln2=ln2, u=u, gu=gu))
        h = h_out
    f, lnf = layernorm(h, P["lnf.g"], P["lnf.b"])
    z = f @ P["wte"].T
    per_row, lse = cross_entropy_rows(z, y.reshape(-1))
    loss = per_row.mean()
    if keep:
        cache.update(layers=layers, f=f, lnf=lnf, z=z, lse=lse, P64=P)
    return loss, per_row.reshape(B, T), cache


def backward(cache, loss_scale: float = 1.0):
    """Gradients of loss_scale * loss for every parameter (chain rule).

    The head and the token embedding share one tensor, so its gradient is
    the sum of the head's and the embedding's parts ([R] weight tying).
    """
    P = cache["P64"]
    L, B, T, H = cache["L"], cache["B"], cache["T"], cache["H"]
    x, y = cache["x"], cache["y"].reshape(-1)
    N = B * T
    C = P["wte"].shape[1]
    D = C // H
    G = {k: np.zeros_like(v) for k, v in P.items()}
    # head + cross-entropy
    dz = np.exp(cache["z"] - cache["lse"][:, None])
    dz[np.arange(N), y] -= 1.0
    dz *= loss_scale / N
    G["wte"] += dz.T @ cache["f"]
    df = dz @ P["wte"]
    xhat, rstd = cache["lnf"]
    dh, G["lnf.g"], G["lnf.b"] = layernorm_backward(df, xhat, rstd, P["lnf.g"])
    for l in reversed(range(L)):
        p = f"h{l}."
        c = cache["layers"][l]
        # MLP branch: h_out = h_mid + gelu(u) Wp^T + bp
        G[p + "mlp_proj.w"] = dh.T @ c["gu"]
        G[p + "mlp_proj.b"] = dh.sum(axis=0)
        dgu = dh @ P[p + "mlp_proj.w"]
        du = gelu_backward(dgu, c["u"])
        G[p + "fc.w"] = du.T @ c["m"]
        G[p + "fc.b"] = du.sum(axis=0)
        dm = du @ P[p + "fc.w"]
        dx2, G[p + "ln2.g"], G[p + "ln2.b"] = layernorm_backward(dm, *c["ln2"], P[p + "ln2.g"])
        dh = dh + dx2
        # attention branch: h_mid = h + o Wo^T + bo
        G[p + "proj.w"] = dh.T @ c["o"]
        G[p + "proj.b"] = dh.sum(axis=0)
        do = (dh @ P[p + "proj.w"]).reshape(B, T, H, D).transpose(0, 2, 1, 3)
        dq, dk, dv = causal_attention_backward(do, c["q"], c["k"], c["v"], c["P"])
        dqkv = np.concatenate([t.transpose(0, 2, 1, 3).reshape(N, C) for t in (dq, dk, dv)],
                              axis=1)
        G[p + "attn.w"] = dqkv.T @ c["a"]
        G[p + "attn.b"] = dqkv.sum(axis=0)
        da = dqkv @ P[p + "attn.w"]
        dx1, G[p + "ln1.g"], G[p + "ln1.b"] = layernorm_backward(da, *c["ln1"], P[p + "ln1.g"])
        dh = dh + dx1
    # embedding: token rows scatter-add, positions summed over the batch
    dh = dh.reshape(B, T, C)
    np.add.at(G["wte"], x.reshape(-1), dh.reshape(N, C))
    G["wpe"][:T] += dh.sum(axis=0)
    return G


def loss_and_grads(params, x, y, n_head: int, loss_scale: float = 1.0):
    loss, per_row, cache = forward(params, x, y, n_head)
    return loss, per_row, backward(cache, loss_scale)


# --------------------------------------------------------------------------
# The second block variant ([C] sections 4 and 6): two RMSNorms per block and
# one at the end, RoPE on Q and K, a SwiGLU feed-forward with three matrices,
# no biases, no learned positions, and an output projection of its own
# (untied from the token embedding).  Readings where the page is silent:
#   * RMSNorm(h) = h / sqrt(mean(h^2) + eps) * g, eps 1e-5 as for LayerNorm;
#   * RoPE rotates each pair of channels (2i, 2i+1) of a head by the angle
#     t * theta^(-2i/D) at position t (t from 0 in every row), theta = 10000;
#   * SiLU(u) = u * sigmoid(u); FFN(x) = (SiLU(x W1^T) * (x W3^T)) W2^T.
# --------------------------------------------------------------------------

def rmsnorm(h, g):
    """RMSNorm over the last axis; returns (y, (xhat, rstd))."""
    rstd = 1.0 / np.sqrt((h * h).mean(axis=-1, keepdims=True) + LN_EPS)
    xhat = h * rstd
    return xhat * g, (xhat, rstd)


def rmsnorm_backward(dout, xhat, rstd, g):
    """Chain rule of rmsnorm: returns dx, dg."""
    dxhat = dout * g
    dg = (dout * xhat).reshape(-1, xhat.shape[-1]).sum(axis=0)
    m2 = (dxhat * xhat).mean(axis=-1, keepdims=True)
    return rstd * (dxhat - xhat * m2), dg


def rope_angles(T: int, D: int, theta: float):
    """[T, D/2] angles t * theta^(-2i/D)."""
    inv = theta ** (-np.arange(0, D, 2, dtype=np.float64) / D)
    return np.arange(T, dtype=np.float64)[:, None] * inv[None, :]


def rope(x, theta: float, inverse: bool = False):
    """Rotate channel pairs (2i, 2i+1) of x [B, H, T, D] by their angles (inverse: by minus them)."""
    T, D = x.shape[-2], x.shape[-1]
    a = rope_angles(T, D, theta)
    c, s = np.cos(a), np.sin(a)
    if inverse:
        s = -s
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def silu(u):
    return u / (1.0 + np.exp(-u))


def silu_backward(dout, u):
    sg = 1.0 / (1.0 + np.exp(-u))
    return dout * sg * (1.0 + u * (1.0 - sg))


def _n_layer_cs336(params):
    L = 0
    while f"h{L}.rms1.g" in params:
        L += 1
    return L


def cs336_forward(params, x, y, n_head: int, theta: float = 10000.0, keep=True):
    """Forward pass and mean next-token loss of the variant; as forward()."""
    P = {k: np.asarray(v, dtype=np.float64) for k, v in params.items()}
    L = _n_layer_cs336(P)
    B, T = x.shape
    C = P["wte"].shape[1]
    H = n_head
    D = C // H
    N = B * T
    cache = {"x": x, "y": y, "B": B, "T": T, "H": H, "L": L, "theta": theta}
    h = P["wte"][x].reshape(N, C)
    layers = []
    for l in range(L):
        p = f"h{l}."
        a, r1 = rmsnorm(h, P[p + "rms1.g"])
        qkv = a @ P[p + "attn.w"].T
        q, k, v = (qkv[:, i * C:(i + 1) * C].reshape(B, T, H, D).transpose(0, 2, 1, 3)
                   for i in range(3))
        qr, kr = rope(q, theta), rope(k, theta)
        o, Pm = causal_attention(qr, kr, v)
        o = o.transpose(0, 2, 1, 3).reshape(N, C)
        h_mid = h + o @ P[p + "proj.w"].T
        m, r2 = rmsnorm(h_mid, P[p + "rms2.g"])
        u1 = m @ P[p + "w1"].T
        u3 = m @ P[p + "w3"].T
        s = silu(u1) * u3
        h_out = h_mid + s @ P[p + "w2"].T
        if keep:
            layers.append(dict(a=a, r1=r1, qr=qr, kr=kr, v=v, P=Pm, o=o, m=m, r2=r2, u1=u1, u3=u3, s=s))
        h = h_out
    f, rf = rmsnorm(h, P["rmsf.g"])
    z = f @ P["lm_head"].T
    per_row, lse = cross_entropy_rows(z, y.reshape(-1))
    loss = per_row.mean()
    if keep:
        cache.update(layers=layers, f=f, rf=rf, z=z, lse=lse, P64=P)
    return loss, per_row.reshape(B, T), cache


def cs336_backward(cache, loss_scale: float = 1.0):
    """Gradients of loss_scale * loss for every parameter of the variant."""
    P = cache["P64"]
    L, B, T, H, theta = cache["L"], cache["B"], cache["T"], cache["H"], cache["theta"]
    x, y = cache["x"], cache["y"].reshape(-1)
    N = B * T
    C = P["wte"].shape[1]
    D = C // H
    G = {k: np.zeros_like(v) for k, v in P.items()}
    dz = np.exp(cache["z"] - cache["lse"][:, None])
    dz[np.arange(N), y] -= 1.0
    dz *= loss_scale / N
    G["lm_head"] = dz.T @ cache["f"]
    df = dz @ P["lm_head"]
    dh, G["rmsf.g"] = rmsnorm_backward(df, *cache["rf"], P["rmsf.g"])
    for l in reversed(range(L)):
        p = f"h{l}."
        c = cache["layers"][l]
        # feed-forward: h_out = h_mid + (silu(u1) * u3) W2^T
        G[p + "w2"] = dh.T @ c["s"]
        ds = dh @ P[p + "w2"]
        du1 = silu_backward(ds * c["u3"], c["u1"])
        du3 = ds * silu(c["u1"])
        G[p + "w1"] = du1.T @ c["m"]
        G[p + "w3"] = du3.T @ c["m"]
        dm = du1 @ P[p + "w1"] + du3 @ P[p + "w3"]
        dx2, G[p + "rms2.g"] = rmsnorm_backward(dm, *c["r2"], P[p + "rms2.g"])
        dh = dh + dx2
        # attention: h_mid = h + o Wo^T, with q and k rotated before the scores
        G[p + "proj.w"] = dh.T @ c["o"]
        do = (dh @ P[p + "proj.w"]).reshape(B, T, H, D).transpose(0, 2, 1, 3)
        dqr, dkr, dv = causal_attention_backward(do, c["qr"], c["kr"], c["v"], c["P"])
        dq, dk = rope(dqr, theta, inverse=True), rope(dkr, theta, inverse=True)
        dqkv = np.concatenate([t.transpose(0, 2, 1, 3).reshape(N, C) for t in (dq, dk, dv)], axis=1)
        G[p + "attn.w"] = dqkv.T @ c["a"]
        da = dqkv @ P[p + "attn.w"]
        dx1, G[p + "rms1.g"] = rmsnorm_backward(da, *c["r1"], P[p + "rms1.g"])
        dh = dh + dx1
    np.add.at(G["wte"], x.reshape(-1), dh.reshape(N, C))
    return G


def cs336_loss_and_grads(params, x, y, n_head: int, theta: float = 10000.0, loss_scale: float = 1.0):
    loss, per_row, cache = cs336_forward(params, x, y, n_head, theta)
    return loss, per_row, cs336_backward(cache, loss_scale)


def cs336_param_count(vocab: int, d_model: int, n_layer: int, d_ff: int, tied: bool = False) -> int:
    """Parameters of the variant: embedding (+ untied head), per block 4 D^2 + 3 D d_ff + 2 D, final norm."""
    per_layer = 4 * d_model * d_model + 3 * d_model * d_ff + 2 * d_model
    return vocab * d_model * (1 if tied else 2) + n_layer * per_layer + d_model


# --------------------------------------------------------------------------
# Optimiser ([C] section 2 AdamW and gradient clipping; [R] AdamW, groups)
# --------------------------------------------------------------------------

def decays(name: str, shape) -> bool:
    """Weight decay applies to 2-D tensors (matrices, embeddings) only."""
    return len(shape) == 2


def adamw_update(p, g, m, v, t: int, lr, beta1, beta2, eps, weight_decay, decay=True):
    """One AdamW step at step index t (from 1), returning new (p, m, v).

    m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;
    a = lr sqrt(1-b2^t) / (1-b1^t);  p <- p (1 - lr wd);  p <- p - a m / (sqrt(v) + eps).
    """
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    a = lr * math.sqrt(1.0 - beta2 ** t) / (1.0 - beta1 ** t)
    if decay:
        p = p * (1.0 - lr * weight_decay)
    p = p - a * m / (np.sqrt(v) + eps)
    return p, m, v


def grad_norm(grads) -> float:
    """Global L2 norm over every gradient tensor taken together."""
    return math.sqrt(sum(float((np.asarray(g, dtype=np.float64) ** 2).sum())
                         for g in grads.values()))


def clip_grads(grads, max_norm: float, eps: float = 1e-6):
    """Scale all gradients by min(1, max_norm / (norm + eps)); returns (grads, norm)."""
    n = grad_norm(grads)
    scale = min(1.0, max_norm / (n + eps))
    return {k: np.asarray(g, dtype=np.float64) * scale for k, g in grads.items()}, n


def adamw_step(params, grads, m, v, t, lr, beta1, beta2, eps, weight_decay):
    """AdamW over every tensor; decay only where `decays` says so."""
    P2, M2, V2 = {}, {}, {}
    for k in params:
        P2[k], M2[k], V2[k] = adamw_update(params[k], grads[k], m[k], v[k], t, lr, beta1,
                                           beta2, eps, weight_decay,
                                           decay=decays(k, np.shape(params[k])))
    return P2, M2, V2


def train_step(params, x, y, n_head, lr=6e-4, betas=(0.9, 0.95), eps=1e-8,
               weight_decay=0.1, grad_clip=0.0, m=None, v=None, t=1):
    """zero grads -> forward + loss -> backward -> (clip) -> AdamW, one step."""
    loss, per_row, G = loss_and_grads(params, x, y, n_head)
    norm = None
    if grad_clip and grad_clip > 0:
        G, norm = clip_grads(G, grad_clip)
    if m is None:
        m = {k: np.zeros(np.shape(a)) for k, a in params.items()}
        v = {k: np.zeros(np.shape(a)) for k, a in params.items()}
    P2, M2, V2 = adamw_step(params, G, m, v, t, lr, betas[0], betas[1], eps, weight_decay)
    return dict(loss=loss, per_row=per_row, grads=G, params=P2, m=M2, v=V2, grad_norm=norm)


# --------------------------------------------------------------------------
# Learning-rate schedule ([C] section 2 learning-rate schedule; [R] LR schedule)
# --------------------------------------------------------------------------

def lr_schedule(step: int, max_lr: float, min_lr: float, warmup: int, total: int) -> float:
    """Learning rate at schedule step `step` (counted from 0).

    Linear warm-up from 0 to max_lr over the first `warmup` steps, then a
    half cosine from max_lr down to min_lr, reached at step `total`; from
    there on it stays at min_lr.  Requires 0 <= warmup < total.
    """
    if not (0 <= warmup < total):
        raise ValueError("need 0 <= warmup < total")
    if step < warmup:
        return max_lr * step / warmup
    if step >= total:
        return min_lr
    frac = (step - warmup) / (total - warmup)
    return min_lr + (max_lr - min_lr) * 0.5 * (1.0 + math.cos(math.pi * frac))


# --------------------------------------------------------------------------
# Resource accounting ([C] section 4)
# --------------------------------------------------------------------------

def forward_matmul_flops(seq: int, d_model: int, n_layer: int, vocab: int,
                         matmul_params_per_layer: int, causal: bool = False) -> float:
    """Forward FLOPs of one sequence counting only the matrix products.

    2 FLOPs per multiply-add: 2*S*(weights per layer)*L for the projections,
    2*S*S*D*L each for Q K^T and P V (halved when only the causal half is
    computed), and 2*S*D*V for the vocabulary projection.
    """
    attn = 4.0 * seq * seq * d_model * n_layer
    if causal:
        attn *= (seq + 1) / (2.0 * seq)
    return (2.0 * seq * matmul_params_per_layer * n_layer + attn
            + 2.0 * seq * d_model * vocab)


def training_flops_per_token(n_layer, n_embd, seq, vocab_padded, causal=True) -> float:
    """Model FLOPs per trained token for the GPT-2 block: 3 x forward (backward = 2 x)."""
    per_layer = 12 * n_embd * n_embd  # qkv 3C^2 + out C^2 + fc 4C^2 + proj 4C^2
    fwd = forward_matmul_flops(seq, n_embd, n_layer, vocab_padded, per_layer, causal)
    return 3.0 * fwd / seq


def state_bytes(n_params: int) -> int:
    """fp32 parameters + gradients + AdamW m and v: 16 bytes per parameter."""
    return 16 * int(n_params)
