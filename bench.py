"""Training throughput of the GPT-2 124M step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--breakdown]
                [--roofline-kernel CLASS] [--copy-calibration BYTES]

One step = make_batch (B*T+1 tokens of a seeded synthetic Zipf(1.1) stream
with end-of-text separators) -> forward + fused head/CE -> backward -> AdamW,
all through libgpt.so.  Prints one JSON line with tokens/s, MFU, the
roofline of one kernel (timed with HIP events on the library's stream inside
the timed region) and the fp64 CPU oracle timed on a bounded sample.

The roofline's "traffic" (HBM bytes per launch of that kernel) comes from
profiles/traffic.json, written from two rocprofv3 --pmc runs (FETCH_SIZE,
WRITE_SIZE) of this script with --copy-calibration, which appends one plain
device copy of known size so the counters can be scaled to bytes.  It is
reported only while the kernel sources hash to what they were when the
counters were taken; otherwise it is null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E, B/s
# kernel classes the library can time (each GEMM class times its main kernel only)
PROFILE_CLASSES = ["gemm_qkv_fwd", "gemm_proj_fwd", "gemm_fc_fwd", "gemm_mlpproj_fwd", "gemm_dgrad_mlp",
                   "gemm_dgrad_attn", "gemm_wgrad_mlp", "gemm_wgrad_attn", "attn_fwd", "attn_bwd",
                   "layernorm_fwd", "layernorm_bwd", "head_logits", "head_ce", "head_dx", "head_dw",
                   "bias_colsum", "param_reduce", "embed_bwd", "adamw"]
METRIC = "train tokens/sec + MFU, GPT-2 124M B=16 T=1024 bf16, 1×MI355X"


# sources whose change invalidates stored counter readings of a kernel class
KERNEL_SOURCES = {
    "gemm": ["csrc/gemm.hip", "csrc/common.h", "csrc/kernels.h"],
    "attn": ["csrc/attention_bf16.hip", "csrc/attention.hip", "csrc/common.h", "csrc/kernels.h"],
}


def sources_sha(kernel_class):
    fam = "attn" if kernel_class.startswith("attn") else "gemm"
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[fam]:
        with open(os.path.join(ROOT, "decoder_only_transformer_train_amd", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(kernel_class):
    """HBM bytes per launch measured by counters, or None when absent or stale."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel") != kernel_class or rec.get("sources_sha256") != sources_sha(kernel_class):
        return None
    return rec.get("bytes_per_launch")


def model_flops_per_token(L, C, T, Vp):
    """3 x forward matmul FLOPs per token; attention counts the causal pairs only."""
    fwd = 2 * 12 * C * C * L + 2 * 2 * C * L * (T + 1) / 2 + 2 * C * Vp
    return 3.0 * fwd


def cpu_baseline(cfg, seconds_cap=30.0):
    """fp64 oracle on one 1024-token sequence (fwd + bwd) plus AdamW over all parameters."""
    import numpy as np
    import oracle
    from decoder_only_transformer_train_amd import synthetic
    try:
        from threadpoolctl import threadpool_info
        threads = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        threads = len(os.sched_getaffinity(0))
    p = synthetic.init_params(cfg.n_layer, cfg.n_embd, cfg.padded_vocab, cfg.max_seq, seed=0)
    toks = synthetic.zipf_eot_stream(cfg.seq + 1, cfg.vocab, seed=0)
    x, y = oracle.make_batch(toks, 0, 1, cfg.seq)
    t0 = time.perf_counter()
    loss, _, G = oracle.loss_and_grads(p, x, y, cfg.n_head)
    t_row = time.perf_counter() - t0
    m = {k: np.zeros(a.shape) for k, a in p.items()}
    v = {k: np.zeros(a.shape) for k, a in p.items()}
    t0 = time.perf_counter()
    oracle.adamw_step(p, G, m, v, 1, 6e-4, 0.9, 0.95, 1e-8, 0.1)
    t_adam = time.perf_counter() - t0
    step_s = cfg.batch * t_row + t_adam
    return {"value": round(cfg.batch * cfg.seq / step_s, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"fp64 NumPy oracle: forward+backward of 1 of the {cfg.batch} sequences "
                       f"({cfg.seq} tokens) in {t_row:.2f} s and AdamW over all parameters in "
                       f"{t_adam:.2f} s, scaled to one {cfg.batch}x{cfg.seq} step"),
            "host_cpus": len(os.sched_getaffinity(0))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true")
    # the largest kernel class that runs alone: the backward's two streams and the head's dW share the GPU
    ap.add_argument("--roofline-kernel", default="gemm_fc_fwd", choices=PROFILE_CLASSES)
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="after the timed steps, copy this many bytes device-to-device once")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from decoder_only_transformer_train_amd import binding, configs, synthetic

    cfg = configs.GPT2_124M
    B, T = cfg.batch, cfg.seq
    W, K = args.warmup, args.steps
    n_tok = (W + K) * B * T + 1
    stream = synthetic.zipf_eot_stream(n_tok, cfg.vocab, seed=0)
    g = binding.GPT(cfg, seed=0, device="cuda:0")
    s = g.stream
    adam = configs.ADAMW

    def step(pos):
        g.make_batch(stream, pos)
        g.forward_loss(1.0, sync=False)
        g.backward()
        g.adamw_step(**adam, grad_clip=0.0, sync=False)
        return binding.next_start(pos, len(stream), B, T)

    pos = 0
    for _ in range(W):
        pos = step(pos)
    torch.cuda.synchronize()
    g.read_losses()

    breakdown = None
    if args.breakdown:
        # per kernel class: time per step and the class's algorithmic rate against its peak
        # (classes on the backward's second stream share the GPU with the first stream)
        breakdown, rates = {}, {}
        for cls in PROFILE_CLASSES:
            g.profile_begin(cls)
            step(0)
            r = g.profile_end()
            breakdown[cls] = round(r["ms"], 3)
            if r["ms"] > 0 and r["flops"] > 0:
                a = r["flops"] / (r["ms"] / 1e3)
                rates[cls] = {"TFLOP/s": round(a / 1e12, 1), "frac": round(a / PEAK_BF16, 3)}
            elif r["ms"] > 0 and r["bytes"] > 0:
                a = r["bytes"] / (r["ms"] / 1e3)
                rates[cls] = {"GB/s": round(a / 1e9, 1), "frac": round(a / PEAK_HBM, 3)}
        g.read_losses()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        # the roofline kernel is timed in the last timed step: its events put
        # barrier packets around each launch (a few us of idle GPU each), which
        # the other steps are spared
        if i == K - 1:
            g.profile_begin(args.roofline_kernel)
        pos = step(pos)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    prof = g.profile_end()
    losses = g.read_losses()

    tokens = K * B * T
    tps = tokens / dt
    fpt = model_flops_per_token(cfg.n_layer, cfg.n_embd, T, cfg.padded_vocab)
    mfu = tps * fpt / PEAK_BF16
    avg_ms = prof["ms"] / max(1, prof["launches"])
    if prof["flops"] > 0:
        achieved = prof["flops"] / max(1, prof["launches"]) / (avg_ms / 1e3)
        roof = {"bound": "mfma", "achieved": round(achieved / 1e12, 2), "peak": PEAK_BF16 / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16, 4), "traffic": None}
    else:
        achieved = prof["bytes"] / max(1, prof["launches"]) / (avg_ms / 1e3)
        roof = {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM, 4), "traffic": None}
    roof["traffic"] = stored_traffic(args.roofline_kernel)
    roof.update({"kernel": args.roofline_kernel, "avg_launch_ms": round(avg_ms, 4),
                 "launches": prof["launches"]})
    if args.copy_calibration > 0:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    out = {
        "metric": METRIC, "value": round(tps, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(dt / K * 1e3, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": ("GPT-2 124M training step: L=12, C=768, H=12, V=50257 padded to 50304, "
                                "T=1024, B=16, bf16 GEMM/attention operands with fp32 master weights "
                                "and AdamW state; Zipf(1.1) tokens with end-of-text every "
                                "Geometric(1/600), random init"),
                   "global_batch": B, "seq_len": T, "tokens_per_step": B * T},
        "mfu": round(mfu, 4), "model_tflop_per_step": round(fpt * B * T / 1e12, 3),
        "final_loss": float(losses[-1]) if len(losses) else None,
        "roofline": roof,
    }
    if breakdown is not None:
        out["breakdown_ms"] = breakdown
        out["breakdown_rate"] = rates
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
