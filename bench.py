"""Training throughput of the GPT-2 training step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--repeats R] [--config NAME]
                [--no-cpu-baseline] [--breakdown] [--roofline-kernel CLASS]
                [--copy-calibration BYTES]

--config gpt2-124m (default, the headline workload: B=16, T=1024), gpt2-350m
(B=8), gpt2-1.5b (B=4 x 4 accumulation micro-steps) or lmhead (the isolated
LM head + cross-entropy, N=65536, V=50257, C=768).

One step = per micro-step make_batch (B*T+1 tokens of a seeded synthetic
Zipf(1.1) stream with end-of-text separators) -> forward + head/CE ->
backward, then AdamW, all through libgpt.so.  W warm-up steps, then R loops
of K timed steps, each between torch.cuda.synchronize() calls; the line
reports the median loop.  It carries tokens/s, MFU, the roofline of the
dominant kernel, the rates of a few more kernel classes (timed in extra steps
after the loops) and the fp64 CPU oracle timed on the GPU's own step-1 weights
and window.  The dominant kernel is the fused LM head + cross-entropy, taken as
one unit: its two passes are the two largest kernels of the step when each runs
alone (GPT-2 124M: pass 2, the tied dW, 2.51 ms in its two launches; pass 1,
loss, log-sum-exp and dF, 2.27 ms; then attention backward, 1.40 ms, of 20.6 ms
of serialised kernel time).  Pass 1 is timed with HIP events in the last step
of the last loop, pass 2 (which runs beside the backward on a stream of its
own, sharing the CUs) in a step of its own; achieved = the head's algorithmic
FLOPs, 6*N*V_pad*C per step (its logit recompute not counted), over the sum of
both passes' times.  Each pass's own rate is listed under kernel_rates.

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
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s
PEAK_F32 = 157.3e12     # MI355X fp32 (MFMA and vector), FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E, B/s
# kernel classes the library can time (each GEMM class times its main kernel only)
PROFILE_CLASSES = ["gemm_qkv_fwd", "gemm_proj_fwd", "gemm_fc_fwd", "gemm_mlpproj_fwd", "gemm_dgrad_mlp",
                   "gemm_dgrad_attn", "gemm_wgrad_mlp", "gemm_wgrad_attn", "attn_fwd", "attn_bwd",
                   "layernorm_fwd", "layernorm_bwd", "head_fwd", "head_dz", "head_dw", "head_dw_dz",
                   "bias_colsum", "param_reduce", "embed_bwd", "adamw"]
# further classes reported beside the dominant one (one extra step each)
MORE_CLASSES = ["head_fwd", "head_dw", "attn_bwd", "attn_fwd", "gemm_fc_fwd", "layernorm_bwd", "adamw"]
METRIC = "train tokens/sec + MFU, GPT-2 124M B=16 T=1024 bf16, 1×MI355X"

WORKLOADS = {
    "gpt2-124m": "GPT-2 124M training step: L=12, C=768, H=12, V=50257 padded to 50304, T=1024, B=16",
    "gpt2-350m": "GPT-2 350M training step: L=24, C=1024, H=16, V=50257 padded to 50304, T=1024, B=8",
    "gpt2-1.5b": ("GPT-2 1.5B training step: L=48, C=1600, H=25, V=50257 padded to 50304, T=1024, "
                  "B=4 x 4 gradient-accumulation micro-steps"),
    "cs336-tinystories": ("RMSNorm/RoPE/SwiGLU block, untied head (CS336 TinyStories model) training step: "
                          "L=4, C=512, H=16, d_ff=1344, V=10000, T=256, B=32, fp32"),
    "cs336-tinystories-bf16": ("RMSNorm/RoPE/SwiGLU block, untied head, TinyStories sizes with 8 heads of 64: "
                               "L=4, C=512, H=8, d_ff=1344, V=10000, T=256, B=32, bf16"),
}
WORKLOAD_TAIL = (", bf16 GEMM/attention operands with fp32 master weights and AdamW state; Zipf(1.1) tokens "
                 "with end-of-text every Geometric(1/600), random init")

# sources whose change invalidates stored counter readings of a kernel class
KERNEL_SOURCES = {
    "gemm": ["csrc/gemm.hip", "csrc/common.h", "csrc/kernels.h"],
    "attn": ["csrc/attention_bf16.hip", "csrc/attention.hip", "csrc/common.h", "csrc/kernels.h"],
    "head": ["csrc/head.hip", "csrc/mfma_lds.h", "csrc/common.h", "csrc/kernels.h"],
}


def sources_sha(kernel_class):
    fam = ("attn" if kernel_class.startswith("attn") else
           "head" if kernel_class in ("head_fwd", "head_dw", "lmhead") else "gemm")
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[fam]:
        with open(os.path.join(ROOT, "decoder_only_transformer_train_amd", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(kernel_class, workload):
    """HBM bytes per launch measured by counters, or None when absent or stale."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            recs = json.load(f)
    except (OSError, ValueError):
        return None
    for rec in recs if isinstance(recs, list) else [recs]:
        if (rec.get("kernel") == kernel_class and rec.get("workload", "gpt2-124m") == workload
                and rec.get("sources_sha256") == sources_sha(kernel_class)):
            return rec.get("bytes_per_launch")
    return None


def host_info():
    """CPU model, usable cores, BLAS library and its thread count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer')})"
                threads = int(i.get("num_threads", 1))
    except Exception:
        pass
    cores = len(os.sched_getaffinity(0))
    return model, cores, blas, threads if threads else cores


def cpu_baseline(cfg, params, stream, repeats):
    """fp64 oracle: forward+backward of the first sequence of the GPU's first window, on the
    GPU's own initial weights, plus AdamW over all parameters; median of `repeats` runs."""
    import numpy as np
    import oracle
    model, cores, blas, threads = host_info()
    x, y = oracle.make_batch(stream, 0, cfg.batch, cfg.seq)
    rows, adams = [], []
    for _ in range(repeats):
        t0 = time.perf_counter()
        _, _, G = oracle.loss_and_grads(params, x[:1], y[:1], cfg.n_head)
        rows.append(time.perf_counter() - t0)
        m = {k: np.zeros(a.shape) for k, a in params.items()}
        v = {k: np.zeros(a.shape) for k, a in params.items()}
        t0 = time.perf_counter()
        oracle.adamw_step(params, G, m, v, 1, 6e-4, 0.9, 0.95, 1e-8, 0.1)
        adams.append(time.perf_counter() - t0)
        del G, m, v
    t_row, t_adam = statistics.median(rows), statistics.median(adams)
    n_rows = cfg.batch * cfg.accum
    step_s = n_rows * t_row + t_adam
    return {"value": round(n_rows * cfg.seq / step_s, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"fp64 NumPy oracle on the GPU's own initial weights and first window: forward+backward "
                       f"of sequence 0 ({cfg.seq} tokens) in {t_row:.2f} s and AdamW over all parameters in "
                       f"{t_adam:.2f} s (medians of {repeats}), scaled to one step of {n_rows} sequences"),
            "cpu_model": model, "host_cpus": cores, "blas": blas, "blas_threads": threads}


def rate(r, peak_mfma=PEAK_BF16):
    """Algorithmic rate of a profiled class against its roofline (contractions
    against the MFMA peak of the context's dtype)."""
    if r["launches"] == 0 or r["ms"] <= 0:
        return None
    avg_ms = r["ms"] / r["launches"]
    if r["flops"] > 0:
        a = r["flops"] / r["launches"] / (avg_ms / 1e3)
        return {"bound": "mfma", "achieved": round(a / 1e12, 2), "peak": peak_mfma / 1e12, "unit": "TFLOP/s",
                "frac": round(a / peak_mfma, 4), "avg_launch_ms": round(avg_ms, 4), "launches": r["launches"]}
    a = r["bytes"] / r["launches"] / (avg_ms / 1e3)
    return {"bound": "hbm", "achieved": round(a / 1e9, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": round(a / PEAK_HBM, 4), "avg_launch_ms": round(avg_ms, 4), "launches": r["launches"]}


def head_operator(fwd, dw, dw_dz):
    """The LM head + cross-entropy of one step as one unit: pass 1 (loss, lse
    and dF: 4*N*V*C) and pass 2 (the tied dW: 2*N*V*C) summed over all their
    launches.  The GEMM form of pass 2 adds the product that recomputes each
    vocabulary block's logits (head_dw_dz): its time counts, its FLOPs do not,
    like the recompute inside the fused pass-2 kernel."""
    return {"ms": fwd["ms"] + dw["ms"] + dw_dz["ms"], "launches": 1,
            "flops": fwd["flops"] + dw["flops"], "bytes": 0.0,
            "parts": fwd["launches"] + dw["launches"] + dw_dz["launches"]}


def copy_calibration(nbytes):
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def bench_model(args, name):
    import torch
    from decoder_only_transformer_train_amd import accounting, binding, configs, synthetic

    cfg = configs.PRESETS[name]
    B, T, A = cfg.batch, cfg.seq, cfg.accum
    W, K, R = args.warmup, args.steps, args.repeats
    n_tok = (W + K * R + 2 + len(MORE_CLASSES)) * A * B * T + 1
    stream = synthetic.zipf_eot_stream(n_tok, cfg.vocab, seed=0, eot=min(synthetic.EOT_ID, cfg.vocab - 1))
    g = binding.GPT(cfg, seed=0, device="cuda:0")
    # the step-1 weights for the CPU oracle baseline (GPT-2 blocks only)
    init_params = None if args.no_cpu_baseline or cfg.block != binding.GPT_BLOCK_GPT2 else g.get_all(binding.PARAM)
    adam = configs.ADAMW
    peak_mfma = PEAK_F32 if cfg.dtype == binding.GPT_F32 else PEAK_BF16

    def step(pos):
        for _ in range(A):
            g.make_batch(stream, pos)
            g.forward_loss(1.0 / A, sync=False)
            g.backward()
            pos = binding.next_start(pos, len(stream), B, T)
        g.adamw_step(**adam, grad_clip=0.0, sync=False)
        return pos

    pos = 0
    for _ in range(W):
        pos = step(pos)
    torch.cuda.synchronize()
    g.read_losses()

    breakdown = rates = None
    if args.breakdown:
        # per kernel class: time per step and the class's algorithmic rate against its peak
        # (classes on the backward's second stream share the GPU with the first stream)
        breakdown, rates = {}, {}
        for cls in PROFILE_CLASSES:
            g.profile_begin(cls)
            step(0)
            r = g.profile_end()
            breakdown[cls] = round(r["ms"], 3)
            rates[cls] = rate(r, peak_mfma)
        g.read_losses()

    loops = []
    prof = None
    for rep in range(R):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            # the roofline kernel is timed in the last step of the last loop: its events put
            # barrier packets around each launch (a few us of idle GPU each), which the other
            # steps are spared
            if rep == R - 1 and i == K - 1:
                g.profile_begin("head_fwd" if args.roofline_kernel == "lm_head" else args.roofline_kernel)
            pos = step(pos)
        torch.cuda.synchronize()
        loops.append(time.perf_counter() - t0)
        if rep == R - 1:
            prof = g.profile_end()
    losses = g.read_losses()
    more, raw = {}, {}
    for cls in MORE_CLASSES + (["head_dw_dz"] if args.roofline_kernel == "lm_head" else []):
        if cls == args.roofline_kernel or (cls == "head_fwd" and args.roofline_kernel == "lm_head"):
            continue
        g.profile_begin(cls)
        pos = step(pos)
        raw[cls] = g.profile_end()
        if cls in MORE_CLASSES:
            more[cls] = rate(raw[cls], peak_mfma)
    g.read_losses()
    if args.roofline_kernel == "lm_head":
        more = {"head_fwd": rate(prof, peak_mfma), **more}
        prof = head_operator(prof, raw["head_dw"], raw["head_dw_dz"])

    dt = statistics.median(loops)
    tokens = K * A * B * T
    tps = tokens / dt
    fp32 = cfg.dtype == binding.GPT_F32
    fpt = accounting.training_flops_per_token(cfg.n_layer, cfg.n_embd, T, cfg.padded_vocab,
                                              cfg.d_ff if cfg.block == binding.GPT_BLOCK_RMS_ROPE_SWIGLU else 0)
    mfu = tps * fpt / peak_mfma
    roof = rate(prof, peak_mfma)
    if args.roofline_kernel == "lm_head":
        parts = [stored_traffic(k, name) for k in ("head_fwd", "head_dw")]
        roof["traffic"] = (sum(parts) if None not in parts and not raw["head_dw_dz"]["launches"]
                           else None)
        roof["kernel"] = ("lm_head: LM head + cross-entropy, pass 1 (loss, lse, dF) and pass 2 "
                          "(head weight gradient dW) of one step as one unit; recomputed logits not counted")
        roof["timed_spans"] = prof["parts"]
    else:
        roof["traffic"] = stored_traffic(args.roofline_kernel, name)
        roof["kernel"] = args.roofline_kernel
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
    out = {
        "metric": METRIC if name == "gpt2-124m" else f"train tokens/sec + MFU, {WORKLOADS[name].split(':')[0]}, 1×MI355X",
        "value": round(tps, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(dt / K * 1e3, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if fp32 else "bf16", "data": "synthetic",
        "config": {"workload": WORKLOADS[name] + (WORKLOAD_TAIL if name.startswith("gpt2") else
                                                  ", Zipf(1.1) tokens with end-of-text separators, random init"),
                   "global_batch": B * A, "seq_len": T,
                   "tokens_per_step": A * B * T, "accumulation": A},
        "mfu": round(mfu, 4), "model_tflop_per_step": round(fpt * A * B * T / 1e12, 3),
        "repeats_ms_per_step": [round(x / K * 1e3, 3) for x in loops],
        "final_loss": float(losses[-1]) if len(losses) else None,
        "roofline": roof,
        "kernel_rates": more,
    }
    if breakdown is not None:
        out["breakdown_ms"] = breakdown
        out["breakdown_rate"] = rates
    g.close()
    del g
    torch.cuda.empty_cache()
    if init_params is not None:
        out["cpu_baseline"] = cpu_baseline(cfg, init_params, stream, 3 if name == "gpt2-124m" else 1)
    return out


def bench_lmhead(args):
    """The isolated LM head + cross-entropy: loss, dX and dW of N=65536 rows, V=50257, C=768."""
    import numpy as np
    import torch
    from decoder_only_transformer_train_amd import accounting, binding, synthetic

    N, V, C = 65536, 50257, 768
    X, Wt, y = synthetic.lmhead_inputs(N, V, C, seed=1)
    Xd = torch.from_numpy(synthetic.bf16_bits(X).view(np.int16)).cuda()
    Wd = torch.from_numpy(synthetic.bf16_bits(Wt).view(np.int16)).cuda()
    yd = torch.from_numpy(np.ascontiguousarray(y, np.int32)).cuda()
    run = binding.LMHead(N, V, C, binding.GPT_BF16)
    for _ in range(args.warmup):
        run(Xd, Wd, yd)
    loops = []
    s = torch.cuda.current_stream()
    for _ in range(args.repeats):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            run(Xd, Wd, yd)
        torch.cuda.synchronize()
        loops.append(time.perf_counter() - t0)
    # one more call between HIP events on the stream the call runs on
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    run(Xd, Wd, yd)
    e1.record(s)
    torch.cuda.synchronize()
    call_ms = e0.elapsed_time(e1)
    dt = statistics.median(loops) / args.steps
    flops = accounting.lmhead_flops(N, V, C)
    roof = {"bound": "mfma", "achieved": round(flops / (call_ms / 1e3) / 1e12, 2), "peak": PEAK_BF16 / 1e12,
            "unit": "TFLOP/s", "frac": round(flops / (call_ms / 1e3) / PEAK_BF16, 4),
            "traffic": stored_traffic("lmhead", "lmhead"), "kernel": "lmhead (whole call)",
            "avg_launch_ms": round(call_ms, 4), "launches": 1}
    out = {
        "metric": "LM head + cross-entropy tokens/sec (loss, dX, dW), N=65536 V=50257 C=768 bf16, 1×MI355X",
        "value": round(N / dt, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": ("LM head + cross-entropy in isolation: X [65536, 768] ~ N(0,1), W [50257, 768] "
                                "~ N(0, 0.02), bf16, Zipf(1.1) targets, seed 1; loss, dX and dW")},
        "model_tflop_per_step": round(flops / 1e12, 3), "tflops": round(flops / dt / 1e12, 2),
        "repeats_ms_per_step": [round(x / args.steps * 1e3, 3) for x in loops],
        "loss": float(run.loss.item()),
        "roofline": roof,
    }
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--repeats", type=int, default=3)
    ap.add_argument("--config", default="gpt2-124m", choices=list(WORKLOADS) + ["lmhead"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true")
    # the dominant kernel class of the step (largest share of the step's kernel time)
    # (lm_head: the fused LM head + cross-entropy as one operator, all its launches)
    ap.add_argument("--roofline-kernel", default="lm_head", choices=["lm_head"] + PROFILE_CLASSES)
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="after the timed steps, copy this many bytes device-to-device once")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.repeats < 1 or args.warmup < 0:
        print("need --steps >= 1, --repeats >= 1, --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    out = bench_lmhead(args) if args.config == "lmhead" else bench_model(args, args.config)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
