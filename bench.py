#!/usr/bin/env python3
"""Batch-1 greedy decode benchmark of the 15-layer, 2.3B-shaped decoder at
context 4096 on one MI355X.

Workload: seeded random fp16 weights (N(0, 0.02)), a 3584-token random
prompt, then greedy decode steps toward 4096 positions (each step reads every
weight once plus the visible KV cache: 5 full-attention layers see all
positions, 10 sliding-window layers at most 1024). Prefill is not timed.
W warm-up steps run first; the sequence is then rewound to the prompt so the
K timed steps replay the same positions 3584 .. 3584+K-1, device-fed (the
greedy token never leaves the GPU), as hipGraph replays.

Prints one JSON line (see the fields below). `--gpus N` with N > 1 is refused:
this path runs on one GPU.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, vendor figure
METRIC = "batch-1 decode tokens/s and achieved HBM GB/s (% of peak) at ctx 4096"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_bytes(cfg, p):
    """Bytes a step at position p must move: every fp16 weight once (the LM
    head and one embedding row included, norm gains excluded) plus K and V of
    the keys each layer sees."""
    d, h = cfg.d_model, 2
    w = cfg.n_layers * h * (cfg.qkv_rows * d + d * cfg.q_dim + 2 * cfg.ffn * d + d * cfg.ffn)
    if cfg.vocab:
        w += h * cfg.vocab * d + h * d
    per_key = 2 * h * cfg.n_kv_heads * cfg.head_dim
    kv = sum(per_key * ((p + 1) if W == 0 else min(p + 1, W)) for W in cfg.windows)
    return w + kv


def gate_up_bytes(cfg):
    """Algorithmic bytes of one gate/up GEMV launch: 2*ffn rows x d_model fp16."""
    return 2 * cfg.ffn * cfg.d_model * 2


def cpu_info():
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def cpu_baseline(cfg, weights, n_steps):
    """The CPU oracle (as it stands, float64) on a bounded sample of the same
    workload: a synthetic cache of 4096 - n_steps positions, then n_steps
    greedy steps ending at position 4095 (context 4096). Weight conversion to
    float64 happens before the clock starts."""
    from oracle import OracleDecoder
    from synth import make_kv
    orc = OracleDecoder(cfg, weights)
    for name in weights:
        orc.w(name)
    start = cfg.max_ctx - n_steps
    K, V = make_kv(cfg, start, seed=2)
    cache = orc.new_cache()
    orc.load_cache(cache, K, V)
    tok = 17
    t0 = time.perf_counter()
    for _ in range(n_steps):
        z = orc.step(cache, token=tok)
        tok = int(z.argmax())
    dt = time.perf_counter() - t0
    return {"value": n_steps / dt, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{n_steps} greedy decode steps at positions {start}..{cfg.max_ctx - 1} of the ctx4096 "
                      f"model (float64 oracle, synthetic cache of {start} positions); host {cpu_info()}, "
                      f"os.cpu_count()={os.cpu_count()}",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512, help="timed decode steps (<= 512)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--kernel-steps", type=int, default=8, help="steps of the per-kernel event timing pass")
    ap.add_argument("--cpu-steps", type=int, default=3, help="oracle steps of the CPU baseline (0 = skip)")
    ap.add_argument("--mode", choices=["default", "persistent", "graph", "eager"], default="default",
                    help="step launch mode (default: the library's choice)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this decode path runs on one GPU; --gpus must be 1 "
              "(the multi-GPU lane exchange is out of scope)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from decode_step_05_amd import Decoder
    from decode_step_05_amd import lfdecode as C
    from synth import WORKLOADS, make_prompt, make_weights

    wl = WORKLOADS["ctx4096"]
    cfg = wl.cfg
    P = wl.prompt_len
    K = args.steps
    if not 1 <= K <= cfg.max_ctx - P:
        print(f"bench.py: --steps must be in [1, {cfg.max_ctx - P}] (decode ends at {cfg.max_ctx} positions)",
              file=sys.stderr)
        sys.exit(2)
    if args.warmup < 0 or args.warmup > cfg.max_ctx - P:
        print("bench.py: --warmup out of range", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    t = time.perf_counter()
    weights = make_weights(cfg, seed=wl.weight_seed, threads=16)
    log(f"[bench] weights generated in {time.perf_counter() - t:.1f}s")
    modes = {"persistent": C.LF_MODE_PERSISTENT, "graph": C.LF_MODE_GRAPH, "eager": C.LF_MODE_EAGER}
    dec = Decoder(cfg, weights, mode=None if args.mode == "default" else modes[args.mode])
    mode_name = {v: k for k, v in modes.items()}[dec.mode]
    log(f"[bench] step launch mode: {mode_name}")
    seq = dec.sequence()
    prompt = make_prompt(cfg, P, seed=wl.prompt_seed)
    torch.cuda.synchronize()
    t = time.perf_counter()
    seq.prefill(prompt)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t
    log(f"[bench] prefill {P} tokens in {prefill_s:.2f}s")

    # warm-up, then rewind so the timed steps replay positions P .. P+K-1
    if args.warmup:
        seq.steps(args.warmup)
    torch.cuda.synchronize()
    seq.set_len(P)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    seq.steps(K)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1)
    tok_s = K / (ms / 1e3)
    moved = sum(step_bytes(cfg, p) for p in range(P, P + K))
    gbs = moved / (ms / 1e3) / 1e9
    last_bytes = step_bytes(cfg, cfg.max_ctx - 1)
    log(f"[bench] {K} steps: {ms:.2f} ms (wall {wall * 1e3:.2f} ms) -> {tok_s:.1f} tok/s, {gbs:.0f} GB/s")

    # per-kernel event timing (kernels launched one by one) for the roofline
    seq.set_len(P)
    torch.cuda.synchronize()
    per_kind = {}
    for _ in range(args.kernel_steps):
        for kind, kms in C.lf_step_kernel_times(dec.handle, seq.handle):
            per_kind.setdefault(kind, []).append(kms)
    avg = {k: float(np.mean(v)) for k, v in per_kind.items()}
    gu_ms = avg["gate_up"]
    gu_gbs = gate_up_bytes(cfg) / (gu_ms / 1e3) / 1e9
    log("[bench] kernel averages (us): " + ", ".join(f"{k} {v * 1e3:.1f}" for k, v in avg.items()))

    # fixed context 4096: repeat the step at p = 4095
    n_fixed = 64
    seq.set_len(cfg.max_ctx - 1)
    seq.step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n_fixed):
        seq.set_len(cfg.max_ctx - 1)
        seq.step()
    e1.record()
    torch.cuda.synchronize()
    fixed_ms = e0.elapsed_time(e1) / n_fixed

    cpu = None
    if args.cpu_steps > 0:
        del seq, dec
        torch.cuda.empty_cache()
        cpu = cpu_baseline(cfg, weights, args.cpu_steps)
        log(f"[bench] cpu oracle {cpu['value']:.3f} tok/s on {cpu['cores']} threads")

    line = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "ctx4096: 15-layer 2.3B-shaped decoder (d 4096, 32q/16kv heads x 128, 8 lanes, "
                               "SwiGLU 7168, vocab 32000, SWA 1024 on 10 layers), random fp16 weights, "
                               f"{P}-token random prompt, greedy decode of positions {P}..{P + K - 1}, batch 1",
                   "prompt": P, "decode_steps": K, "max_ctx": cfg.max_ctx},
        "hbm_gbs": round(gbs, 1),
        "hbm_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
        "bytes_per_step_avg": moved // K,
        "roofline_tok_s_avg": round(PEAK_HBM_GBS * 1e9 / (moved / K), 1),
        "frac_of_roofline": round(tok_s / (PEAK_HBM_GBS * 1e9 / (moved / K)), 4),
        "fixed_ctx4096": {"ms_per_step": round(fixed_ms, 4), "tok_s": round(1e3 / fixed_ms, 1),
                          "bytes_per_step": last_bytes,
                          "hbm_gbs": round(last_bytes / (fixed_ms / 1e3) / 1e9, 1),
                          "roofline_tok_s": round(PEAK_HBM_GBS * 1e9 / last_bytes, 1),
                          "note": "each step preceded by a length reset; includes that launch"},
        "prefill_s": round(prefill_s, 2),
        "kernel_avg_us": {k: round(v * 1e3, 2) for k, v in avg.items()},
        "roofline": {"bound": "hbm", "kernel": "gate_up GEMV (RMSNorm + SwiGLU fused), 14336x4096 fp16",
                     "achieved": round(gu_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "bytes_per_launch": gate_up_bytes(cfg), "avg_launch_us": round(gu_ms * 1e3, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
