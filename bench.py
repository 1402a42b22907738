#!/usr/bin/env python3
"""Batch-1 greedy decode benchmark of the 15-layer, 2.3B-shaped decoder at
context 4096 on one MI355X.

Workload: seeded random fp16 weights (N(0, 0.02)), a 3584-token random
prompt, then greedy decode steps up to 4096 positions (each step reads every
weight once plus the visible KV cache: 5 full-attention layers see all
positions, 10 sliding-window layers at most 1024). The prompt is filled by
the batched prompt pass on the matrix cores, timed on its own (`prefill`).
The whole greedy generation (positions 3584 .. 4095) then runs once untimed,
device-fed, and its tokens are compared with the oracle's stored tokens of
the same seeded workload (tests/golden/oracle_ctx4096.npz). The K timed steps
are the last K of that generation, positions 4096-K .. 4095 (context 4096 at
the last), replayed after W warm-up steps as hipGraph replays, device-fed
(the greedy token never leaves the GPU). After every timed region the
sequence's status word is read: a wait between workgroups that gave up, or a
token id that had to be clamped, ends the run with an error, and the timed
region's tokens must equal those of the checked generation.

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
PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16 matrix-core peak, vendor figure
PREFILL_CHUNK = 3584

# HBM bytes per gate/up GEMV launch measured with rocprofv3 FETCH_SIZE and
# WRITE_SIZE (a 512 MiB device copy reads as 0.5x FETCH_SIZE, writes as 1.0x
# WRITE_SIZE; both factors applied), for the GEMV kernel sources whose sha256
# is given: reported only while the sources are unchanged.
GATE_UP_TRAFFIC = {"bytes": 118175985,
                   "sources": ("decode_step_05_amd/csrc/lf_device.h", "decode_step_05_amd/csrc/lf_exchange.h",
                               "decode_step_05_amd/csrc/lf_kernels.h"),
                   "sha256": "82b47b42a3e7bfc227dcd168b563167ab7f5b027f59c82fc2067a8d4abb33779"}


def measured_traffic(entry):
    import hashlib
    h = hashlib.sha256()
    for path in entry["sources"]:
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return entry["bytes"] if h.hexdigest() == entry["sha256"] else None
METRIC = "batch-1 decode tokens/s and achieved HBM GB/s (% of peak) at ctx 4096"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(cfg):
    """Every fp16 weight a step reads once: the projections, the LM head and
    one embedding row (norm gains excluded)."""
    d, h = cfg.d_model, 2
    w = cfg.n_layers * h * (cfg.qkv_rows * d + d * cfg.q_dim + 2 * cfg.ffn * d + d * cfg.ffn)
    if cfg.vocab:
        w += h * cfg.vocab * d + h * d
    return w


def kv_bytes(cfg, p):
    """K and V of the keys each layer sees at position p."""
    per_key = 2 * 2 * cfg.n_kv_heads * cfg.head_dim
    return sum(per_key * ((p + 1) if W == 0 else min(p + 1, W)) for W in cfg.windows)


def step_bytes(cfg, p):
    """Bytes a step at position p must move: every fp16 weight once plus K and
    V of the keys each layer sees."""
    return weight_bytes(cfg) + kv_bytes(cfg, p)


def golden_tokens(name):
    """The oracle's greedy tokens of a generation workload, stored by
    tests/golden/make_golden.py (token s = greedy choice at prompt_len-1+s),
    with the oracle's top-2 gaps; None if the file is missing."""
    import numpy as np
    path = os.path.join(ROOT, "tests", "golden", f"oracle_{name}.npz")
    if not os.path.exists(path):
        return None
    g = np.load(path)
    return g["tokens"], g["gaps"]


def compare_tokens(got, gold, what, near=4e-2):
    """True if the device-fed chain gives the oracle's tokens. A first
    difference where the oracle's top-2 gap is at most `near` (twice the
    parity bound on a logit) is a near-tie: the chains may part there, the
    run goes on, and the tokens before it matched. Any other difference ends
    the run."""
    if gold is None:
        log(f"[bench] {what}: no stored oracle tokens, not checked")
        return False
    toks, gaps = gold
    n = min(len(got), len(toks))
    for s in range(n):
        if int(got[s]) != int(toks[s]):
            if gaps[s] <= near:
                log(f"[bench] {what}: near-tie at step {s} (oracle gap {gaps[s]:.2e}); {s} tokens matched")
                return True
            log(f"[bench] {what}: token {int(got[s])} != oracle {int(toks[s])} at step {s} (gap {gaps[s]:.3f})")
            sys.exit(1)
    log(f"[bench] {what}: all {n} tokens equal the oracle's")
    return True


def check_status(seq, want_len, what):
    """End the run if a wait between workgroups gave up (status bit 1), a token
    id was clamped (bit 0), or the sequence is not where it should be."""
    n, _, flags = seq.status()
    if flags or n != want_len:
        log(f"[bench] {what}: sequence status length {n} (expected {want_len}), flags {flags}: results invalid")
        sys.exit(1)


def check_timed(seq, want_len, ref_tokens, first, what):
    """check_status, and the tokens the timed steps wrote (history entries
    P+first+1 ..) equal those of the checked generation."""
    import numpy as np
    check_status(seq, want_len, what)
    P = want_len - (len(ref_tokens) - 1)
    n = len(ref_tokens) - 1 - first
    got = seq.tokens(P + first + 1, n).cpu().numpy()
    if not np.array_equal(got, ref_tokens[first + 1:]):
        log(f"[bench] {what}: tokens differ from the checked generation")
        sys.exit(1)


def lane_share(torch, Decoder):
    """Per-token latency of one lane's share of the decoder (the per-GPU
    slice of the 8-way lane split) at ctx 4096: hidden-state steps, no
    exchange, synthetic cache."""
    from synth import LANE, make_hidden, make_kv, make_weights
    cfg = LANE
    start, n = cfg.max_ctx - 65, 64
    dec = Decoder(cfg, make_weights(cfg, seed=0, threads=16))
    seq = dec.sequence()
    K_, V_ = make_kv(cfg, start, seed=2)
    seq.load_cache(K_, V_)
    xin = torch.from_numpy(make_hidden(cfg, seed=2)).cuda()
    xout = torch.empty_like(xin)
    for _ in range(4):
        seq.step_hidden(xin, xout)
    seq.set_len(start)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        seq.step_hidden(xin, xout)
    e1.record()
    torch.cuda.synchronize()
    check_status(seq, start + n, "lane share")
    us = e0.elapsed_time(e1) * 1e3 / n
    moved = sum(step_bytes(cfg, p) for p in range(start, start + n)) / n
    return {"workload": "lane: 15 layers, 4 q / 2 kv heads x 128, QKV 1024x4096, O 4096x512, gate/up 1792x4096, "
                        "down 4096x896, hidden in/out, positions 4031..4094",
            "us_per_token": round(us, 2), "bytes_per_token": int(moved),
            "hbm_gbs": round(moved / (us * 1e-6) / 1e9, 1), "roofline_us": round(moved / (PEAK_HBM_GBS * 1e3), 2)}


def layer_rate(torch, Decoder, weights):
    """Per-layer HBM rate of the Laneformer-shaped layer (d 4096, 32 q / 16 kv
    heads x 128, SwiGLU 7168) at batch 1, cache of 2048 synthetic positions,
    full causal and with a 1024-key window. Eight copies of the layer (the
    first eight layers' weights of the full model, 2.2 GB) run as one
    hidden-state chain so that no copy is still in the 256 MB last-level cache
    when it is read again; 32 steps from p = 2048, time per layer = step / 8."""
    from synth import LAYER_FULL, make_hidden, make_kv
    from synth.gen import weight_names
    n_copies, start, n = 8, 2048, 32
    out = {}
    for name, W in (("full", 0), ("swa1024", 1024)):
        cfg = LAYER_FULL.replace(n_layers=n_copies, windows=(W,) * n_copies, name=f"layer_x8_{name}")
        dec = Decoder(cfg, {k: weights[k] for k, _ in weight_names(cfg)})
        seq = dec.sequence()
        K_, V_ = make_kv(cfg, start, seed=2)
        seq.load_cache(K_, V_)
        xin = torch.from_numpy(make_hidden(cfg, seed=2)).cuda()
        xout = torch.empty_like(xin)
        for _ in range(4):
            seq.step_hidden(xin, xout)
        best = None
        for _ in range(3):
            seq.set_len(start)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                seq.step_hidden(xin, xout)
            e1.record()
            torch.cuda.synchronize()
            check_status(seq, start + n, f"single layer {name}")
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        moved = sum(step_bytes(cfg, p) for p in range(start, start + n))
        us_layer = best * 1e3 / (n * n_copies)
        out[name] = {"us_per_layer": round(us_layer, 2), "bytes_per_layer": moved // (n * n_copies),
                     "hbm_gbs": round(moved / (best / 1e3) / 1e9, 1),
                     "roofline_us": round(moved / (n * n_copies) / (PEAK_HBM_GBS * 1e3), 2)}
        del seq, dec
        torch.cuda.empty_cache()
    out["workload"] = ("one Laneformer-shaped layer (d 4096, 32q/16kv x 128, SwiGLU 7168) x 8 weight copies, "
                       "hidden in/out, cache of 2048 synthetic positions, 32 steps from p 2048; best of 3")
    return out


def ctx1024_rate(torch, dec, P=512, K=512):
    """tok/s of the full model on the 512-token workload: a 512-token random
    prompt through the prompt pass, then 512 device-fed greedy steps
    (positions 512..1023, every window still covers the whole context)."""
    from synth import make_prompt
    cfg = dec.cfg
    seq = dec.sequence()
    prompt = torch.from_numpy(make_prompt(cfg, P, seed=1)).cuda()
    seq.prefill_batched(prompt, chunk=PREFILL_CHUNK)
    seq.step()
    torch.cuda.synchronize()
    runs = []
    for _ in range(3):
        seq.set_len(P)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        seq.steps(K)
        e1.record()
        torch.cuda.synchronize()
        check_status(seq, P + K, "ctx1024")
        runs.append(e0.elapsed_time(e1))
    checked = compare_tokens(seq.tokens(P, K + 1).cpu().numpy(), golden_tokens("ctx1024"), "ctx1024 generation")
    ms = float(sorted(runs)[1])
    moved = sum(step_bytes(cfg, p) for p in range(P, P + K))
    del seq
    return {"workload": f"ctx1024: the same model, {P}-token random prompt, greedy decode of positions "
                        f"{P}..{P + K - 1}; median of 3",
            "tok_s": round(K / (ms / 1e3), 1), "ms_per_step": round(ms / K, 4), "checked": checked,
            "hbm_gbs": round(moved / (ms / 1e3) / 1e9, 1),
            "roofline_tok_s_avg": round(PEAK_HBM_GBS * 1e9 / (moved / K), 1)}


def tiny_latency(torch, Decoder):
    """Per-step latency of the tiny 2-layer decoder (d 256, 8 q / 4 kv heads x
    32, SwiGLU 688, vocab 1024, layer 0 window 64): 128-token random prompt,
    then 32 device-fed greedy steps. Its 3.4 MB of weights stay in cache, so
    this is the launch-bound floor of a step, not an HBM measurement."""
    from synth import TINY, make_prompt, make_weights
    cfg = TINY
    P, n = 128, 32
    dec = Decoder(cfg, make_weights(cfg, seed=0))
    seq = dec.sequence()
    seq.prefill_batched(torch.from_numpy(make_prompt(cfg, P, seed=1)).cuda(), chunk=P)
    seq.steps(4)
    runs = []
    for _ in range(5):
        seq.set_len(P)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        seq.steps(n)
        e1.record()
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1) * 1e3 / n)
    del seq, dec
    return {"workload": f"tiny: 2 layers, d 256, 8q/4kv heads x 32, SwiGLU 688, vocab 1024, {P}-token prompt, "
                        f"{n} greedy steps at positions {P}..{P + n - 1}; median of 5",
            "us_per_step": round(float(sorted(runs)[2]), 2), "tok_s": round(1e6 / sorted(runs)[2], 1)}


def sampling_time(torch, C, vocab=32000):
    """Microseconds per lf_sample launch (temperature 0.8) over 1 and 8 rows
    of vocab-wide fp32 logits, seeded N(0, 1.28) like the LM head's output at
    random init; 100 launches back to back between two events."""
    import numpy as np
    out = {}
    for rows in (1, 8):
        rng = np.random.default_rng(4)
        z = torch.from_numpy((rng.standard_normal((rows, vocab)) * 1.28).astype(np.float32)).cuda()
        u = torch.from_numpy(rng.random(rows).astype(np.float32)).cuda()
        tok = torch.empty(rows, dtype=torch.int32, device="cuda")
        C.lf_sample(z, 0.8, u, tok)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(100):
            C.lf_sample(z, 0.8, u, tok)
        e1.record()
        torch.cuda.synchronize()
        out[f"rows{rows}_us"] = round(e0.elapsed_time(e1) * 10, 2)
    out["workload"] = f"temperature sampling of {vocab}-wide fp32 logits, 1 and 8 rows per launch"
    return out


def sampled_rate(torch, C, dec, seq, P, n=64, T=0.8):
    """tok/s of sampled decoding on the ctx4096 model: after one greedy step
    at position P, n steps at P+1 .. P+n, each a copy of the logits, a
    temperature draw (lf_sample, T = 0.8, seeded u) and the decode step fed
    with the drawn token; all on the device, between two events."""
    import numpy as np
    u = torch.from_numpy(np.random.default_rng(5).random(n).astype(np.float32)).cuda()
    z = torch.empty(dec.cfg.vocab, dtype=torch.float32, device="cuda")
    tok = torch.empty(n, dtype=torch.int32, device="cuda")
    seq.set_len(P)
    seq.step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(n):
        C.lf_logits(dec.handle, seq.handle, z)
        C.lf_sample(z, T, u[k:k + 1], tok[k:k + 1])
        seq.step(tok[k:k + 1])
    e1.record()
    torch.cuda.synchronize()
    check_status(seq, P + 1 + n, "sampled decode")
    ms = e0.elapsed_time(e1) / n
    return {"workload": f"sampled decode at T {T} of positions {P + 1}..{P + n}: logits copy, lf_sample, "
                        "decode step fed with the drawn token",
            "ms_per_step": round(ms, 4), "tok_s": round(1e3 / ms, 1)}


def pass_at_n(torch, C, dec, P, prompt_dev, K=32, T=0.8, ns=(1, 2, 4, 8)):
    """Aggregate tok/s of the batched step (lf_decode_step_batch) for N = 1,
    2, 4, 8 continuations of one prompt: the prompt's cache is filled once by
    the batched prompt pass and copied to the other N - 1 sequences; each
    timed region is the last K steps of the context (positions 4096-K ..
    4095), device-fed greedy, then the same with a temperature draw per
    sequence per step (logits of the N sequences, one lf_sample launch over
    the N rows, the batch step fed with the draws). Roofline bytes per step:
    the weights once plus each sequence's visible cache."""
    import numpy as np
    cfg = dec.cfg
    start = cfg.max_ctx - K
    seqs = [dec.sequence() for _ in range(8)]
    seqs[0].prefill_batched(prompt_dev, chunk=PREFILL_CHUNK)
    seqs[0].steps(start - P)  # greedy up to the timed region
    torch.cuda.synchronize()
    for q in seqs[1:]:
        q.buf.copy_(seqs[0].buf)  # state, history and caches; each handle keeps its own buffer
        q.set_len(start)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    zbuf = torch.empty((8, cfg.vocab), dtype=torch.float32, device="cuda")
    tok = torch.empty((K, 8), dtype=torch.int32, device="cuda")
    u = torch.from_numpy(np.random.default_rng(9).random((K, 8)).astype(np.float32)).cuda()
    out = {}
    for n in ns:
        b = seqs[:n]
        res = {}
        for mode in ("greedy", "sampled"):
            for rep in range(2):  # the first run warms up (and records the graph)
                for q in b:
                    q.set_len(start)
                torch.cuda.synchronize()
                e0.record()
                for k in range(K):
                    if mode == "greedy":
                        dec.step_batch(b)
                    else:
                        for i, q in enumerate(b):
                            C.lf_logits(dec.handle, q.handle, zbuf[i])
                        C.lf_sample(zbuf[:n], T, u[k, :n], tok[k, :n])
                        dec.step_batch(b, tok[k, :n])
                e1.record()
                torch.cuda.synchronize()
                for q in b:
                    check_status(q, cfg.max_ctx, f"pass@{n} {mode}")
            ms = e0.elapsed_time(e1) / K
            moved = sum(weight_bytes(cfg) + n * kv_bytes(cfg, p) for p in range(start, cfg.max_ctx)) / K
            res[mode] = {"ms_per_step": round(ms, 4), "tok_s": round(n * 1e3 / ms, 1),
                         "hbm_gbs": round(moved / (ms / 1e3) / 1e9, 1),
                         "roofline_tok_s": round(n * PEAK_HBM_GBS * 1e9 / moved, 1)}
        out[f"n{n}"] = res
    del seqs
    out["workload"] = (f"N continuations of the {P}-token prompt, the last {K} steps of the context (positions "
                       f"{start}..{cfg.max_ctx - 1}), batched step; sampled: T {T}, one lf_sample over the N rows "
                       "per step; roofline bytes = weights once + N visible caches")
    return out


def prefill_flops(cfg, n):
    """Algorithmic flops of the prompt pass over positions 0..n-1: every
    projection as a GEMM of n rows (2 flops per weight per row), attention
    over exactly the visible keys of each query (q.k and the weighted sum of
    v: 4 * head_dim flops per (query head, key)), and the LM head for the last
    position."""
    d, q, f = cfg.d_model, cfg.n_q_heads * cfg.head_dim, cfg.ffn
    per_row = cfg.n_layers * (cfg.qkv_rows * d + d * q + 2 * f * d + d * f)
    pairs = 0
    for w in cfg.windows:
        pairs += sum(p + 1 if w == 0 else min(p + 1, w) for p in range(n))
    return 2 * n * per_row + 4 * cfg.head_dim * cfg.n_q_heads * pairs + 2 * cfg.vocab * d


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
    ap.add_argument("--steps", type=int, default=512, help="timed decode steps, the last of the generation (<= 512)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--kernel-steps", type=int, default=8, help="steps of the per-kernel event timing pass")
    ap.add_argument("--cpu-steps", type=int, default=96,
                    help="oracle steps of the CPU baseline, about 10 s on 16 host threads (0 = skip)")
    ap.add_argument("--mode", choices=["default", "graph", "eager"], default="default",
                    help="step launch mode (default: the library's choice)")
    ap.add_argument("--synthetic-cache", action="store_true",
                    help="load a seeded random KV cache of the prompt's length instead of prefilling it "
                         "(same kernels and bytes per step; for hardware-counter runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="only copy a MB-MiB device buffer three times and exit (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    ap.add_argument("--prefill-chunk", type=int, default=PREFILL_CHUNK, help="positions per chunk of the batched prompt pass")
    ap.add_argument("--pass-at-n-only", type=int, default=0, metavar="N",
                    help="run only the batched-step measurement for N sequences (for a kernel trace) and exit")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time the batched prompt pass (3 runs) and print its JSON object")
    ap.add_argument("--headline-only", action="store_true",
                    help="stop after the timed decode steps (for hardware-counter runs): the line carries no "
                         "per-kernel, side-workload or CPU-baseline figures")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this decode path runs on one GPU; --gpus must be 1 "
              "(the multi-GPU lane exchange is out of scope)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return
    from decode_step_05_amd import Decoder
    from decode_step_05_amd import lfdecode as C
    from synth import WORKLOADS, make_kv, make_prompt, make_weights

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
    modes = {"graph": C.LF_MODE_GRAPH, "eager": C.LF_MODE_EAGER}
    dec = Decoder(cfg, weights, mode=None if args.mode == "default" else modes[args.mode])
    mode_name = {v: k for k, v in modes.items()}[dec.mode]
    log(f"[bench] step launch mode: {mode_name}")
    prompt = make_prompt(cfg, P, seed=wl.prompt_seed)
    prompt_dev = torch.tensor(prompt, dtype=torch.int32, device="cuda")

    # the batched prompt pass on the matrix cores: 3 timed runs from an empty cache
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    pseq = dec.sequence()
    pseq.prefill_batched(prompt_dev, chunk=args.prefill_chunk)
    pf_ms = []
    for _ in range(3):
        pseq.set_len(0)
        torch.cuda.synchronize()
        e0.record()
        pseq.prefill_batched(prompt_dev, chunk=args.prefill_chunk)
        e1.record()
        torch.cuda.synchronize()
        pf_ms.append(e0.elapsed_time(e1))
    del pseq
    pf_med = float(np.median(pf_ms))
    pf_tflops = prefill_flops(cfg, P) / (pf_med / 1e3) / 1e12
    log(f"[bench] batched prompt pass of {P} positions: {', '.join(f'{x:.2f}' for x in pf_ms)} ms "
        f"-> {pf_tflops:.0f} TFLOP/s")
    prefill = {"positions": P, "chunk": args.prefill_chunk, "runs_ms": [round(x, 3) for x in pf_ms],
               "ms": round(pf_med, 3), "tok_s": round(P / (pf_med / 1e3), 1),
               "roofline": {"bound": "mfma", "kernel": "whole batched prompt pass (lf_prefill_batched)",
                            "achieved": round(pf_tflops, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(pf_tflops / PEAK_F16_TFLOPS, 4), "traffic": None,
                            "flops": prefill_flops(cfg, P),
                            "note": "algorithmic flops; the fp32 activations enter the fp16 matrix "
                                    "instructions as hi + lo parts, so the GEMMs issue twice these flops"}}
    if args.prefill_only:
        print(json.dumps({"prefill": prefill}), flush=True)
        return
    if args.pass_at_n_only:
        if not 1 <= args.pass_at_n_only <= C.LF_MAX_BATCH:
            raise SystemExit(f"--pass-at-n-only takes 1 .. {C.LF_MAX_BATCH}")
        batch = pass_at_n(torch, C, dec, P, prompt_dev, ns=(args.pass_at_n_only,))
        print(json.dumps({"pass_at_n": batch}), flush=True)
        return

    seq = dec.sequence()
    torch.cuda.synchronize()
    t = time.perf_counter()
    if args.synthetic_cache:
        K_, V_ = make_kv(cfg, P, seed=wl.data_seed)
        seq.load_cache(K_, V_)
        seq.set_len(P)
        del K_, V_
    else:
        seq.prefill_batched(prompt_dev, chunk=PREFILL_CHUNK)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t
    log(f"[bench] {'synthetic cache' if args.synthetic_cache else 'prefill'} {P} positions in {prefill_s:.2f}s")

    # the whole generation once, untimed, checked against the oracle's tokens
    n_gen = cfg.max_ctx - P
    for i in range(0, n_gen, 64):
        seq.steps(min(64, n_gen - i))
        torch.cuda.synchronize()
    check_status(seq, cfg.max_ctx, "untimed generation")
    gen_tokens = seq.tokens(P, n_gen + 1).cpu().numpy()
    # the stored oracle tokens belong to the prompt's own cache, not to a synthetic one
    gold = None if args.synthetic_cache else golden_tokens("ctx4096")
    checked = compare_tokens(gen_tokens, gold, "ctx4096 generation")

    # warm-up, then the timed region: the last K steps of the generation,
    # positions start .. 4095, replayed from the same cache
    start = cfg.max_ctx - K
    done = 0
    while done < args.warmup:
        seq.set_len(start)
        n = min(K, args.warmup - done)
        seq.steps(n)
        done += n
    torch.cuda.synchronize()
    seq.set_len(start)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    seq.steps(K)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1)
    check_timed(seq, cfg.max_ctx, gen_tokens, start - P, "timed region")
    tok_s = K / (ms / 1e3)
    moved = sum(step_bytes(cfg, p) for p in range(start, cfg.max_ctx))
    gbs = moved / (ms / 1e3) / 1e9
    last_bytes = step_bytes(cfg, cfg.max_ctx - 1)
    log(f"[bench] {K} steps at positions {start}..{cfg.max_ctx - 1}: {ms:.2f} ms (wall {wall * 1e3:.2f} ms) -> "
        f"{tok_s:.1f} tok/s, {gbs:.0f} GB/s; tokens and status checked")

    # four more runs of the same timed region (the reported value is the first)
    runs = [tok_s]
    for _ in range(4):
        seq.set_len(start)
        torch.cuda.synchronize()
        e0.record()
        seq.steps(K)
        e1.record()
        torch.cuda.synchronize()
        check_timed(seq, cfg.max_ctx, gen_tokens, start - P, "repeated timed region")
        runs.append(K / (e0.elapsed_time(e1) / 1e3))
    log("[bench] runs (tok/s): " + ", ".join(f"{r:.1f}" for r in runs))
    if args.headline_only:
        print(json.dumps({"metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K,
                          "warmup": args.warmup, "ms_per_step": round(ms / K, 4), "higher_is_better": True,
                          "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
                          "checked": checked, "runs_tok_s": [round(r, 1) for r in runs],
                          "note": "headline only (hardware-counter run)"}), flush=True)
        return

    # per-step latency: the last 64 device-fed steps, each between two events
    seq.set_len(cfg.max_ctx - 64)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(65)]
    evs[0].record()
    for i in range(64):
        seq.step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    check_status(seq, cfg.max_ctx, "per-step latency")
    lat = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(64))

    # per-kernel timing: eager launches of one step (launch gaps included), and
    # for the roofline the gate/up GEMVs launched back to back in a graph, as
    # the timed graph replays run them (the kernel duration rocprofv3 reports)
    seq.set_len(P)
    torch.cuda.synchronize()
    per_kind = {}
    n_kernels = 0
    for _ in range(args.kernel_steps):
        ks = C.lf_step_kernel_times(dec.handle, seq.handle)
        n_kernels = len(ks)
        for kind, kms in ks:
            per_kind.setdefault(kind, []).append(kms)
    avg = {k: float(np.mean(v)) for k, v in per_kind.items()}
    log("[bench] eager kernel averages (us): " + ", ".join(f"{k} {v * 1e3:.1f}" for k, v in avg.items()))
    seq.set_len(P)
    # all 15 layers' launches in turn: each streams its own 117 MB from HBM
    # (one layer's weights repeated would stay in the 256 MB last-level cache)
    gu_ms = C.lf_kernel_time(dec.handle, seq.handle, "gate_up", -1, reps=1, iters=16)
    gu_gbs = gate_up_bytes(cfg) / (gu_ms / 1e3) / 1e9
    log(f"[bench] gate_up back to back: {gu_ms * 1e3:.2f} us per launch, {gu_gbs:.0f} GB/s")

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
    check_status(seq, cfg.max_ctx, "fixed context 4096")
    fixed_ms = e0.elapsed_time(e1) / n_fixed
    fused = dec.fused
    sampled = sampled_rate(torch, C, dec, seq, P)
    log(f"[bench] sampled decode: {sampled['tok_s']:.1f} tok/s")
    batch = pass_at_n(torch, C, dec, P, prompt_dev)
    log("[bench] pass@N batched step (tok/s greedy / sampled): " +
        ", ".join(f"N={k[1:]} {v['greedy']['tok_s']:.0f} / {v['sampled']['tok_s']:.0f}"
                  for k, v in batch.items() if k.startswith("n")))

    # practical read ceiling: a plain streaming read of 4 GiB
    buf = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    ceiling = C.lf_read_bandwidth(buf, iters=5)
    del buf
    log(f"[bench] streaming-read ceiling {ceiling:.0f} GB/s")

    # one lane's share (4 q / 2 kv heads, 1/8 of the FFN, 15 layers, no LM
    # head, no exchange): per-token latency of 64 hidden-state steps at
    # positions 4031..4094
    lane = lane_share(torch, Decoder)
    log(f"[bench] lane share: {lane['us_per_token']:.1f} us per token")

    # the 512-token workload on the same model, then the single layer
    ctx1024 = ctx1024_rate(torch, dec)
    log(f"[bench] ctx1024: {ctx1024['tok_s']:.1f} tok/s")
    layer = layer_rate(torch, Decoder, weights)
    log(f"[bench] layer: full {layer['full']['us_per_layer']:.1f} us, swa {layer['swa1024']['us_per_layer']:.1f} us")
    tiny = tiny_latency(torch, Decoder)
    log(f"[bench] tiny decoder: {tiny['us_per_step']:.1f} us per step")
    sampling = sampling_time(torch, C)
    log(f"[bench] sampling: {sampling['rows1_us']:.1f} us (1 row), {sampling['rows8_us']:.1f} us (8 rows)")

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
                               f"{P}-token random prompt, greedy decode to 4096 positions; timed: the last {K} "
                               f"steps, positions {start}..{cfg.max_ctx - 1}, batch 1",
                   "prompt": P, "decode_steps": K, "first_position": start, "last_position": cfg.max_ctx - 1,
                   "max_ctx": cfg.max_ctx},
        "checked": checked,
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
        "runs_tok_s": [round(r, 1) for r in runs],
        "median_tok_s": round(float(np.median(runs)), 1),
        "step_latency_ms": {"p50": round(lat[32], 4), "p90": round(lat[57], 4), "max": round(lat[-1], 4),
                            "note": "64 device-fed steps at positions 4032..4095, one event pair per step"},
        "kernels_per_step": n_kernels,
        "qkv_attention_fused": bool(fused),
        "stream_read_ceiling_gbs": round(ceiling, 1),
        "lane_share": lane,
        "ctx1024": ctx1024,
        "single_layer": layer,
        "tiny_latency": tiny,
        "sampling": sampling,
        "sampled_decode": sampled,
        "pass_at_n": batch,
        "prefill_s": round(prefill_s, 3),
        "prefill": prefill,
        "kernel_avg_us_eager": {k: round(v * 1e3, 2) for k, v in avg.items()},
        "roofline": {"bound": "hbm", "kernel": "gate_up GEMV (RMSNorm + SwiGLU fused), 14336x4096 fp16",
                     "achieved": round(gu_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic(GATE_UP_TRAFFIC),
                     "bytes_per_launch": gate_up_bytes(cfg), "avg_launch_us": round(gu_ms * 1e3, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
