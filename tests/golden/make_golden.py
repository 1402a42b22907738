"""Write the stored oracle results of the full-model generation workloads.

Runs only the CPU oracle (oracle/) on the seeded inputs of synth/ and stores,
per compared position, what the GPU test needs to check its logits and greedy
tokens without re-running a float64 model of 2.3B parameters:
  * the oracle's greedy token (decided on float32-rounded logits),
  * the gap between its two largest logits (for the near-tie rule),
  * the logits at the 8 largest indices and at 128 fixed sampled indices,
  * the full logits vector at every 16th position (0, 16, ..., 512), so that
    whole 32000-wide vectors are compared along each generation.

Workloads: ctx1024 (512-token prompt, 512 greedy steps) and ctx4096
(3584-token prompt, 512 greedy steps) of the 15-layer decoder.

    python tests/golden/make_golden.py [ctx1024|ctx4096 ...]
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import OracleDecoder, greedy  # noqa: E402
from synth import WORKLOADS, make_prompt, make_weights  # noqa: E402

N_TOP = 8
N_SAMPLE = 128
FULL_EVERY = 16


def sample_indices(vocab, seed=7):
    return np.sort(np.random.default_rng(seed).choice(vocab, size=N_SAMPLE, replace=False)).astype(np.int32)


def run(name):
    wl = WORKLOADS[name]
    cfg = wl.cfg
    t0 = time.time()
    w = make_weights(cfg, seed=wl.weight_seed)
    prompt = make_prompt(cfg, wl.prompt_len, seed=wl.prompt_seed)
    dec = OracleDecoder(cfg, w)
    cache = dec.new_cache()
    z = dec.forward_sequence(tokens=prompt, cache=cache)[-1]
    print(f"[{name}] prefill {wl.prompt_len} in {time.time() - t0:.0f}s", flush=True)
    idx = sample_indices(cfg.vocab)
    n = wl.steps + 1
    toks = np.zeros(n, np.int32)
    gaps = np.zeros(n, np.float64)
    top_i = np.zeros((n, N_TOP), np.int32)
    top_v = np.zeros((n, N_TOP), np.float64)
    samp = np.zeros((n, N_SAMPLE), np.float64)
    full_at = np.arange(0, n, FULL_EVERY, dtype=np.int32)
    full = np.zeros((len(full_at), cfg.vocab), np.float32)
    for s in range(n):
        if s:
            z = dec.step(cache, token=int(toks[s - 1]))
        toks[s] = greedy(z)
        order = np.argsort(-z, kind="stable")
        top_i[s] = order[:N_TOP]
        top_v[s] = z[order[:N_TOP]]
        gaps[s] = z[order[0]] - z[order[1]]
        samp[s] = z[idx]
        if s in full_at:
            full[list(full_at).index(s)] = z.astype(np.float32)
        if s % 64 == 0:
            print(f"[{name}] step {s}/{n - 1} {time.time() - t0:.0f}s", flush=True)
    out = os.path.join(HERE, f"oracle_{name}.npz")
    np.savez_compressed(out, prompt_len=wl.prompt_len, steps=wl.steps, tokens=toks, gaps=gaps, top_i=top_i,
                        top_v=top_v, sample_idx=idx, sample_v=samp, full_at=full_at, full=full)
    print(f"[{name}] wrote {out} ({os.path.getsize(out) / 1e3:.0f} KB) in {time.time() - t0:.0f}s", flush=True)


if __name__ == "__main__":
    for name in (sys.argv[1:] or ["ctx1024", "ctx4096"]):
        run(name)
