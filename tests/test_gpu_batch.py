"""The batched decode step (lf_decode_step_batch: n sequences of one model
step together, each weight read once for all) against the oracle, through the
C ABI.

Stochastic decoding scored as pass@N (asector.ru summary, "Performance and
infrastructure") runs N continuations of one prompt side by side. Each
sequence of a batch must get exactly what the single-sequence step gives it:
its own logits (within the parity bar of parity.py; the projections run on
the matrix cores with hi/lo fp16 activations, so not bitwise) and greedy
tokens. The cases cover 1, 3, 5 and 8 sequences of different lengths, the
ragged 3-lane head_dim-64 shape (d_model 264: K not a multiple of the 32-wide
k-step), 4 query heads per kv head, teacher-forced and free-running greedy
steps, sampled steps through lf_sample (pass@N of one prompt), graph replay
against eager launches, and the full 2.3B-shaped model with 8 sequences at
positions up to 4095.
"""
import numpy as np
import pytest

from oracle import OracleDecoder, greedy, interval_of, sample_token
from synth import FULL, TINY, DecoderConfig, make_kv, make_prompt, make_weights

from parity import assert_close, check_token

pytestmark = pytest.mark.gpu

RAGGED = DecoderConfig("ragged", n_layers=3, d_model=264, n_q_heads=6, n_kv_heads=3, head_dim=64, ffn=360,
                       vocab=1000, n_lanes=3, max_ctx=96, windows=(7, 0, 13))
WIDE_GROUP = DecoderConfig("group4", n_layers=2, d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1024,
                           vocab=777, n_lanes=1, max_ctx=300, windows=(100, 0))


def say(*a):
    print(*a, flush=True)


def _prompts(cfg, n, base_len):
    # sequence s: its own prompt of base_len + 3 s tokens
    return [make_prompt(cfg, base_len + 3 * s, seed=10 + s) for s in range(n)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("cfg,n,plen,steps,graph", [
    (TINY, 1, 40, 6, True),
    (TINY, 3, 40, 6, True),
    (TINY, 8, 100, 10, True),
    (TINY, 8, 100, 10, False),
    (RAGGED, 5, 20, 8, True),
    (WIDE_GROUP, 8, 150, 6, True),
])
def test_batch_steps_match_oracle(cfg, n, plen, steps, graph):
    import torch
    from decode_step_05_amd import Decoder
    say(f"[batch] cfg={cfg.name} n={n} prompts {plen}..{plen + 3 * (n - 1)} steps={steps} graph={graph} seeds=(0,10+s)")
    w = make_weights(cfg, seed=0)
    prompts = _prompts(cfg, n, plen)
    refs = [OracleDecoder(cfg, w).generate(p, steps) for p in prompts]
    dec = Decoder(cfg, w, graph=graph)
    seqs = [dec.sequence() for _ in range(n)]
    for q, p in zip(seqs, prompts):
        q.prefill(p)
    worst = (0.0, 0.0)
    for k in range(steps):
        dec.step_batch(seqs, [int(refs[s][1][k]) for s in range(n)])
        for s, q in enumerate(seqs):
            z, a = q.logits()
            z = z.cpu().numpy()
            ma, r = assert_close(z, refs[s][0][k + 1], f"{cfg.name} seq {s} step {k}")
            worst = (max(worst[0], ma), max(worst[1], r))
            assert check_token(int(a.item()), refs[s][0][k + 1], ma), (s, k)
            assert int(a.item()) == greedy(z.astype(np.float64))
    for s, q in enumerate(seqs):
        st = q.status()
        assert st[0] == len(prompts[s]) + steps and st[2] == 0, st
    say(f"[batch] {cfg.name} n={n}: teacher-forced worst max|d|={worst[0]:.2e} rel={worst[1]:.2e}")
    # free-running greedy: every sequence's device-fed chain gives the oracle's tokens
    for q, p in zip(seqs, prompts):
        q.set_len(len(p))
    for _ in range(steps):
        dec.step_batch(seqs)
    torch.cuda.synchronize()
    for s, q in enumerate(seqs):
        got = q.tokens(len(prompts[s]), steps + 1).cpu().numpy()
        want = refs[s][1]
        for k in range(steps + 1):
            if got[k] != want[k]:
                assert check_token(int(got[k]), refs[s][0][k], 1e-2) == "near-tie", (s, k)
                break
    say(f"[batch] {cfg.name} n={n}: free-running chains match the oracle")


@pytest.mark.timeout(300)
def test_batch_graph_equals_eager_and_single_sequence_state():
    """Graph replay and eager launches of the batch give bitwise the same
    logits; and a batch of one sequence is the single-sequence step (same
    length, argmax, history and logits)."""
    import torch
    from decode_step_05_amd import Decoder
    cfg = TINY
    say(f"[batch] graph vs eager cfg={cfg.name} n=4")
    w = make_weights(cfg, seed=0)
    prompts = _prompts(cfg, 4, 30)
    out = []
    for graph in (True, False, True):
        dec = Decoder(cfg, w, graph=graph)
        seqs = [dec.sequence() for _ in range(4)]
        for q, p in zip(seqs, prompts):
            q.prefill(p)
        zs = []
        for _ in range(5):
            dec.step_batch(seqs)
            zs.append(np.stack([q.logits()[0].cpu().numpy() for q in seqs]))
        out.append(np.stack(zs))
        torch.cuda.synchronize()
    assert np.array_equal(out[0], out[1]), "batched graph replay differs from eager launches"
    assert np.array_equal(out[0], out[2]), "two batched runs differ"
    dec = Decoder(cfg, w)
    a, b = dec.sequence(), dec.sequence()
    a.prefill(prompts[0])
    b.prefill(prompts[0])
    for _ in range(5):
        a.step()
        dec.step_batch([b])
    assert a.status() == b.status()
    n = len(prompts[0]) + 6
    assert np.array_equal(a.tokens(0, n).cpu().numpy(), b.tokens(0, n).cpu().numpy())
    assert np.array_equal(b.logits()[0].cpu().numpy(), a.logits()[0].cpu().numpy()), "batch of one vs single step"


@pytest.mark.timeout(300)
def test_batch_sampled_pass_at_n():
    """pass@N: 8 continuations of one prompt, each step a temperature draw per
    sequence (lf_sample over the 8 rows of logits, seeded u) fed back through
    the batch. The oracle follows each sequence with the GPU's tokens and
    draws its own token from its own logits with the same u; a different draw
    is accepted only within the logits' error of an interval boundary."""
    import torch
    from decode_step_05_amd import Decoder
    from decode_step_05_amd import lfdecode as C
    cfg, n, steps, T = TINY, 8, 12, 0.8
    say(f"[batch] sampled pass@{n} cfg={cfg.name} prompt 64 (seed 1) steps={steps} T={T}")
    w = make_weights(cfg, seed=0)
    prompt = make_prompt(cfg, 64, seed=1)
    orc = OracleDecoder(cfg, w)
    caches = []
    z0 = None
    for _ in range(n):
        c = orc.new_cache()
        z0 = orc.forward_sequence(tokens=prompt, cache=c)[-1]
        caches.append(c)
    dec = Decoder(cfg, w)
    seqs = [dec.sequence() for _ in range(n)]
    for q in seqs:
        q.prefill(prompt)
    rng = np.random.default_rng(8)
    zbuf = torch.empty((n, cfg.vocab), dtype=torch.float32, device="cuda")
    tok = torch.empty(n, dtype=torch.int32, device="cuda")
    ref_z = [z0] * n
    differ = 0
    for k in range(steps):
        for s, q in enumerate(seqs):
            C.lf_logits(dec.handle, q.handle, zbuf[s])
        u = rng.random(n).astype(np.float32)
        C.lf_sample(zbuf, T, torch.from_numpy(u).cuda(), tok)
        got_z = zbuf.cpu().numpy()
        drawn = tok.cpu().numpy()
        for s in range(n):
            ma, _ = assert_close(got_z[s], ref_z[s], f"seq {s} step {k}")
            o = sample_token(ref_z[s], T, float(u[s]))
            if int(drawn[s]) != o:
                lo, hi = interval_of(ref_z[s], T, int(drawn[s]))
                d = 2 * ma / T + 1e-5
                assert lo - d <= u[s] < hi + d, (s, k, int(drawn[s]), o)
                differ += 1
        dec.step_batch(seqs, tok)
        for s in range(n):
            ref_z[s] = orc.step(caches[s], token=int(drawn[s]))
    for s, q in enumerate(seqs):
        assert q.status()[0] == len(prompt) + steps
    assert len({tuple(q.tokens(len(prompt) + 1, steps).cpu().numpy()) for q in seqs}) > 1, "all draws alike"
    say(f"[batch] sampled pass@{n}: {differ} of {n * steps} draws differ from the oracle's (near a boundary)")
    assert differ <= 2


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n", [8, 3, 2])
def test_batch_full_model_at_ctx4096(n):
    """n sequences of the full model over one synthetic cache, of lengths
    4092, 4087, ... (each its own), 3 batched steps each fed its own token:
    all 32000 logits of every sequence and step against the float64 oracle.
    The batch sizes take different attention split plans: at 8 sequences 4
    splits per sequence and kv head, read in double-buffered rounds on every
    layer; at 3 and 2, 10 and 16 splits on the full-attention layers (double
    buffered) and 8 splits of 128 keys, one round each, on the windowed ones."""
    import torch
    from decode_step_05_amd import Decoder
    cfg, steps = FULL, 3
    lens = [4092 - 5 * s for s in range(n)]
    say(f"[batch] full model n={n} cache lengths {lens} (seed 2) steps={steps}")
    w = make_weights(cfg, seed=0, threads=16)
    K, V = make_kv(cfg, max(lens), seed=2)
    toks = [[17 + 101 * s + 7 * k for k in range(steps)] for s in range(n)]
    ref = []
    orc = OracleDecoder(cfg, w)
    for s in range(n):
        c = orc.new_cache()
        orc.load_cache(c, K[:, :lens[s]], V[:, :lens[s]])
        ref.append([orc.step(c, token=toks[s][k]) for k in range(steps)])
        del c
    del orc
    say("[batch] full model: oracle done")
    dec = Decoder(cfg, w)
    del w
    seqs = [dec.sequence() for _ in range(n)]
    for q, L in zip(seqs, lens):
        q.load_cache(K[:, :L], V[:, :L])
    worst = (0.0, 0.0)
    for k in range(steps):
        dec.step_batch(seqs, [toks[s][k] for s in range(n)])
        for s, q in enumerate(seqs):
            z, a = q.logits()
            ma, r = assert_close(z.cpu().numpy(), ref[s][k], f"full seq {s} (p={lens[s] + k}) step {k}")
            worst = (max(worst[0], ma), max(worst[1], r))
            assert check_token(int(a.item()), ref[s][k], ma)
    torch.cuda.synchronize()
    for q, L in zip(seqs, lens):
        st = q.status()
        assert st[0] == L + steps and st[2] == 0, st
    say(f"[batch] full model n={n}: worst max|d|={worst[0]:.2e} rel={worst[1]:.2e}")


@pytest.mark.timeout(300)
def test_batch_edge_positions():
    """One batch whose sequences sit at the edges of the context: an empty
    sequence (its first position attends to itself only), one cached key,
    63, 64 and 65 cached keys around the 64-key window of the tiny decoder's
    first layer, and the last position of the context (4095 cached keys):
    each sequence's logits and greedy token against the oracle; then a step
    of the batch, which now holds a full sequence, is refused."""
    import torch
    from decode_step_05_amd import Decoder
    from decode_step_05_amd import lfdecode as C
    cfg = TINY
    lens = [0, 1, 63, 64, 65, cfg.max_ctx - 1]
    toks = [5 + 37 * s for s in range(len(lens))]
    say(f"[batch] edge positions cfg={cfg.name} cache lengths {lens} (seed 2) tokens {toks}")
    w = make_weights(cfg, seed=0)
    K, V = make_kv(cfg, max(lens), seed=2)
    orc = OracleDecoder(cfg, w)
    refs = []
    for L, t in zip(lens, toks):
        c = orc.new_cache()
        if L:
            orc.load_cache(c, K[:, :L], V[:, :L])
        refs.append(orc.step(c, token=t))
    dec = Decoder(cfg, w)
    seqs = [dec.sequence() for _ in lens]
    for q, L in zip(seqs, lens):
        if L:
            q.load_cache(K[:, :L], V[:, :L])
        else:
            q.set_len(0)
    dec.step_batch(seqs, toks)
    worst = (0.0, 0.0)
    for s, q in enumerate(seqs):
        z, a = q.logits()
        ma, r = assert_close(z.cpu().numpy(), refs[s], f"edge seq {s} (p={lens[s]})")
        worst = (max(worst[0], ma), max(worst[1], r))
        assert check_token(int(a.item()), refs[s], ma), s
        st = q.status()
        assert st[0] == lens[s] + 1 and st[2] == 0, (s, st)
    with pytest.raises(C.LfError) as e:
        dec.step_batch(seqs, toks)
    assert e.value.code == C.LF_ERANGE
    torch.cuda.synchronize()
    say(f"[batch] edge positions: worst max|d|={worst[0]:.2e} rel={worst[1]:.2e}")
