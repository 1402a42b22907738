"""The recorded-graph cache of a model is bounded: past 64 keys (a
sequence with its hidden-state buffers; a batch of sequence handles) a step
launches its kernels one by one instead of recording another graph, with the
same results. Through the C ABI, on the tiny decoder."""
import numpy as np
import pytest

from synth import TINY, make_hidden, make_kv, make_prompt, make_weights

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.mark.timeout(300)
def test_hidden_steps_past_the_cache_bound_match_eager():
    import torch
    from decode_step_05_amd import Decoder
    cfg = TINY.replace(vocab=0, name="tiny_hidden")
    say(f"[graphs] cfg={cfg.name}: 70 hidden-state steps, each with its own output buffer (seeds 0, 2)")
    w = make_weights(cfg, seed=0)
    K, V = make_kv(cfg, 20, seed=2)
    dec = Decoder(cfg, w)
    seq = dec.sequence()
    seq.load_cache(K, V)
    xin = torch.from_numpy(make_hidden(cfg, seed=2)).cuda()
    outs = [torch.empty_like(xin) for _ in range(70)]
    for o in outs:  # 70 graph keys: the last 6 run eagerly
        seq.set_len(20)
        seq.step_hidden(xin, o)
    dec.set_graph(False)
    ref = torch.empty_like(xin)
    seq.set_len(20)
    seq.step_hidden(xin, ref)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, ref), i
    assert seq.status()[2] == 0


@pytest.mark.timeout(300)
def test_batched_steps_past_the_cache_bound_match_eager():
    import torch
    from decode_step_05_amd import Decoder
    cfg = TINY
    say(f"[graphs] cfg={cfg.name}: batched steps of all 72 ordered pairs of 9 sequences (seeds 0, 1)")
    w = make_weights(cfg, seed=0)
    dec = Decoder(cfg, w)
    seqs = [dec.sequence() for _ in range(9)]
    lens = []
    for i, q in enumerate(seqs):
        p = make_prompt(cfg, 20 + i, seed=1 + i)
        q.prefill(p)
        lens.append(len(p))
    pairs = [(i, j) for i in range(9) for j in range(9) if i != j]

    def run():
        out = []
        for i, j in pairs:
            a, b = seqs[i], seqs[j]
            a.set_len(lens[i])
            b.set_len(lens[j])
            dec.step_batch([a, b], [3 + i, 5 + j])
            out.append((a.logits()[0].cpu().numpy(), b.logits()[0].cpu().numpy()))
        torch.cuda.synchronize()
        return out

    graph = run()  # 72 keys: the last 8 run eagerly
    dec.set_graph(False)
    eager = run()
    for k, ((a, b), (a2, b2)) in enumerate(zip(graph, eager)):
        assert np.array_equal(a, a2) and np.array_equal(b, b2), pairs[k]
    for q in seqs:
        assert q.status()[2] == 0
