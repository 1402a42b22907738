"""A wait between workgroups that gives up must be reported, not hidden:
with the model's give-up flag raised from the host (as a bounded poll that
ran out would raise it; no kernel faults or hangs), the next step sets bit 1
of lf_kv_status, for the split-KV attention and its merge (tiny decoder,
graph replay and eager launches), the batched step, and QKV fused with
attention (one Laneformer-shaped layer); lf_kv_set_len clears the flag, and
the same step then gives the oracle's result."""
import numpy as np
import pytest

from oracle import OracleDecoder
from synth import LAYER_FULL, TINY, make_hidden, make_kv, make_prompt, make_weights

from parity import assert_close

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _gave_up(seq):
    return bool(seq.status()[2] & 2)


@pytest.mark.timeout(300)
def test_give_up_reported_and_cleared():
    import torch
    from decode_step_05_amd import Decoder
    from decode_step_05_amd import lfdecode as C
    cfg, plen, tok = TINY, 40, 77
    say(f"[give-up] cfg={cfg.name} prompt={plen} (seed 1) token={tok}")
    w = make_weights(cfg, seed=0)
    prompt = make_prompt(cfg, plen, seed=1)
    orc = OracleDecoder(cfg, w)
    cache = orc.new_cache()
    orc.forward_sequence(tokens=prompt, cache=cache)
    want = orc.step(cache, token=tok)
    dec = Decoder(cfg, w)
    for mode in (C.LF_MODE_GRAPH, C.LF_MODE_EAGER):
        dec.set_mode(mode)
        seq = dec.sequence()
        seq.prefill(prompt)
        assert not _gave_up(seq)
        C.lf_model_raise_give_up(dec.handle)
        seq.step(tok)
        assert _gave_up(seq), f"mode {mode}: a step after a give-up must report it"
        seq.set_len(plen)
        assert not _gave_up(seq)
        seq.step(tok)
        assert not _gave_up(seq)
        z, _ = seq.logits()
        a, r = assert_close(z.cpu().numpy(), want, f"mode {mode} after the flag was cleared")
        say(f"[give-up] mode {mode}: reported, cleared, then max|d|={a:.2e} rel={r:.2e}")
        del seq
    # batched step: the flag is the model's, so both sequences report it
    dec.set_mode(C.LF_MODE_GRAPH)
    seqs = [dec.sequence() for _ in range(2)]
    for q in seqs:
        q.prefill(prompt)
    C.lf_model_raise_give_up(dec.handle)
    dec.step_batch(seqs, [tok, tok])
    assert all(_gave_up(q) for q in seqs)
    for q in seqs:
        q.set_len(plen)
    assert not any(_gave_up(q) for q in seqs)
    dec.step_batch(seqs, [tok, tok])
    for s, q in enumerate(seqs):
        assert not _gave_up(q)
        assert_close(q.logits()[0].cpu().numpy(), want, f"batched sequence {s} after the flag was cleared")
    torch.cuda.synchronize()
    say("[give-up] batched step: reported, cleared, then close to the oracle")


@pytest.mark.timeout(300)
def test_give_up_reported_by_fused_qkv_attention():
    import torch
    from decode_step_05_amd import Decoder
    from decode_step_05_amd import lfdecode as C
    cfg, kv_len = LAYER_FULL, 300
    say(f"[give-up] cfg={cfg.name} kv={kv_len} (seed 2) hidden step, fused")
    w = make_weights(cfg, seed=0)
    K, V = make_kv(cfg, kv_len, seed=2)
    x = make_hidden(cfg, seed=3)
    orc = OracleDecoder(cfg, w)
    cache = orc.new_cache()
    orc.load_cache(cache, K, V)
    want = orc.step(cache, x=x)
    dec = Decoder(cfg, w)
    assert dec.fused
    seq = dec.sequence()
    seq.load_cache(K, V)
    xin = torch.from_numpy(x).cuda()
    xout = torch.empty_like(xin)
    C.lf_model_raise_give_up(dec.handle)
    seq.step_hidden(xin, xout)
    assert _gave_up(seq)
    seq.set_len(kv_len)
    seq.step_hidden(xin, xout)
    assert not _gave_up(seq)
    a, r = assert_close(xout.cpu().numpy(), want, "fused layer after the flag was cleared")
    torch.cuda.synchronize()
    say(f"[give-up] fused layer: reported, cleared, then max|d|={a:.2e} rel={r:.2e}")
