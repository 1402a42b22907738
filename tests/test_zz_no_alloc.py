"""lf_prefill_batched_static, the prompt pass that allocates nothing (its
scratch is an array the library holds on each device), against
lf_prefill_batched with a caller workspace, through the C ABI.

Both run the same kernels with the same chunking, so the logits, the greedy
token, the token history and the K/V caches must be identical; they are also
checked against the oracle (the tiny decoder's logits computed here, the full
model's stored logits of the two generation workloads) at the parity bar.
Each case makes two calls in a row on one sequence, the second with a shorter
prompt, so the second call runs over the scratch the first one left.
"""
import os

import numpy as np
import pytest

from oracle import OracleDecoder
from synth import FULL, TINY, WORKLOADS, make_prompt, make_weights

from parity import assert_close

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def say(*a):
    print(*a, flush=True)


def _state(seq, n):
    """Logits, device argmax, history [0, n+1) and the caches of the first n positions."""
    z, a = seq.logits()
    hist = seq.tokens(0, n + 1)
    return (z.cpu().numpy(), int(a.item()), hist.cpu().numpy(), seq.K[:, :, :n].cpu().numpy(),
            seq.V[:, :, :n].cpu().numpy())


def _same(got, want, what):
    z, a, h, K, V = got
    z2, a2, h2, K2, V2 = want
    assert a == a2, (what, a, a2)
    assert np.array_equal(h, h2), what
    assert np.array_equal(z, z2), (what, float(np.max(np.abs(z - z2))))
    assert np.array_equal(K, K2) and np.array_equal(V, V2), what


@pytest.mark.timeout(300)
def test_static_prompt_pass_tiny_two_calls():
    import torch
    from decode_step_05_amd import Decoder
    from decode_step_05_amd import lfdecode as C
    cfg = TINY
    w = make_weights(cfg, seed=0)
    dec = Decoder(cfg, w)
    seq = dec.sequence()
    for n, chunk in ((128, 0), (40, 16)):
        say(f"[no-alloc] cfg={cfg.name} prompt={n} chunk={chunk} seeds=(0,1)")
        prompt = make_prompt(cfg, n, seed=1 + n)
        t = torch.as_tensor(prompt).cuda()
        seq.set_len(0)
        C.lf_prefill_batched_static(dec.handle, seq.handle, t, chunk)
        got = _state(seq, n)
        assert seq.status() == (n, got[1], 0)
        ref = dec.sequence()
        ref.prefill_batched(t, chunk=n if chunk == 0 else chunk)
        _same(got, _state(ref, n), f"tiny n={n}")
        want = OracleDecoder(cfg, w).generate(prompt, 0)[0][0]
        a, r = assert_close(got[0], want, f"tiny n={n} vs oracle")
        say(f"[no-alloc] tiny n={n}: identical to the workspace pass; vs oracle max|d|={a:.2e} rel={r:.2e}")
        del ref
    torch.cuda.synchronize()


@pytest.mark.timeout(600)
def test_static_prompt_pass_full_model_two_calls():
    """The 3584-token prompt (chunk 0: the largest that fits, 282 positions,
    so 12 chunks and a ragged 200), then the 512-token prompt on the same
    sequence (282 + 230), each against the workspace pass with chunk 282 and
    against the oracle's stored logits of its last position."""
    import torch
    from decode_step_05_amd import Decoder
    from decode_step_05_amd import lfdecode as C
    cfg = FULL
    w = make_weights(cfg, seed=0, threads=16)
    dec = Decoder(cfg, w)
    del w
    seq = dec.sequence()
    for name in ("ctx4096", "ctx1024"):
        wl = WORKLOADS[name]
        g = np.load(os.path.join(GOLDEN, f"oracle_{name}.npz"))
        n = wl.prompt_len
        say(f"[no-alloc] cfg={cfg.name} {name}: prompt {n}, chunk 0 (static scratch {C.LF_STATIC_SCRATCH_BYTES} B)")
        t = torch.as_tensor(make_prompt(cfg, n, seed=wl.prompt_seed)).cuda()
        seq.set_len(0)
        C.lf_prefill_batched_static(dec.handle, seq.handle, t, 0)
        got = _state(seq, n)
        st = seq.status()
        assert st[0] == n and st[2] == 0, st
        ref = dec.sequence()
        ref.prefill_batched(t, chunk=282)
        _same(got, _state(ref, n), name)
        del ref
        torch.cuda.empty_cache()
        k = list(g["full_at"]).index(0)
        a, r = assert_close(got[0], g["full"][k], f"{name} last prompt position vs oracle")
        assert got[1] == int(g["tokens"][0])
        say(f"[no-alloc] {name}: identical to the workspace pass; vs oracle max|d|={a:.2e} rel={r:.2e}")
    # a chunk whose scratch does not fit is refused before any device work
    with pytest.raises(C.LfError, match="static scratch"):
        C.lf_prefill_batched_static(dec.handle, seq.handle, t, 283)
    torch.cuda.synchronize()
