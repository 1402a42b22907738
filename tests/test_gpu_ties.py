"""Greedy choice on exact logit ties, on the GPU, against the oracle.

Greedy decoding (Kog Laneformer 2B blog, TL;DR) picks the maximal logit; on
an exact tie both sides take the lowest index (the oracle's greedy(), which is
numpy's first-maximum argmax on fp32 logits). Identical LM-head rows give
bitwise identical logits, so copying the row of the maximal logit to chosen
indices makes exact ties there. The model is the tiny 2-layer decoder with a
32000-entry vocabulary, so that its LM head runs in the launch shape of the
full model's: 500 workgroups of 4 waves, wave w of workgroup b holding rows
4b + w + 2000k for k < 16. The tie sets below put the tied rows in one wave
(different row groups), in the waves of one workgroup, in workgroups on
different XCDs, and across the whole launch, plus two all-tie heads: every row
zero (all logits exactly 0) and every row the same.
"""
import numpy as np
import pytest

from oracle import OracleDecoder, greedy
from synth import TINY, make_prompt, make_weights

from parity import assert_close

pytestmark = pytest.mark.gpu

CFG = TINY.replace(vocab=32000, name="tiny_vocab32000")
PROMPT = 12


def say(*a):
    print(*a, flush=True)


def _run(w, prompt):
    """Last-position logits and device argmax after a token-by-token prefill,
    plus the greedy token the step recorded in the history."""
    import torch
    from decode_step_05_amd import Decoder
    dec = Decoder(CFG, w)
    seq = dec.sequence()
    seq.prefill(prompt)
    z, a = seq.logits()
    hist = seq.tokens(len(prompt), 1)
    torch.cuda.synchronize()
    st = seq.status()
    assert st[2] == 0, st
    return z.cpu().numpy(), int(a.item()), int(hist.item())


def _tie_cases(a):
    """(name, rows that receive a copy of row a, whether row a itself is zeroed)."""
    r = a % 2000
    return [
        ("one wave, 16 row groups", [r + 2000 * k for k in range(16)], False),
        ("four waves of one workgroup", [1000, 1001, 1002, 1003], False),
        ("eight workgroups (eight XCDs)", [4 * b + 3 for b in range(1, 9)], False),
        ("first, middle and last workgroup", [2, 16001, 31999], False),
        ("last workgroup only", [1999, 29999, 31999], True),
    ]


@pytest.mark.timeout(300)
def test_exact_ties_take_the_lowest_index():
    w = make_weights(CFG, seed=0)
    prompt = make_prompt(CFG, PROMPT, seed=1)
    say(f"[ties] cfg={CFG.name} prompt={PROMPT} seeds=(0,1): untouched head")
    z0, a0, _ = _run(w, prompt)
    a = int(np.argmax(z0))
    assert a0 == a and z0[a] > 0
    base = w["lm_head"]
    for name, rows, drop in _tie_cases(a):
        head = base.copy()
        head[rows] = base[a]
        if drop and a not in rows:
            head[a] = 0  # its logit becomes 0, below the (positive) maximum
        tie = sorted(set(rows) | (set() if drop else {a}))
        wt = dict(w)
        wt["lm_head"] = head
        say(f"[ties] {name}: rows {tie[:6]}{'...' if len(tie) > 6 else ''} tie at the maximum")
        z, got, hist = _run(wt, prompt)
        tied = z[tie]
        assert np.all(tied == tied[0]), "identical rows must give bitwise identical logits"
        assert np.max(z) == tied[0]
        ref = OracleDecoder(CFG, wt).generate(prompt, 0)[0][0]
        assert_close(z, ref, name)
        assert greedy(ref) == tie[0], (greedy(ref), tie)
        assert got == tie[0] and hist == got, (name, got, hist, tie[0])


@pytest.mark.timeout(300)
@pytest.mark.parametrize("head", ["zero", "one row everywhere"])
def test_all_rows_tied(head):
    # every logit exactly equal: the greedy token is 0, whichever workgroup
    # finishes first
    w = make_weights(CFG, seed=0)
    prompt = make_prompt(CFG, PROMPT, seed=1)
    say(f"[ties] cfg={CFG.name} all {CFG.vocab} rows tied ({head})")
    wt = dict(w)
    if head == "zero":
        wt["lm_head"] = np.zeros_like(w["lm_head"])
    else:
        wt["lm_head"] = np.repeat(w["lm_head"][5:6], CFG.vocab, axis=0)
    z, got, hist = _run(wt, prompt)
    assert np.all(z == z[0])
    if head == "zero":
        assert np.all(z == 0.0)
    ref = OracleDecoder(CFG, wt).generate(prompt, 0)[0][0]
    assert_close(z, ref, f"all tied ({head})")
    assert greedy(ref) == 0
    assert got == 0 and hist == 0, (got, hist)
