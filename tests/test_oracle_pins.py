"""Pins of the CPU oracle to facts that do not come from the oracle itself:
closed forms, hand-computed special cases, invariants of the method, a
whole-sequence recompute with explicit masks, and the structural facts the
pages state. Each test names the mistake it is there to catch."""
import json
import math
import os

import numpy as np
import pytest

from oracle import (OracleDecoder, apply_rope, attend, greedy, kv_head_of, rmsnorm, silu, softmax,
                    visible_range)
from synth import FULL, LANE, TINY, DecoderConfig, make_prompt, make_weights, param_count

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_cfg(**kw):
    base = dict(name="small", n_layers=2, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16, ffn=96,
                vocab=97, n_lanes=2, max_ctx=64, windows=(5, 0))
    base.update(kw)
    return DecoderConfig(**base)


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_closed_form():
    # with unit gain the output RMS is sqrt(ms / (ms + eps)); catches a dropped
    # sqrt, sum-instead-of-mean, or eps outside the root
    rng = np.random.default_rng(0)
    x = rng.standard_normal(4096) * 3.0
    for eps in (0.0, 1e-5, 0.5):
        y = rmsnorm(x, np.ones_like(x), eps)
        ms = np.mean(x * x)
        assert np.sqrt(np.mean(y * y)) == pytest.approx(math.sqrt(ms / (ms + eps)), rel=1e-12)
        # direction is unchanged
        assert np.allclose(y / x, y[0] / x[0])


def test_rmsnorm_hand_value_and_gain():
    # x = (3, 4): mean square 12.5, so y = (3, 4)/sqrt(12.5) = (0.8485..., 1.1313...)
    y = rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 1.0]), 0.0)
    assert y == pytest.approx([0.848528137423857, 1.131370849898476], rel=1e-12)
    g = np.array([2.0, -0.5])
    assert rmsnorm(np.array([3.0, 4.0]), g, 0.0) == pytest.approx(g * y, rel=1e-12)


# --------------------------------------------------------------------- RoPE

def test_rope_hand_values():
    # hd=2: the only pair rotates by angle p (frequency theta^0 = 1), counter-clockwise
    y = apply_rope(np.array([[1.0, 0.0]]), 1, 10000.0)
    assert y[0] == pytest.approx([math.cos(1), math.sin(1)], abs=1e-15)
    # hd=4: pair (1, 3) has frequency 10000^(-2/4) = 1/100, so p=100 gives angle 1;
    # pair (0, 2) has frequency 1, angle 100. Catches interleaved pairing and a
    # wrong exponent.
    y = apply_rope(np.array([[0.0, 1.0, 0.0, 0.0]]), 100, 10000.0)
    assert y[0] == pytest.approx([0.0, math.cos(1), 0.0, math.sin(1)], abs=1e-14)
    y = apply_rope(np.array([[1.0, 0.0, 0.0, 0.0]]), 100, 10000.0)
    assert y[0] == pytest.approx([math.cos(100), 0.0, math.sin(100), 0.0], abs=1e-13)


def test_rope_invariants():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 128))
    k = rng.standard_normal((3, 128))
    # identity at position 0
    assert np.array_equal(apply_rope(q, 0, 1e4), q)
    # each pair keeps its length
    r = apply_rope(q, 777, 1e4)
    assert np.allclose(r[:, :64] ** 2 + r[:, 64:] ** 2, q[:, :64] ** 2 + q[:, 64:] ** 2, rtol=1e-12)
    # scores depend only on the position difference
    d1 = np.sum(apply_rope(q, 10, 1e4) * apply_rope(k, 3, 1e4), axis=-1)
    d2 = np.sum(apply_rope(q, 4010, 1e4) * apply_rope(k, 4003, 1e4), axis=-1)
    assert np.allclose(d1, d2, rtol=1e-9, atol=1e-9)
    # the sequence form agrees with the single-position form
    seq = apply_rope(np.stack([q, q]), np.array([5, 9]), 1e4)
    assert np.allclose(seq[1], apply_rope(q, 9, 1e4), rtol=1e-15)


# --------------------------------------------------------------------- SiLU

def test_silu_values():
    assert silu(np.array(0.0)) == 0.0
    assert silu(np.array(1.0)) == pytest.approx(0.7310585786300049, rel=1e-15)
    assert silu(np.array(-1.0)) == pytest.approx(-0.2689414213699951, rel=1e-15)
    assert silu(np.array(40.0)) == pytest.approx(40.0, rel=1e-15)
    assert abs(silu(np.array(-40.0))) < 1e-15


# ---------------------------------------------------------------- attention

def test_attention_hand_case_scale():
    # q.k0 = 2 and hd = 4, so the scaled score is 2/sqrt(4) = 1; q.k1 = 0.
    # Output = (e v0 + v1) / (e + 1). Catches a missing or wrong 1/sqrt(hd).
    q = np.array([[2.0, 0, 0, 0]])
    K = np.array([[[1.0, 0, 0, 0]], [[0.0, 1, 0, 0]]])
    V = np.array([[[1.0, 2, 3, 4]], [[-1.0, 0, 5, 0]]])
    e = math.e
    want = (e * V[0, 0] + V[1, 0]) / (e + 1)
    assert attend(q, K, V, 1)[0] == pytest.approx(want, rel=1e-14)


def test_attention_single_key_and_normalisation():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((8, 32))
    K = rng.standard_normal((1, 4, 32))
    V = rng.standard_normal((1, 4, 32))
    out = attend(q, K, V, 4)
    for i in range(8):
        assert np.array_equal(out[i], V[0, kv_head_of(i, 8, 4)])
    s = rng.standard_normal((5, 100)) * 30
    assert np.allclose(softmax(s).sum(-1), 1.0, rtol=1e-14)
    assert np.allclose(softmax(s + 1234.5), softmax(s), rtol=1e-12)


def test_gqa_mapping_consecutive():
    # consecutive query heads share a kv head: 32/16 -> (0,1)->0, (2,3)->1 ...
    assert [kv_head_of(i, 32, 16) for i in range(6)] == [0, 0, 1, 1, 2, 2]
    assert [kv_head_of(i, 8, 4) for i in range(8)] == [0, 0, 1, 1, 2, 2, 3, 3]


def _mha_weights(cfg, w):
    """Same model as MHA: kv head j of the MHA copy = kv head kv_head_of(j) of
    the GQA model (query head j's group), duplicated consecutively."""
    hd, nq, nk = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    group = nq // nk
    out = dict(w)
    for l in range(cfg.n_layers):
        W = w[f"layers.{l}.wqkv"]
        q = W[:nq * hd]
        k = W[nq * hd:(nq + nk) * hd].reshape(nk, hd, -1)
        v = W[(nq + nk) * hd:].reshape(nk, hd, -1)
        k2 = np.repeat(k, group, axis=0).reshape(nq * hd, -1)
        v2 = np.repeat(v, group, axis=0).reshape(nq * hd, -1)
        out[f"layers.{l}.wqkv"] = np.concatenate([q, k2, v2])
    return out


def test_gqa_equals_mha_with_duplicated_kv():
    cfg = small_cfg()
    w = make_weights(cfg, seed=3)
    mha = cfg.replace(n_kv_heads=cfg.n_q_heads)
    toks = make_prompt(cfg, 12, seed=4)
    a = OracleDecoder(cfg, w).forward_sequence(tokens=toks)
    b = OracleDecoder(mha, _mha_weights(cfg, w)).forward_sequence(tokens=toks)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------- masks and SWA

def test_visible_range_matches_mask():
    dec = OracleDecoder(small_cfg(), {})
    for W in (0, 1, 3, 7):
        M = dec.mask(20, W)
        for p in range(20):
            lo, hi = visible_range(p, W)
            assert list(np.nonzero(M[p])[0]) == list(range(lo, hi))
    # window counts the current key: W = 1 sees only itself
    assert visible_range(10, 1) == (10, 11)
    assert visible_range(10, 4) == (7, 11)


def test_swa_equals_full_within_window():
    # P-1: while p + 1 <= W, the sliding window hides nothing
    cfg = small_cfg(windows=(16, 16))
    full = cfg.with_windows((0, 0))
    w = make_weights(cfg, seed=5)
    toks = make_prompt(cfg, 16, seed=6)
    a = OracleDecoder(cfg, w).forward_sequence(tokens=toks)
    b = OracleDecoder(full, w).forward_sequence(tokens=toks)
    assert np.array_equal(a, b)
    # and past the window it does change the result
    toks = make_prompt(cfg, 30, seed=6)
    a = OracleDecoder(cfg, w).forward_sequence(tokens=toks)
    b = OracleDecoder(full, w).forward_sequence(tokens=toks)
    assert np.array_equal(a[:16], b[:16]) and not np.allclose(a[16:], b[16:])


def test_swa_receptive_field_single_layer():
    # one SWA layer of width W: position p reads keys p-W+1..p only, so the
    # token at p-W cannot move its logits while the token at p-W+1 does.
    # Pins the "window includes the current key" reading.
    W = 4
    cfg = small_cfg(n_layers=1, windows=(W,))
    w = make_weights(cfg, seed=7)
    toks = make_prompt(cfg, 12, seed=8)
    dec = OracleDecoder(cfg, w)
    base = dec.forward_sequence(tokens=toks)
    p = 11
    t2 = toks.copy(); t2[p - W] = (t2[p - W] + 1) % cfg.vocab
    assert np.array_equal(dec.forward_sequence(tokens=t2)[p], base[p])
    t3 = toks.copy(); t3[p - W + 1] = (t3[p - W + 1] + 1) % cfg.vocab
    assert not np.allclose(dec.forward_sequence(tokens=t3)[p], base[p])


def test_causality():
    cfg = small_cfg(windows=(0, 0))
    w = make_weights(cfg, seed=9)
    toks = make_prompt(cfg, 10, seed=10)
    dec = OracleDecoder(cfg, w)
    a = dec.forward_sequence(tokens=toks)
    t2 = toks.copy(); t2[7] = (t2[7] + 5) % cfg.vocab
    b = dec.forward_sequence(tokens=t2)
    assert np.array_equal(a[:7], b[:7]) and not np.allclose(a[7], b[7])


# -------------------------------------------- incremental vs whole sequence

@pytest.mark.parametrize("kv_fp16", [False, True])
def test_incremental_equals_full_recompute(kv_fp16):
    # P-4: teacher-forced decode with the KV cache equals the whole-sequence
    # pass with explicit masks; the window (5) is exceeded so SWA is active
    cfg = small_cfg()
    w = make_weights(cfg, seed=11)
    toks = make_prompt(cfg, 24, seed=12)
    dec = OracleDecoder(cfg, w, kv_fp16=kv_fp16)
    full = dec.forward_sequence(tokens=toks)
    cache = dec.new_cache()
    for p, t in enumerate(toks):
        z = dec.step(cache, token=t)
        assert np.allclose(z, full[p], rtol=1e-11, atol=1e-11), p
    # prefill by the sequence form then decode equals decode all the way
    cache2 = dec.new_cache()
    dec.forward_sequence(tokens=toks[:10], cache=cache2)
    for p in range(10, 24):
        z = dec.step(cache2, token=toks[p])
        assert np.allclose(z, full[p], rtol=1e-11, atol=1e-11)


def test_kv_cache_holds_fp16_values():
    cfg = small_cfg()
    w = make_weights(cfg, seed=13)
    dec = OracleDecoder(cfg, w, kv_fp16=True)
    cache = dec.new_cache()
    for t in make_prompt(cfg, 6, seed=14):
        dec.step(cache, token=t)
    K = cache["K"][:, :6]
    assert np.array_equal(K.astype(np.float16).astype(np.float64), K)
    dec32 = OracleDecoder(cfg, w, kv_fp16=False)
    c2 = dec32.new_cache()
    for t in make_prompt(cfg, 6, seed=14):
        dec32.step(c2, token=t)
    assert not np.array_equal(c2["K"][:, :6], K)
    assert np.allclose(c2["K"][:, :6], K, rtol=2e-3, atol=1e-3)


# ------------------------------------------------------------- lane split

def test_lane_partition_equals_monolithic():
    # P-3: each lane owns Hq/lanes query heads and Hkv/lanes kv heads and a
    # 1/lanes slice of the FFN; the sum over lanes of the row-parallel
    # products reproduces the monolithic layer. Catches a head mapping that
    # crosses lanes.
    for lanes in (1, 2, 4):
        cfg = TINY.replace(n_layers=1, windows=(0,), vocab=0, n_lanes=lanes)
        w = make_weights(cfg, seed=15)
        dec = OracleDecoder(cfg, w, kv_fp16=False)
        rng = np.random.default_rng(16)
        xs = rng.standard_normal((9, cfg.d_model))
        cache = dec.new_cache()
        dec.forward_sequence(xs=xs[:8], cache=cache)
        p = 8
        want = dec.step(dict(K=cache["K"].copy(), V=cache["V"].copy(), len=8), x=xs[8])

        hd, nq, nk = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
        qpl, kpl, fpl = nq // lanes, nk // lanes, cfg.ffn // lanes
        Wqkv = w["layers.0.wqkv"].astype(np.float64)
        Wo = w["layers.0.wo"].astype(np.float64)
        Wgu = w["layers.0.wgate_up"].astype(np.float64)
        Wd = w["layers.0.wdown"].astype(np.float64)
        x = xs[8]
        h = rmsnorm(x, 1.0, cfg.rms_eps)
        attn = np.zeros(cfg.d_model)
        for L in range(lanes):
            qr = Wqkv[L * qpl * hd:(L + 1) * qpl * hd]
            kr = Wqkv[nq * hd + L * kpl * hd: nq * hd + (L + 1) * kpl * hd]
            vr = Wqkv[(nq + nk) * hd + L * kpl * hd:(nq + nk) * hd + (L + 1) * kpl * hd]
            q = apply_rope((qr @ h).reshape(qpl, hd), p, cfg.rope_theta)
            k = apply_rope((kr @ h).reshape(kpl, hd), p, cfg.rope_theta)
            v = (vr @ h).reshape(kpl, hd)
            K = np.concatenate([cache["K"][0, :8, L * kpl:(L + 1) * kpl], k[None]])
            V = np.concatenate([cache["V"][0, :8, L * kpl:(L + 1) * kpl], v[None]])
            o = attend(q, K, V, kpl)   # lane-local heads only
            attn += Wo[:, L * qpl * hd:(L + 1) * qpl * hd] @ o.reshape(-1)
        x = x + attn
        h = rmsnorm(x, 1.0, cfg.rms_eps)
        f = np.zeros(cfg.d_model)
        for L in range(lanes):
            g = Wgu[L * fpl:(L + 1) * fpl] @ h
            u = Wgu[cfg.ffn + L * fpl:cfg.ffn + (L + 1) * fpl] @ h
            f += Wd[:, L * fpl:(L + 1) * fpl] @ (silu(g) * u)
        assert np.allclose(x + f, want, rtol=1e-10, atol=1e-10), lanes


# ------------------------------------------------- reductions to closed forms

def test_zero_blocks_reduce_to_embedding_head():
    # with W_o = 0 and W_down = 0 every layer passes x through, so
    # logits = W_lm . rmsnorm(E[t]). Catches a missing residual, a tied or
    # swapped embedding / head, and the final norm.
    cfg = small_cfg()
    w = make_weights(cfg, seed=17)
    for l in range(cfg.n_layers):
        w[f"layers.{l}.wo"] = np.zeros_like(w[f"layers.{l}.wo"])
        w[f"layers.{l}.wdown"] = np.zeros_like(w[f"layers.{l}.wdown"])
    dec = OracleDecoder(cfg, w)
    cache = dec.new_cache()
    for t in (3, 50, 96):
        z = dec.step(cache, token=t)
        e = w["embed"][t].astype(np.float64)
        want = w["lm_head"].astype(np.float64) @ (e / np.sqrt(np.mean(e * e) + cfg.rms_eps))
        assert np.allclose(z, want, rtol=1e-12, atol=1e-12)


def test_swiglu_hand_case():
    # d = ffn = 4, attention output zeroed, gate = 1*I, up = 2*I, down = I:
    # out = x + silu(h) * 2h with h = x / rms(x). Catches silu applied to the
    # up half instead of the gate half (which would give silu(2h) * h).
    cfg = DecoderConfig("hand", 1, 4, 1, 1, 4, 4, 0, 1, 8, (0,), rms_eps=0.0)
    I = np.eye(4, dtype=np.float16)
    w = {"layers.0.attn_norm": np.ones(4, np.float16), "layers.0.ffn_norm": np.ones(4, np.float16),
         "layers.0.wqkv": np.ones((12, 4), np.float16), "layers.0.wo": np.zeros((4, 4), np.float16),
         "layers.0.wgate_up": np.concatenate([I, 2 * I]), "layers.0.wdown": I}
    x = np.array([1.0, -2.0, 3.0, 0.5])
    out = OracleDecoder(cfg, w).step(OracleDecoder(cfg, w).new_cache(), x=x)
    rms = math.sqrt((1 + 4 + 9 + 0.25) / 4)
    want = [xi + (xi / rms) / (1 + math.exp(-xi / rms)) * 2 * (xi / rms) for xi in x]
    assert out == pytest.approx(want, rel=1e-14)


def test_greedy_ties_lowest_index():
    assert greedy(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert greedy(np.zeros(7)) == 0
    assert greedy(np.array([-np.inf, -5.0, -5.0])) == 1
    # decided in float32: values equal after rounding to float32 tie
    assert greedy(np.array([1.0, 1.0 + 1e-12, 0.5])) == 0
    assert greedy(np.array([1.0, 1.0 + 1e-6, 0.5])) == 1


def test_generate_feeds_greedy_tokens():
    cfg = small_cfg()
    w = make_weights(cfg, seed=18)
    dec = OracleDecoder(cfg, w)
    prompt = make_prompt(cfg, 8, seed=19)
    logits, toks = dec.generate(prompt, 6)
    assert logits.shape == (7, cfg.vocab)
    assert all(toks[i] == greedy(logits[i]) for i in range(7))
    # teacher forcing by the whole-sequence pass gives the same logits
    seq = np.concatenate([prompt, toks[:6]])
    full = dec.forward_sequence(tokens=seq)
    assert np.allclose(full[7:], logits, rtol=1e-11, atol=1e-11)


# --------------------------------------------------- facts the pages state

def test_page_facts():
    f = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    c = FULL
    assert c.n_layers == f["n_layers"]
    assert sum(1 for w in c.windows if w) == f["n_swa_layers"]
    assert (c.n_q_heads, c.n_kv_heads, c.n_lanes) == (f["n_q_heads"], f["n_kv_heads"], f["n_lanes"])
    assert c.n_q_heads % c.n_lanes == 0 and c.n_kv_heads % c.n_lanes == 0
    assert c.max_ctx == f["max_ctx"]
    assert round(param_count(c) / 1e9, 1) == f["params_billions_stated"]
    # one lane's share is 1/8 of each head-sliced projection
    assert LANE.n_q_heads * 8 == c.n_q_heads and LANE.ffn * 8 == c.ffn
