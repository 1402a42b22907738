"""GPU parity of the HIP decode step against the CPU oracle, through the C ABI.

Every case prints its name, shape and seed before touching the GPU so a
failing run names itself. Acceptance: tests/parity.py.
"""
import numpy as np
import pytest

from oracle import OracleDecoder
from synth import FULL, LANE, LAYER_FULL, LAYER_SWA, TINY, DecoderConfig, make_hidden, make_kv, make_prompt, make_weights

from parity import assert_close, check_token, greedy_fp32, vec_err

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _dec(cfg, w, graph=True, mode=None):
    from decode_step_05_amd import Decoder
    return Decoder(cfg, w, graph=graph, mode=mode)


def _modes():
    from decode_step_05_amd import lfdecode as C
    return {"graph": C.LF_MODE_GRAPH, "eager": C.LF_MODE_EAGER}


def say(*a):
    print(*a, flush=True)


# A ragged shape: 3 lanes, head_dim 64, widths that are not powers of two and
# leave partial tiles everywhere, windows narrower than the prompt.
RAGGED = DecoderConfig("ragged", n_layers=3, d_model=264, n_q_heads=6, n_kv_heads=3, head_dim=64, ffn=360,
                       vocab=1000, n_lanes=3, max_ctx=96, windows=(7, 0, 13))
# G = 4 query heads per kv head and 2 kv heads per lane at head_dim 128.
WIDE_GROUP = DecoderConfig("group4", n_layers=2, d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1024,
                           vocab=777, n_lanes=1, max_ctx=300, windows=(100, 0))


def _generate_gpu(dec, prompt, ref_toks, steps, force=True):
    """Prefill, then `steps` steps. force=True feeds the oracle's tokens
    (teacher forcing); force=False feeds the device's own greedy tokens."""
    torch = _torch()
    seq = dec.sequence()
    seq.prefill(prompt)
    out = []
    z, a = seq.logits()
    out.append((z.cpu().numpy(), int(a.item())))
    for s in range(steps):
        seq.step(int(ref_toks[s]) if force else None)
        z, a = seq.logits()
        out.append((z.cpu().numpy(), int(a.item())))
    torch.cuda.synchronize()
    return seq, out


@pytest.mark.parametrize("cfg,plen,steps,mode", [
    (TINY, 128, 32, "graph"),
    (TINY, 128, 32, "eager"),
    (RAGGED, 40, 24, "graph"),
    (RAGGED, 40, 24, "eager"),
    (WIDE_GROUP, 150, 12, "graph"),
])
def test_generate_matches_oracle(cfg, plen, steps, mode):
    say(f"[parity] generate cfg={cfg.name} prompt={plen} steps={steps} mode={mode} seeds=(0,1)")
    w = make_weights(cfg, seed=0)
    prompt = make_prompt(cfg, plen, seed=1)
    ref_z, ref_t = OracleDecoder(cfg, w).generate(prompt, steps)
    dec = _dec(cfg, w, mode=_modes()[mode])
    assert dec.mode == _modes()[mode]
    _, out = _generate_gpu(dec, prompt, ref_t, steps, force=True)
    ties = 0
    worst = (0.0, 0.0)
    for s, (z, tok) in enumerate(out):
        a, r = assert_close(z, ref_z[s], f"{cfg.name} step {s}")
        worst = (max(worst[0], a), max(worst[1], r))
        ok = check_token(tok, ref_z[s], a)
        assert ok, f"{cfg.name} step {s}: gpu token {tok} != oracle {ref_t[s]} (gap too large)"
        ties += ok == "near-tie"
        assert tok == greedy_fp32(z), "device argmax disagrees with its own logits"
    say(f"[parity] {cfg.name}: {len(out)} vectors, worst max|d|={worst[0]:.2e} rel={worst[1]:.2e}, near-ties={ties}")
    # free-running greedy chain on the device gives the oracle's tokens
    _, free = _generate_gpu(dec, prompt, ref_t, steps, force=False)
    for s, (_, tok) in enumerate(free):
        if tok != ref_t[s]:
            assert check_token(tok, ref_z[s], 1e-2) == "near-tie", f"free run diverged at step {s}"
            break


def test_graph_replay_equals_eager_and_is_deterministic():
    cfg = RAGGED
    say(f"[parity] graph-vs-eager cfg={cfg.name}")
    w = make_weights(cfg, seed=0)
    prompt = make_prompt(cfg, 30, seed=1)
    runs = []
    for mode in ("graph", "eager", "graph"):
        dec = _dec(cfg, w, mode=_modes()[mode])
        _, out = _generate_gpu(dec, prompt, [0] * 8, 8, force=False)
        runs.append(np.stack([z for z, _ in out]))
    assert np.array_equal(runs[0], runs[1]), "graph replay differs from eager launches"
    assert np.array_equal(runs[0], runs[2]), "two graph runs differ"


def test_rewind_reproduces_logits():
    cfg = TINY
    say(f"[parity] rewind cfg={cfg.name}")
    torch = _torch()
    w = make_weights(cfg, seed=0)
    dec = _dec(cfg, w)
    seq = dec.sequence()
    seq.prefill(make_prompt(cfg, 70, seed=1))
    first = []
    for _ in range(6):
        seq.step()
        first.append(seq.logits()[0].cpu().numpy())
    seq.set_len(70)
    for i in range(6):
        seq.step()
        assert np.array_equal(seq.logits()[0].cpu().numpy(), first[i])
    assert seq.status()[0] == 76
    torch.cuda.synchronize()


def test_kernel_timing_leaves_the_sequence_intact():
    # lf_kernel_time repeats single kernels of the next step; the step that
    # follows must still give the same logits, bit for bit
    cfg = TINY
    say(f"[parity] kernel timing cfg={cfg.name}")
    from decode_step_05_amd import lfdecode as C
    w = make_weights(cfg, seed=0)
    dec = _dec(cfg, w)
    seq = dec.sequence()
    seq.prefill(make_prompt(cfg, 70, seed=1))
    seq.step()
    want = seq.logits()[0].cpu().numpy()
    seq.set_len(70)
    for kind in ("qkv", "attn", "o", "gate_up", "down"):
        for l in range(cfg.n_layers):
            ms = C.lf_kernel_time(dec.handle, seq.handle, kind, l, reps=4, iters=2)
            assert 0.0 < ms < 10.0, (kind, l, ms)
    for kind in ("qkv", "attn", "o", "gate_up", "down"):
        assert 0.0 < C.lf_kernel_time(dec.handle, seq.handle, kind, -1, reps=2, iters=2) < 10.0
    assert seq.status()[0] == 70
    seq.step()
    assert np.array_equal(seq.logits()[0].cpu().numpy(), want)
    with pytest.raises(C.LfError):
        C.lf_kernel_time(dec.handle, seq.handle, "lm_head", 0)


def test_first_position_and_context_limit():
    # ctx = 1 (attention over a single key) and the exact max_ctx boundary
    cfg = TINY.replace(max_ctx=70, name="tiny70")
    say(f"[parity] boundary cfg={cfg.name}")
    from decode_step_05_amd.lfdecode import LF_ERANGE, LfError
    w = make_weights(cfg, seed=0)
    prompt = make_prompt(cfg, 70, seed=1)
    ref = OracleDecoder(cfg, w).forward_sequence(tokens=prompt)
    dec = _dec(cfg, w)
    seq = dec.sequence()
    seq.prefill(prompt[:1])
    assert_close(seq.logits()[0].cpu().numpy(), ref[0], "position 0")
    seq.prefill(prompt[1:69])
    seq.step(int(prompt[69]))
    assert seq.len == 70
    assert_close(seq.logits()[0].cpu().numpy(), ref[69], "last position")
    with pytest.raises(LfError) as e:
        seq.step()
    assert e.value.code == LF_ERANGE
    assert seq.status()[0] == 70


def test_model_freed_before_sequence():
    # regression: a sequence released after its model (as a garbage collector
    # may order it) must not touch the freed model
    import gc
    from decode_step_05_amd import lfdecode as C
    cfg = TINY
    say("[parity] model freed before sequence")
    dec = _dec(cfg, make_weights(cfg, seed=0))
    seq = dec.sequence()
    seq.prefill(np.array([1, 2, 3], dtype=np.int32))
    _torch().cuda.synchronize()
    dec.close()
    with pytest.raises(C.LfError) as e:
        seq.set_len(0)
    assert e.value.code == C.LF_EINVAL
    seq.close()
    del e
    gc.collect()


def test_bad_token_is_clamped_and_flagged():
    cfg = TINY
    say("[parity] bad token")
    w = make_weights(cfg, seed=0)
    dec = _dec(cfg, w)
    seq = dec.sequence()
    seq.prefill(np.array([5, cfg.vocab + 7], dtype=np.int32))
    assert seq.status()[2] == 1
    ref = OracleDecoder(cfg, w).forward_sequence(tokens=np.array([5, cfg.vocab - 1]))
    assert_close(seq.logits()[0].cpu().numpy(), ref[1], "clamped token")


# ----------------------------------------------------- hidden-mode layers

def _hidden_case(cfg, kv_len, seed=2):
    torch = _torch()
    w = make_weights(cfg, seed=0)
    K, V = make_kv(cfg, kv_len, seed=seed)
    x = make_hidden(cfg, seed=seed)
    dec = _dec(cfg, w)
    seq = dec.sequence()
    seq.load_cache(K, V)
    xin = torch.from_numpy(x).cuda()
    xout = torch.empty_like(xin)
    seq.step_hidden(xin, xout)
    got = xout.cpu().numpy()
    orc = OracleDecoder(cfg, w, cache_weights=False)
    cache = orc.new_cache()
    orc.load_cache(cache, K, V)
    want = orc.step(cache, x=x)
    return got, want, seq


@pytest.mark.parametrize("cfg", [LAYER_FULL, LAYER_SWA], ids=["full", "swa"])
def test_single_layer_full_shape(cfg):
    # one Laneformer-shaped layer, cache of 2048 synthetic positions, step at p = 2048
    say(f"[parity] layer cfg={cfg.name} kv=2048 p=2048")
    got, want, _ = _hidden_case(cfg, 2048)
    a, r = assert_close(got, want, cfg.name)
    say(f"[parity] {cfg.name}: max|d|={a:.2e} rel={r:.2e}")


# QKV fused with attention (the default for the Laneformer layer shape):
# positions that start, end and straddle splits, for split sizes of 32, 64,
# 128 and 256 keys (max_ctx 512, the 1024-key window, max_ctx 2000, 4096),
# each against the oracle and against the two-kernel path.
_FUSED_CASES = [
    (LAYER_FULL, (0, 1, 255, 256, 2047, 4095)),
    (LAYER_SWA, (0, 63, 64, 1023, 1024, 1025, 3000)),
    (LAYER_FULL.replace(max_ctx=2000, name="layer_full2000"), (124, 125, 1999)),
    (LAYER_SWA.replace(max_ctx=512, name="layer_swa512"), (31, 32, 511)),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg,lens", _FUSED_CASES, ids=[c.name for c, _ in _FUSED_CASES])
def test_fused_qkv_attention_positions(cfg, lens):
    torch = _torch()
    w = make_weights(cfg, seed=0)
    dec = _dec(cfg, w)
    assert dec.fused, "QKV and attention should run fused for this shape on MI355X"
    orc = OracleDecoder(cfg, w)
    x = make_hidden(cfg, seed=3)
    xin = torch.from_numpy(x).cuda()
    for kv_len in lens:
        say(f"[parity] fused cfg={cfg.name} kv={kv_len} p={kv_len}")
        K, V = make_kv(cfg, kv_len, seed=2)
        seq = dec.sequence()
        seq.load_cache(K, V)
        out = {}
        for fused in (True, False):
            dec.set_fused(fused)
            seq.set_len(kv_len)
            xout = torch.empty_like(xin)
            seq.step_hidden(xin, xout)
            out[fused] = xout.cpu().numpy()
        dec.set_fused(True)
        cache = orc.new_cache()
        orc.load_cache(cache, K, V)
        want = orc.step(cache, x=x)
        a1, r1 = assert_close(out[True], want, f"{cfg.name} fused kv={kv_len}")
        assert_close(out[False], want, f"{cfg.name} two kernels kv={kv_len}")
        d = float(np.max(np.abs(out[True] - out[False])))
        assert d <= 1e-4, (kv_len, d)
        say(f"[parity] fused {cfg.name} kv={kv_len}: max|d|={a1:.2e} rel={r1:.2e} fused-vs-two={d:.1e}")
        del seq


def test_fusion_switch_and_kernel_kinds():
    # QKV and attention run fused only for the Laneformer layer shape; the
    # per-kernel timer refuses kinds the model does not launch
    torch = _torch()
    say("[parity] fusion switch cfg=tiny")
    from decode_step_05_amd import lfdecode as C
    dec = _dec(TINY, make_weights(TINY, seed=0))
    assert not dec.fused
    with pytest.raises(C.LfError):
        dec.set_fused(True)
    dec.set_fused(False)
    seq = dec.sequence()
    seq.prefill(np.array([1, 2, 3], dtype=np.int32))
    with pytest.raises(C.LfError):
        C.lf_kernel_time(dec.handle, seq.handle, "qkv_attn", -1, reps=1, iters=1)
    assert C.lf_kernel_time(dec.handle, seq.handle, "qkv", -1, reps=1, iters=1) > 0
    say("[parity] read bandwidth probe")
    buf = torch.ones(1 << 20, dtype=torch.float32, device="cuda")
    assert C.lf_read_bandwidth(buf, iters=2) > 0


def test_lane_share_full_depth():
    # one lane's slice of all 15 layers at ctx 4096
    say("[parity] lane share kv=4095 p=4095")
    got, want, seq = _hidden_case(LANE, 4095)
    a, r = assert_close(got, want, "lane")
    assert seq.status()[0] == 4096
    say(f"[parity] lane: max|d|={a:.2e} rel={r:.2e}")
    # the same step launched eagerly (the lane's 2 kv heads run QKV and
    # attention as two kernels)
    torch = _torch()
    dec = seq.dec
    xin = torch.from_numpy(make_hidden(LANE, seed=2)).cuda()
    for mode in ("eager",):
        dec.set_mode(_modes()[mode])
        seq.set_len(4095)
        xout = torch.empty_like(xin)
        seq.step_hidden(xin, xout)
        assert seq.status()[0] == 4096 and seq.status()[2] == 0
        a, r = assert_close(xout.cpu().numpy(), want, f"lane {mode}")
        say(f"[parity] lane {mode}: max|d|={a:.2e} rel={r:.2e}")


def test_hidden_in_place():
    torch = _torch()
    cfg = LAYER_SWA.replace(max_ctx=64, d_model=512, ffn=512, n_q_heads=8, n_kv_heads=4, n_lanes=2, name="inplace")
    say(f"[parity] hidden in-place cfg={cfg.name}")
    w = make_weights(cfg, seed=0)
    K, V = make_kv(cfg, 10)
    x = make_hidden(cfg)
    dec = _dec(cfg, w)
    seq = dec.sequence()
    seq.load_cache(K, V)
    buf = torch.from_numpy(x).cuda()
    seq.step_hidden(buf, buf)
    orc = OracleDecoder(cfg, w)
    cache = orc.new_cache()
    orc.load_cache(cache, K, V)
    assert_close(buf.cpu().numpy(), orc.step(cache, x=x), "in place")


# ---------------------------------------------- full model at max context

@pytest.mark.timeout(600)
def test_full_model_step_at_ctx4096():
    # the benchmark's fixed-context step: full 15-layer model, synthetic cache of
    # 4095 positions, one token at p = 4095 (5 full layers see 4096 keys, the
    # SWA layers 1024); the logits are compared in full against the oracle,
    # for QKV and attention fused and as two kernels, replayed and eager
    torch = _torch()
    cfg = FULL
    say("[parity] full model kv=4095 p=4095 token=17")
    w = make_weights(cfg, seed=0)
    K, V = make_kv(cfg, 4095, seed=2)
    results = {}
    for mode in ("graph", "graph-two-kernels", "eager"):
        dec = _dec(cfg, w, mode=_modes()[mode.split("-")[0]])
        if mode == "graph":
            assert dec.fused
        dec.set_fused(mode == "graph")
        seq = dec.sequence()
        seq.load_cache(K, V)
        seq.step(17)
        z, a = seq.logits()
        results[mode] = (z.cpu().numpy(), int(a.item()))
        assert seq.status()[2] == 0
        del seq, dec
    torch.cuda.empty_cache()
    orc = OracleDecoder(cfg, w, cache_weights=False)
    cache = orc.new_cache()
    orc.load_cache(cache, K, V)
    want = orc.step(cache, token=17)
    for mode, (got, tok) in results.items():
        ma, r = assert_close(got, want, f"full@4096 {mode}")
        assert check_token(tok, want, ma), (mode, tok, greedy_fp32(want))
        say(f"[parity] full@4096 {mode}: max|d|={ma:.2e} rel={r:.2e} token={tok}")
    # temperature draws from the full-size logits: the GPU samples its own, the
    # oracle its own, with the same u; a different token only where u lies
    # within 2 max|d| / T (plus fp32 rounding) of the GPU token's interval
    from decode_step_05_amd import lfdecode as C
    from oracle import interval_of, sample_token
    got, _ = results["graph"]
    ma = float(np.abs(got - want).max())
    T, n = 0.8, 16
    u = np.random.default_rng(6).random(n).astype(np.float32)
    zd = torch.from_numpy(np.repeat(got[None, :], n, axis=0)).cuda()
    tok = torch.empty(n, dtype=torch.int32, device="cuda")
    C.lf_sample(zd, T, torch.from_numpy(u).cuda(), tok)
    differ = 0
    for k, g in enumerate(tok.cpu().numpy().tolist()):
        o = sample_token(want, T, float(u[k]))
        if g != o:
            lo, hi = interval_of(want, T, g)
            d = 2 * ma / T + 1e-5
            assert lo - d <= u[k] < hi + d, (k, g, o, float(u[k]), lo, hi)
            differ += 1
    say(f"[parity] full@4096 sampled at T={T}: {differ} of {n} draws differ (near a boundary)")
    assert differ <= 2
