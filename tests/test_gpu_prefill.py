"""GPU parity of the batched prompt pass (lf_prefill_batched: matrix-core
GEMMs and attention over chunks of the prompt) against the CPU oracle, through
the C ABI.

For every shape: the logits and greedy token of the last prompt position, the
keys and values written to the cache (compared with the oracle's
full-sequence pass, which fills its cache as decoding would), and decode
steps that continue from the batched pass. The chunk sizes leave ragged
chunks, and the sliding windows are narrower than a chunk. The 15-layer
decoder's 512- and 3584-token prompts are compared with the stored oracle
results of those workloads. Acceptance: tests/parity.py.
"""
import os

import numpy as np
import pytest

from oracle import OracleDecoder
from synth import TINY, WORKLOADS, DecoderConfig, make_prompt, make_weights

from parity import MAX_ABS, MAX_REL, assert_close, check_token, greedy_fp32, vec_err
from test_gpu_parity import RAGGED, WIDE_GROUP

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# one query head per kv head (G = 1) at head_dim 128, 3 lanes, a window
# narrower than the chunk on the second layer
MHA = DecoderConfig("mha", n_layers=2, d_model=384, n_q_heads=3, n_kv_heads=3, head_dim=128, ffn=528,
                    vocab=600, n_lanes=3, max_ctx=200, windows=(0, 45))


# Projections wide enough, over a prompt long enough, that the 128 x 256
# double-buffered GEMM runs (its grid fills the device) on ragged tiles: 4000
# positions in one chunk (the last 128-row tile holds 32 rows), gate/up 2000
# rows and O / down 2056 rows (part-filled last 256-row tiles), K = 2056 and
# 1000 (a part-filled last K step, and an odd number of K steps).
WIDE_RAGGED = DecoderConfig("wide_ragged", n_layers=2, d_model=2056, n_q_heads=8, n_kv_heads=4, head_dim=64,
                            ffn=1000, vocab=1000, n_lanes=4, max_ctx=4096, windows=(0, 300))


def say(*a):
    print(*a, flush=True)


def _cache_np(seq, n):
    """The device caches as [layer, pos, kv_head, hd] float64 for positions [0, n)."""
    c = seq.dec.c
    L, hkv, hd = c.n_layers, c.n_kv_heads, c.head_dim
    out = []
    for t in (seq.K, seq.V):
        out.append(t[:, :, :n].permute(0, 2, 1, 3, 4).reshape(L, n, hkv, hd).float().cpu().numpy().astype(np.float64))
    return out


def _check_caches(seq, cache, n, what):
    K, V = _cache_np(seq, n)
    worst = 0.0
    for l in range(K.shape[0]):
        for name, got, want in (("K", K[l], cache["K"][l, :n]), ("V", V[l], cache["V"][l, :n])):
            a, r = vec_err(got.ravel(), want.ravel())
            assert a <= MAX_ABS and r <= MAX_REL, f"{what}: layer {l} {name} cache max|d|={a:.3e} rel={r:.3e}"
            worst = max(worst, r)
    return worst


@pytest.mark.parametrize("cfg,plen,chunk,steps,mode", [
    (TINY, 1, 1, 4, "graph"),
    (TINY, 128, 128, 8, "graph"),
    (TINY, 128, 48, 8, "graph"),
    (TINY, 128, 48, 8, "eager"),
    (RAGGED, 40, 17, 6, "graph"),
    (WIDE_GROUP, 150, 64, 6, "graph"),
    (MHA, 130, 100, 6, "graph"),
])
def test_prefill_batched_matches_oracle(cfg, plen, chunk, steps, mode):
    """The decode steps after the batched pass run in the given launch mode."""
    import torch
    from decode_step_05_amd import Decoder
    from decode_step_05_amd import lfdecode as C

    say(f"[prefill] cfg={cfg.name} prompt={plen} chunk={chunk} steps={steps} mode={mode} seeds=(0,1)")
    w = make_weights(cfg, seed=0)
    prompt = make_prompt(cfg, plen, seed=1)
    o = OracleDecoder(cfg, w)
    cache = o.new_cache()
    o.forward_sequence(tokens=prompt, cache=cache)
    ref_z, ref_t = o.generate(prompt, steps)

    modes = {"graph": C.LF_MODE_GRAPH, "eager": C.LF_MODE_EAGER}
    dec = Decoder(cfg, w, mode=modes[mode])
    assert dec.mode == modes[mode]
    seq = dec.sequence()
    seq.prefill_batched(prompt, chunk=chunk)
    z, a = seq.logits()
    z = z.cpu().numpy()
    amax, rel = assert_close(z, ref_z[0], f"{cfg.name} last prompt position")
    assert check_token(int(a.item()), ref_z[0], amax), f"{cfg.name}: token {int(a.item())} != oracle {ref_t[0]}"
    assert int(a.item()) == greedy_fp32(z)
    assert seq.status()[0] == plen
    hist = seq.tokens(0, plen + 1).cpu().numpy()
    assert np.array_equal(hist[:plen], prompt) and hist[plen] == int(a.item())
    crel = _check_caches(seq, cache, plen, cfg.name)

    # decoding continues from the cache the batched pass wrote
    for s in range(steps):
        seq.step(int(ref_t[s]))
        zs, _ = seq.logits()
        assert_close(zs.cpu().numpy(), ref_z[s + 1], f"{cfg.name} decode step {s} after the batched pass")
    torch.cuda.synchronize()
    say(f"[prefill] {cfg.name}: logits max|d|={amax:.2e} rel={rel:.2e}, worst cache rel={crel:.2e}, "
        f"{steps} decode steps close")


def test_prefill_batched_after_a_prefix_and_bad_token():
    """Positions already in the cache (written by token-by-token steps) are
    attended to by the batched pass, which starts at len > 0; a token id out
    of range is clamped and flagged as in the decode path."""
    import torch
    from decode_step_05_amd import Decoder

    cfg = TINY
    say(f"[prefill] prefix cfg={cfg.name} prompt=50+78 chunk=32")
    w = make_weights(cfg, seed=0)
    prompt = make_prompt(cfg, 128, seed=1)
    o = OracleDecoder(cfg, w)
    cache = o.new_cache()
    ref = o.forward_sequence(tokens=prompt, cache=cache)
    dec = Decoder(cfg, w)
    seq = dec.sequence()
    seq.prefill(prompt[:50])
    seq.prefill_batched(prompt[50:], chunk=32)
    z, _ = seq.logits()
    assert_close(z.cpu().numpy(), ref[-1], "prefix + batched")
    _check_caches(seq, cache, 128, "prefix + batched")
    assert seq.status()[2] == 0

    bad = np.array(prompt[:20], np.int32)
    bad[7] = cfg.vocab + 5
    seq2 = dec.sequence()
    seq2.prefill_batched(bad, chunk=16)
    assert seq2.status()[2] & 1, "out-of-range token not flagged"
    fixed = bad.copy()
    fixed[7] = cfg.vocab - 1
    ref2 = o.forward_sequence(tokens=fixed)
    assert_close(seq2.logits()[0].cpu().numpy(), ref2[-1], "clamped token")
    torch.cuda.synchronize()


def test_prefill_batched_argument_errors():
    from decode_step_05_amd import Decoder
    from decode_step_05_amd import lfdecode as C

    cfg = TINY
    say(f"[prefill] argument errors cfg={cfg.name}")
    dec = Decoder(cfg, make_weights(cfg, seed=0))
    seq = dec.sequence()
    import torch
    toks = torch.zeros(8, dtype=torch.int32, device="cuda")
    need = C.lf_prefill_workspace_bytes(dec.c, 8)
    ws = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    with pytest.raises(C.LfError, match="workspace"):
        C.lf_prefill_batched(dec.handle, seq.handle, toks, 8, ws[: need - 256])
    with pytest.raises(C.LfError, match="aligned"):
        C.lf_prefill_batched(dec.handle, seq.handle, toks, 8, ws[16:])
    with pytest.raises(C.LfError, match="chunk"):
        C.lf_prefill_batched(dec.handle, seq.handle, toks, 0, ws)
    seq.set_len(cfg.max_ctx - 4)
    with pytest.raises(C.LfError) as e:
        C.lf_prefill_batched(dec.handle, seq.handle, toks, 8, ws)
    assert e.value.code == C.LF_ERANGE
    assert seq.len == cfg.max_ctx - 4


@pytest.mark.timeout(600)
def test_prefill_batched_wide_ragged_tiles():
    """WIDE_RAGGED: a 4000-position prompt as one chunk, then 2 decode steps:
    the last position's logits, the caches and the steps against the oracle."""
    import torch
    from decode_step_05_amd import Decoder

    cfg, plen, steps = WIDE_RAGGED, 4000, 2
    say(f"[prefill] cfg={cfg.name} prompt={plen} chunk={plen} steps={steps} seeds=(0,1)")
    w = make_weights(cfg, seed=0)
    prompt = make_prompt(cfg, plen, seed=1)
    o = OracleDecoder(cfg, w)
    cache = o.new_cache()
    o.forward_sequence(tokens=prompt, cache=cache)
    ref_z, ref_t = o.generate(prompt, steps)
    say(f"[prefill] {cfg.name}: oracle done")
    dec = Decoder(cfg, w)
    seq = dec.sequence()
    seq.prefill_batched(prompt, chunk=plen)
    z, a = seq.logits()
    z = z.cpu().numpy()
    amax, rel = assert_close(z, ref_z[0], f"{cfg.name} last prompt position")
    assert check_token(int(a.item()), ref_z[0], amax)
    assert seq.status()[0] == plen
    crel = _check_caches(seq, cache, plen, cfg.name)
    for s in range(steps):
        seq.step(int(ref_t[s]))
        zs, _ = seq.logits()
        assert_close(zs.cpu().numpy(), ref_z[s + 1], f"{cfg.name} decode step {s} after the batched pass")
    torch.cuda.synchronize()
    say(f"[prefill] {cfg.name}: logits max|d|={amax:.2e} rel={rel:.2e}, worst cache rel={crel:.2e}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,chunk", [("ctx1024", 200), ("ctx4096", 1024), ("ctx4096", 2048), ("ctx4096", 3584)])
def test_prefill_batched_full_size_matches_stored_oracle(name, chunk):
    """The 15-layer decoder's prompt (512 positions in chunks of 200, 200, 112;
    3584 in chunks of 1024, the last one 512; 3584 in chunks of 2048 and 1536,
    and as one chunk, where the tail tiles of the GEMMs are split over K), then
    32 teacher-forced decode steps over the cache it wrote, against the stored
    oracle results of the generation workload."""
    import torch
    from decode_step_05_amd import Decoder

    g = np.load(os.path.join(GOLDEN, f"oracle_{name}.npz"))
    wl = WORKLOADS[name]
    cfg = wl.cfg
    say(f"[prefill] {name}: batched prompt {wl.prompt_len} chunk {chunk}, seeds ({wl.weight_seed},{wl.prompt_seed})")
    w = make_weights(cfg, seed=wl.weight_seed, threads=16)
    prompt = make_prompt(cfg, wl.prompt_len, seed=wl.prompt_seed)
    dec = Decoder(cfg, w)
    del w
    seq = dec.sequence()
    seq.prefill_batched(prompt, chunk=chunk)
    z, a = seq.logits()
    a0, r0 = vec_err(z.cpu().numpy(), g["full"][0])
    assert a0 <= MAX_ABS and r0 <= MAX_REL, f"last prompt position: max|d|={a0:.3e} rel={r0:.3e}"
    toks = g["tokens"]
    assert int(a.item()) == toks[0] or g["gaps"][0] <= 2 * a0
    idx = torch.from_numpy(g["sample_idx"].astype(np.int64)).cuda()
    top_i = torch.from_numpy(g["top_i"].astype(np.int64)).cuda()
    worst = (a0, r0)
    for s in range(1, 33):
        seq.step(int(toks[s - 1]))
        zs, _ = seq.logits()
        a1, r1 = vec_err(zs[idx].cpu().numpy(), g["sample_v"][s])
        a2, _ = vec_err(zs[top_i[s]].cpu().numpy(), g["top_v"][s])
        assert max(a1, a2) <= MAX_ABS and r1 <= MAX_REL, f"decode step {s}: max|d|={max(a1, a2):.3e} rel={r1:.3e}"
        worst = (max(worst[0], a1, a2), max(worst[1], r1))
    torch.cuda.synchronize()
    say(f"[prefill] {name}: last prompt position and 32 decode steps, worst max|d|={worst[0]:.2e} rel={worst[1]:.2e}")


@pytest.mark.timeout(600)
def test_prefill_batched_whole_context_in_one_chunk():
    """Maximum sizes: the 3584-token prompt followed by the oracle's 512 greedy
    tokens, 4096 positions (the whole context) as one chunk of 4096, must give
    the stored oracle logits of position 4095 (computed there by 512
    teacher-forced decode steps) and leave the sequence full."""
    import torch
    from decode_step_05_amd import Decoder
    from decode_step_05_amd import lfdecode as C

    name = "ctx4096"
    g = np.load(os.path.join(GOLDEN, f"oracle_{name}.npz"))
    wl = WORKLOADS[name]
    cfg = wl.cfg
    say(f"[prefill] {name}: whole context 4096 in one chunk, seeds ({wl.weight_seed},{wl.prompt_seed})")
    w = make_weights(cfg, seed=wl.weight_seed, threads=16)
    prompt = make_prompt(cfg, wl.prompt_len, seed=wl.prompt_seed)
    toks = np.concatenate([prompt, g["tokens"][:wl.steps]]).astype(np.int32)
    assert toks.size == cfg.max_ctx
    dec = Decoder(cfg, w)
    del w
    seq = dec.sequence()
    seq.prefill_batched(toks, chunk=cfg.max_ctx)
    z, a = seq.logits()
    k = list(g["full_at"]).index(wl.steps)
    a0, r0 = vec_err(z.cpu().numpy(), g["full"][k])
    assert a0 <= MAX_ABS and r0 <= MAX_REL, f"position 4095: max|d|={a0:.3e} rel={r0:.3e}"
    assert int(a.item()) == g["tokens"][wl.steps] or g["gaps"][wl.steps] <= 2 * a0
    assert seq.status()[0] == cfg.max_ctx
    with pytest.raises(C.LfError) as e:
        seq.step(0)
    assert e.value.code == C.LF_ERANGE
    torch.cuda.synchronize()
    say(f"[prefill] {name}: position 4095 after one 4096-position chunk, max|d|={a0:.2e} rel={r0:.2e}")
