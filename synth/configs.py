"""Decoder shapes and workload recipes.

The Laneformer 2B release fixes: 15 layers; causal grouped-query attention with
32 query and 16 key/value heads spread evenly over 8 lanes; sliding-window
attention on 10 of the 15 layers; FP16 at batch 1; a context of 4,096 tokens
(Kog Laneformer 2B blog, section "Designing the architecture"; asector.ru
summary, sections on architecture and operational risks). The remaining shape
parameters (d_model 4096, head_dim 128, SwiGLU width 7168, vocab 32000 with an
untied LM head, RMSNorm, RoPE theta 10000, window 1024 with full attention on
layers 2, 5, 8, 11 and 14) are not on the pages; they are the plainest choice
that lands on the stated 2.3B parameters.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class DecoderConfig:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int            # 0: hidden-in / hidden-out, no embedding and no LM head
    n_lanes: int
    max_ctx: int
    windows: tuple        # per layer: 0 = full causal, W > 0 = keys j with p - W < j <= p
    rope_theta: float = 10000.0
    rms_eps: float = 1e-5

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    def with_windows(self, windows, name=None) -> "DecoderConfig":
        d = dict(self.__dict__)
        d["windows"] = tuple(windows)
        if name:
            d["name"] = name
        return DecoderConfig(**d)

    def replace(self, **kw) -> "DecoderConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return DecoderConfig(**d)


def param_count(cfg: DecoderConfig) -> int:
    """Weights of the decoder: per-layer projections and two norm gains, the
    final norm gain, and (when vocab > 0) untied embedding and LM head."""
    d, hd = cfg.d_model, cfg.head_dim
    per_layer = (cfg.qkv_rows * d + d * cfg.q_dim + 2 * cfg.ffn * d + d * cfg.ffn + 2 * d)
    total = cfg.n_layers * per_layer + d
    if cfg.vocab:
        total += 2 * cfg.vocab * d
    return total


_FULL_LAYERS = (2, 5, 8, 11, 14)
_SWA_W = 1024


def _pattern(n_layers: int):
    return tuple(0 if l in _FULL_LAYERS else _SWA_W for l in range(n_layers))


# Tiny 2-layer decoder: layer 0 slides a 64-key window, layer 1 is full causal.
TINY = DecoderConfig("tiny", n_layers=2, d_model=256, n_q_heads=8, n_kv_heads=4, head_dim=32,
                     ffn=688, vocab=1024, n_lanes=4, max_ctx=4096, windows=(64, 0))

# One Laneformer-shaped layer, hidden in / hidden out.
LAYER_FULL = DecoderConfig("layer_full", n_layers=1, d_model=4096, n_q_heads=32, n_kv_heads=16,
                           head_dim=128, ffn=7168, vocab=0, n_lanes=8, max_ctx=4096, windows=(0,))
LAYER_SWA = LAYER_FULL.with_windows((_SWA_W,), name="layer_swa")

# The full 15-layer, 2.3B-shaped decoder.
FULL = DecoderConfig("full", n_layers=15, d_model=4096, n_q_heads=32, n_kv_heads=16, head_dim=128,
                     ffn=7168, vocab=32000, n_lanes=8, max_ctx=4096, windows=_pattern(15))

# One lane's share of the full decoder: 4 q / 2 kv heads, 1/8 of the FFN.
LANE = DecoderConfig("lane", n_layers=15, d_model=4096, n_q_heads=4, n_kv_heads=2, head_dim=128,
                     ffn=896, vocab=0, n_lanes=1, max_ctx=4096, windows=_pattern(15))


@dataclass(frozen=True)
class Workload:
    """A seeded run: either a prompt followed by greedy steps (vocab > 0), or a
    synthetic KV cache of `kv_len` positions followed by one hidden-state step."""
    name: str
    cfg: DecoderConfig
    prompt_len: int = 0
    steps: int = 0
    kv_len: int = 0
    weight_seed: int = 0
    prompt_seed: int = 1
    data_seed: int = 2


WORKLOADS = {
    "tiny": Workload("tiny", TINY, prompt_len=128, steps=32),
    "layer_full": Workload("layer_full", LAYER_FULL, kv_len=2048),
    "layer_swa": Workload("layer_swa", LAYER_SWA, kv_len=2048),
    "ctx1024": Workload("ctx1024", FULL, prompt_len=512, steps=512),
    "ctx4096": Workload("ctx4096", FULL, prompt_len=3584, steps=512),
    "lane": Workload("lane", LANE, kv_len=4095),
}
