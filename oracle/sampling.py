"""CPU oracle for temperature sampling of the next token (test infrastructure
only; the HIP library shares no code with it).

The asector.ru summary ("Performance and infrastructure") proposes stochastic
decoding, scored as pass@N, to raise accuracy on code: several sampled
continuations of one prompt, affordable because one pass is fast. The pages
name neither the sampler nor its random numbers. The plainest
reading, taken here: the next token is drawn from softmax(z / T) by inverting
its cumulative distribution at a uniform number u in [0, 1) that the caller
supplies, so that no random generator has to match between implementations.

Token i covers the half-open interval [c_{i-1}, c_i) of u, where c_i is the sum
of the probabilities of tokens 0..i (c_{-1} = 0): the answer is the smallest i
with c_i > u. Tokens of probability 0 cover an empty interval and are never
drawn; if rounding leaves the total below u, the last token of positive
probability is drawn. Arithmetic in float64.
"""
from __future__ import annotations

import numpy as np


def sample_probs(z, temperature: float) -> np.ndarray:
    """softmax(z / T) in float64, T > 0."""
    if not temperature > 0:
        raise ValueError("temperature must be positive")
    z = np.asarray(z, dtype=np.float64)
    w = np.exp((z - z.max()) / temperature)
    return w / w.sum()


def sample_token(z, temperature: float, u: float) -> int:
    """The token whose cumulative-probability interval holds u."""
    if not 0.0 <= u < 1.0:
        raise ValueError("u must lie in [0, 1)")
    p = sample_probs(z, temperature)
    c = np.cumsum(p)
    hit = np.nonzero(c > u)[0]
    if hit.size:
        return int(hit[0])
    return int(np.nonzero(p > 0)[0][-1])


def interval_of(z, temperature: float, token: int):
    """(c_{token-1}, c_token): the interval of u that draws `token`."""
    c = np.cumsum(sample_probs(z, temperature))
    lo = float(c[token - 1]) if token > 0 else 0.0
    return lo, float(c[token])
