"""CPU oracle (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package. The HIP library never calls it and shares no code with it.
"""
from .decoder import (OracleDecoder, rmsnorm, apply_rope, rope_angles, silu, attend, softmax,
                      kv_head_of, visible_range, greedy)
from .sampling import sample_probs, sample_token, interval_of

__all__ = ["OracleDecoder", "rmsnorm", "apply_rope", "rope_angles", "silu", "attend", "softmax",
           "kv_head_of", "visible_range", "greedy", "sample_probs", "sample_token", "interval_of"]
