"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/lfdecode.h declares, and rejects invalid arguments before any
HIP call. No compute runs here."""
import ctypes
import os
import re

import pytest

from decode_step_05_amd import lfdecode as C
from synth import FULL, LANE, LAYER_FULL, TINY

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "lfdecode.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lf_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = C.load()
    declared = header_functions()
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in lfdecode.h but not exported"
    assert sorted(C.EXPORTS) == declared


def test_sizes_of_the_workloads():
    # workspace = the weights once + the rotary table, activations and
    # attention exchange buffers (a few MB) + the batched step's buffers for
    # 8 sequences (activations, partial sums, attention split states: about
    # 20 MB); sequence buffer = caches + state
    for cfg in (TINY, LAYER_FULL, FULL, LANE):
        c = C.make_config(cfg)
        ws, kv = C.lf_workspace_bytes(c), C.lf_kv_bytes(c)
        assert ws > 0 and kv > 0, C.lf_last_error()
    c = C.make_config(FULL)
    cache = 2 * 15 * 4096 * 16 * 128 * 2
    assert cache <= C.lf_kv_bytes(c) < cache + 4096 * 4 + 32000 * 4 + 4096
    weights = 2338451456 * 2
    assert weights <= C.lf_workspace_bytes(c) < weights + 32 * 2 ** 20


@pytest.mark.parametrize("field,value,msg", [
    ("head_dim", 48, "head_dim"),
    ("n_kv_heads", 5, "multiple of n_kv_heads"),
    ("n_lanes", 3, "n_lanes"),
    ("max_ctx", 4097, "max_ctx"),
    ("max_ctx", 0, "max_ctx"),
    ("d_model", 260, "d_model"),
    ("ffn", 0, "ffn"),
    ("n_layers", 0, "n_layers"),
    ("vocab", -1, "vocab"),
])
def test_invalid_configs_rejected(field, value, msg):
    c = C.make_config(TINY)
    setattr(c, field, value)
    assert C.lf_workspace_bytes(c) == 0
    assert msg in C.lf_last_error()
    assert C.lf_kv_bytes(c) == 0


def test_group_and_lane_limits():
    c = C.make_config(FULL)
    c.n_kv_heads = 4          # 8 query heads per kv head
    c.n_lanes = 4
    assert C.lf_workspace_bytes(c) == 0 and "query heads per kv head" in C.lf_last_error()
    c = C.make_config(FULL)
    c.n_lanes = 1             # 16 kv heads in one lane: more than 512/128 = 4
    assert C.lf_workspace_bytes(c) == 0 and "kv heads per lane" in C.lf_last_error()
    c = C.make_config(TINY)
    c.window[0] = -3
    assert C.lf_workspace_bytes(c) == 0 and "window" in C.lf_last_error()


def test_init_argument_errors_before_any_device_call():
    lib = C.load()
    c = C.make_config(TINY)
    out = ctypes.c_void_p()
    w = C.lf_weight_ptrs()
    # null weights / workspace
    assert lib.lf_model_init(ctypes.byref(c), None, None, 0, None, ctypes.byref(out)) == C.LF_EINVAL
    # misaligned workspace
    rc = lib.lf_model_init(ctypes.byref(c), ctypes.byref(w), 0x1001, 1 << 30, None, ctypes.byref(out))
    assert rc == C.LF_EINVAL and "aligned" in C.lf_last_error()
    # undersized workspace
    rc = lib.lf_model_init(ctypes.byref(c), ctypes.byref(w), 0x10000, 16, None, ctypes.byref(out))
    assert rc == C.LF_EINVAL and "workspace" in C.lf_last_error()
    # null per-layer arrays
    rc = lib.lf_model_init(ctypes.byref(c), ctypes.byref(w), 0x10000, 1 << 40, None, ctypes.byref(out))
    assert rc == C.LF_EINVAL and "per-layer" in C.lf_last_error()
    assert out.value is None


def test_null_handles_rejected():
    lib = C.load()
    assert lib.lf_prefill(None, None, None, 1, None) == C.LF_EINVAL
    assert lib.lf_decode_step(None, None, None, None) == C.LF_EINVAL
    assert lib.lf_decode_step_hidden(None, None, None, None, None) == C.LF_EINVAL
    assert lib.lf_logits(None, None, None, None, None) == C.LF_EINVAL
    assert lib.lf_kv_set_len(None, 0, None) == C.LF_EINVAL
    assert lib.lf_kv_alloc(None, None, 0, ctypes.byref(ctypes.c_void_p())) == C.LF_EINVAL
    assert lib.lf_kv_len(None) == -1
    lib.lf_model_free(None)
    lib.lf_kv_free(None)
    assert lib.lf_model_set_fused(None, 1) == C.LF_EINVAL
    assert lib.lf_model_fused(None) == -1
    assert lib.lf_model_raise_give_up(None, None) == C.LF_EINVAL


def test_read_bandwidth_argument_errors_before_any_device_call():
    lib = C.load()
    g = ctypes.c_float()
    assert lib.lf_read_bandwidth(None, 1 << 20, 1, 0x1000, ctypes.byref(g), None) == C.LF_EINVAL
    assert lib.lf_read_bandwidth(0x1000, 1 << 20, 1, None, ctypes.byref(g), None) == C.LF_EINVAL
    rc = lib.lf_read_bandwidth(0x1008, 1 << 20, 1, 0x1000, ctypes.byref(g), None)
    assert rc == C.LF_EINVAL and "aligned" in C.lf_last_error()
    assert lib.lf_read_bandwidth(0x1000, 8, 1, 0x1000, ctypes.byref(g), None) == C.LF_EINVAL
    assert lib.lf_read_bandwidth(0x1000, 1 << 20, 0, 0x1000, ctypes.byref(g), None) == C.LF_EINVAL


def test_prefill_workspace_sizes_and_null_checks():
    # chunk rows of fp32: the residual, the widest projection output (gate/up,
    # 2 x 7168), the widest GEMM input (the SwiGLU output, 7168) and the
    # queries (4096); each region 256-byte aligned
    lib = C.load()
    c = C.make_config(FULL)
    for mc in (1, 100, 1024, 4096):
        exact = mc * (4096 * 4 + 14336 * 4 + 7168 * 4 + 4096 * 4)
        assert exact <= C.lf_prefill_workspace_bytes(c, mc) < exact + 4 * 256
    assert C.lf_prefill_workspace_bytes(c, 0) == 0
    assert C.lf_prefill_workspace_bytes(c, 4097) == 0
    assert lib.lf_prefill_workspace_bytes(None, 16) == 0
    assert C.lf_prefill_workspace_bytes(C.make_config(TINY), 64) > 0
    assert lib.lf_prefill_batched(None, None, None, 1, 16, None, 0, None) == C.LF_EINVAL
    assert lib.lf_prefill_batched(None, None, 0x1000, 1, 16, 0x1000, 1 << 20, None) == C.LF_EINVAL


def test_sample_argument_errors_before_any_device_call():
    lib = C.load()
    assert lib.lf_sample(None, 1, 10, 1.0, 0x1000, 0x1000, None) == C.LF_EINVAL
    assert lib.lf_sample(0x1000, 1, 10, 1.0, None, 0x1000, None) == C.LF_EINVAL
    assert lib.lf_sample(0x1000, 1, 10, 1.0, 0x1000, None, None) == C.LF_EINVAL
    assert lib.lf_sample(0x1000, 0, 10, 1.0, 0x1000, 0x1000, None) == C.LF_EINVAL
    assert lib.lf_sample(0x1000, 1, 0, 1.0, 0x1000, 0x1000, None) == C.LF_EINVAL
    assert lib.lf_sample(0x1000, 1, (1 << 24) + 1, 1.0, 0x1000, 0x1000, None) == C.LF_EINVAL
    # 1e-45 is a subnormal fp32 whose reciprocal overflows to inf
    for t in (0.0, -1.0, float("nan"), float("inf"), 1e-45, -1e-45):
        rc = lib.lf_sample(0x1000, 1, 10, t, 0x1000, 0x1000, None)
        assert rc == C.LF_EINVAL and "temperature" in C.lf_last_error(), t


def test_attention_plan():
    """Layouts whose workgroups wait on each other are chosen only where the
    device holds all of those workgroups at once."""
    c = C.make_config(FULL)
    # MI355X: 256 CUs, one fused workgroup per CU (its key copies fill most of
    # the LDS), several attention workgroups per CU, launches dealt to XCDs in turn
    fused, xcd = C.lf_plan_attention(c, 256, 8, 1, True)
    assert fused and xcd == [True] * 15
    # no room for the fused kernel's 256 workgroups at once, or too few CUs
    assert C.lf_plan_attention(c, 256, 8, 0, True)[0] is False
    assert C.lf_plan_attention(c, 128, 8, 1, True)[0] is False
    # workgroups not dealt to the XCDs in turn: neither the fused kernel nor the XCD layout
    fused, xcd = C.lf_plan_attention(c, 256, 8, 1, False)
    assert not fused and not any(xcd)
    # the XCD layout needs all S * n_kv = 16 * 16 attention workgroups at once
    assert C.lf_plan_attention(c, 32, 8, 1, True)[1] == [True] * 15
    assert C.lf_plan_attention(c, 31, 8, 1, True)[1] == [False] * 15
    # 256 kv heads of 32 dims: 16 splits each, 4096 workgroups; no room for
    # all of them, so each kv head's splits run as consecutive workgroups
    big = C.make_config(FULL)
    big.n_q_heads, big.n_kv_heads, big.head_dim, big.n_lanes = 256, 256, 32, 16
    fused, xcd = C.lf_plan_attention(big, 256, 8, 1, True)
    assert not fused and not any(xcd)
    # a layer whose 16 splits of one kv head cannot be resident together is rejected
    with pytest.raises(C.LfError, match="cannot be resident"):
        C.lf_plan_attention(c, 15, 1, 1, True)
    lib = C.load()
    one = ctypes.c_int32()
    layers = (ctypes.c_int32 * 15)()
    assert lib.lf_plan_attention(ctypes.byref(c), 0, 8, 1, 1, ctypes.byref(one), layers) == C.LF_EINVAL
    assert lib.lf_plan_attention(ctypes.byref(c), 256, 8, 1, 1, None, layers) == C.LF_EINVAL


def test_batch_step_argument_errors_before_any_device_call():
    lib = C.load()
    arr = (ctypes.c_void_p * 9)()
    assert lib.lf_decode_step_batch(None, arr, 1, None, None) == C.LF_EINVAL
    assert lib.lf_decode_step_batch(0x1000, None, 1, None, None) == C.LF_EINVAL
    assert C.LF_MAX_BATCH == 8
