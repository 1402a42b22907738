"""Python binding of liblfdecode.so (include/lfdecode.h).

Argument marshalling only: every function here forwards to the C entry point
of the same name; all device work runs in the HIP library. PyTorch provides
device memory (tensors) and streams. There is no fallback: if the library is
missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblfdecode.so")
MAX_LAYERS = 64

LF_OK, LF_EINVAL, LF_ERANGE, LF_EHIP = 0, -1, -2, -3
LF_STATIC_SCRATCH_BYTES = 32 << 20
LF_MAX_BATCH = 8
LF_MODE_EAGER, LF_MODE_GRAPH = 0, 1

# Every symbol include/lfdecode.h declares.
EXPORTS = (
    "lf_workspace_bytes", "lf_kv_bytes", "lf_model_init", "lf_model_free", "lf_model_set_graph",
    "lf_model_set_mode", "lf_model_mode", "lf_model_set_fused", "lf_model_fused", "lf_model_raise_give_up",
    "lf_plan_attention",
    "lf_kv_alloc", "lf_kv_free", "lf_kv_cache_ptrs", "lf_kv_set_len", "lf_kv_len", "lf_kv_tokens", "lf_prefill",
    "lf_prefill_workspace_bytes", "lf_prefill_batched", "lf_prefill_batched_static",
    "lf_decode_step", "lf_decode_steps", "lf_decode_step_batch", "lf_decode_step_hidden", "lf_logits", "lf_kv_status",
    "lf_step_kernel_times", "lf_kernel_time", "lf_read_bandwidth", "lf_sample", "lf_last_error",
)

KERNEL_KINDS = ("qkv", "attn", "o", "gate_up", "down", "lm_head", "qkv_attn")


class lf_config(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn",
                                        "vocab", "n_lanes", "max_ctx")] + [
        ("window", c_int32 * MAX_LAYERS), ("rope_theta", c_float), ("rms_eps", c_float)]


class lf_weight_ptrs(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("lm_head", c_void_p), ("final_norm", c_void_p),
                ("attn_norm", POINTER(c_void_p)), ("wqkv", POINTER(c_void_p)), ("wo", POINTER(c_void_p)),
                ("ffn_norm", POINTER(c_void_p)), ("wgate_up", POINTER(c_void_p)), ("wdown", POINTER(c_void_p))]


class LfError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"lfdecode error {code}: {msg}")
        self.code = code


_lib = None


def load():
    """Load the library (once) and declare the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m decode_step_05_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    sig = {
        "lf_workspace_bytes": (c_size_t, [POINTER(lf_config)]),
        "lf_kv_bytes": (c_size_t, [POINTER(lf_config)]),
        "lf_model_init": (c_int, [POINTER(lf_config), POINTER(lf_weight_ptrs), P, c_size_t, P, POINTER(P)]),
        "lf_model_free": (None, [P]),
        "lf_model_set_graph": (c_int, [P, c_int]),
        "lf_model_set_mode": (c_int, [P, c_int]),
        "lf_model_mode": (c_int, [P]),
        "lf_model_set_fused": (c_int, [P, c_int]),
        "lf_model_fused": (c_int, [P]),
        "lf_model_raise_give_up": (c_int, [P, P]),
        "lf_plan_attention": (c_int, [POINTER(lf_config), c_int32, c_int32, c_int32, c_int32, POINTER(c_int32),
                                      POINTER(c_int32)]),
        "lf_kv_alloc": (c_int, [P, P, c_size_t, POINTER(P)]),
        "lf_kv_free": (None, [P]),
        "lf_kv_cache_ptrs": (c_int, [P, POINTER(P), POINTER(P)]),
        "lf_kv_set_len": (c_int, [P, c_int32, P]),
        "lf_kv_len": (c_int32, [P]),
        "lf_kv_tokens": (c_int, [P, P, c_int32, c_int32, P]),
        "lf_prefill": (c_int, [P, P, P, c_int32, P]),
        "lf_prefill_workspace_bytes": (c_size_t, [POINTER(lf_config), c_int32]),
        "lf_prefill_batched": (c_int, [P, P, P, c_int32, c_int32, P, c_size_t, P]),
        "lf_prefill_batched_static": (c_int, [P, P, P, c_int32, c_int32, P]),
        "lf_decode_step": (c_int, [P, P, P, P]),
        "lf_decode_steps": (c_int, [P, P, c_int32, P]),
        "lf_decode_step_batch": (c_int, [P, POINTER(P), c_int32, P, P]),
        "lf_decode_step_hidden": (c_int, [P, P, P, P, P]),
        "lf_logits": (c_int, [P, P, P, P, P]),
        "lf_kv_status": (c_int, [P, POINTER(c_int32), P]),
        "lf_step_kernel_times": (c_int, [P, P, P, P, P, POINTER(c_float), POINTER(c_int32), c_int32,
                                         POINTER(c_int32), P]),
        "lf_kernel_time": (c_int, [P, P, c_int32, c_int32, c_int32, c_int32, P, P, POINTER(c_float), P]),
        "lf_read_bandwidth": (c_int, [P, c_size_t, c_int32, P, POINTER(c_float), P]),
        "lf_sample": (c_int, [P, c_int32, c_int32, c_float, P, P, P]),
        "lf_last_error": (c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(rc):
    if rc != LF_OK:
        raise LfError(rc, load().lf_last_error().decode())
    return rc


def _ptr(t):
    """Device address of a tensor (or None / an int passed through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(cfg) -> lf_config:
    """lf_config from any object with the decoder-shape attributes (or a dict)."""
    g = cfg.get if isinstance(cfg, dict) else (lambda k: getattr(cfg, k))
    c = lf_config()
    for n in ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "n_lanes", "max_ctx"):
        setattr(c, n, int(g(n)))
    w = list(g("windows"))
    if len(w) != c.n_layers or len(w) > MAX_LAYERS:
        raise ValueError("windows must list one entry per layer")
    for i, v in enumerate(w):
        c.window[i] = int(v)
    c.rope_theta = float(g("rope_theta"))
    c.rms_eps = float(g("rms_eps"))
    return c


# ------------------------------------------------------------ C entry points

def lf_last_error() -> str:
    return load().lf_last_error().decode()


def lf_workspace_bytes(cfg: lf_config) -> int:
    return load().lf_workspace_bytes(ctypes.byref(cfg))


def lf_kv_bytes(cfg: lf_config) -> int:
    return load().lf_kv_bytes(ctypes.byref(cfg))


def lf_model_init(cfg: lf_config, weights: dict, workspace, stream=None):
    """weights: name -> fp16 device tensor, names as 'embed', 'lm_head',
    'final_norm', 'layers.{l}.attn_norm|wqkv|wo|ffn_norm|wgate_up|wdown'."""
    n = cfg.n_layers
    arrays = {}
    for key in ("attn_norm", "wqkv", "wo", "ffn_norm", "wgate_up", "wdown"):
        arr = (c_void_p * n)()
        for l in range(n):
            t = weights.get(f"layers.{l}.{key}")
            arr[l] = _ptr(t) if t is not None else None
        arrays[key] = arr
    w = lf_weight_ptrs()
    w.embed = _ptr(weights.get("embed"))
    w.lm_head = _ptr(weights.get("lm_head"))
    w.final_norm = _ptr(weights.get("final_norm"))
    for key, arr in arrays.items():
        setattr(w, key, ctypes.cast(arr, POINTER(c_void_p)))
    out = c_void_p()
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().lf_model_init(ctypes.byref(cfg), ctypes.byref(w), _ptr(workspace), nbytes, _stream(stream),
                                ctypes.byref(out)))
    return out.value


def lf_model_free(model) -> None:
    load().lf_model_free(model)


def lf_model_set_graph(model, enabled: bool) -> None:
    _check(load().lf_model_set_graph(model, int(bool(enabled))))


def lf_model_set_mode(model, mode: int) -> None:
    _check(load().lf_model_set_mode(model, int(mode)))


def lf_model_mode(model) -> int:
    return load().lf_model_mode(model)


def lf_model_set_fused(model, enabled: bool) -> None:
    _check(load().lf_model_set_fused(model, int(bool(enabled))))


def lf_model_fused(model) -> bool:
    return load().lf_model_fused(model) == 1


def lf_model_raise_give_up(model, stream=None) -> None:
    _check(load().lf_model_raise_give_up(model, _stream(stream)))


def lf_plan_attention(cfg: lf_config, n_cu: int, attn_wg_per_cu: int, fused_wg_per_cu: int, xcd_classes: bool):
    """(fused, [xcd layout per layer]) that lf_model_init would choose (host only)."""
    fused = c_int32()
    layers = (c_int32 * cfg.n_layers)()
    _check(load().lf_plan_attention(ctypes.byref(cfg), int(n_cu), int(attn_wg_per_cu), int(fused_wg_per_cu),
                                    int(bool(xcd_classes)), ctypes.byref(fused), layers))
    return bool(fused.value), [bool(v) for v in layers]


def lf_kv_alloc(model, buf):
    out = c_void_p()
    _check(load().lf_kv_alloc(model, _ptr(buf), buf.numel() * buf.element_size(), ctypes.byref(out)))
    return out.value


def lf_kv_free(kv) -> None:
    load().lf_kv_free(kv)


def lf_kv_cache_ptrs(kv):
    k, v = c_void_p(), c_void_p()
    _check(load().lf_kv_cache_ptrs(kv, ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


def lf_kv_set_len(kv, length: int, stream=None) -> None:
    _check(load().lf_kv_set_len(kv, int(length), _stream(stream)))


def lf_kv_len(kv) -> int:
    return load().lf_kv_len(kv)


def lf_kv_tokens(kv, out, start: int, n: int, stream=None) -> None:
    _check(load().lf_kv_tokens(kv, _ptr(out), int(start), int(n), _stream(stream)))


def lf_prefill(model, kv, tokens, n=None, stream=None) -> None:
    n = tokens.numel() if n is None else n
    _check(load().lf_prefill(model, kv, _ptr(tokens), int(n), _stream(stream)))


def lf_prefill_workspace_bytes(cfg: lf_config, chunk: int) -> int:
    return load().lf_prefill_workspace_bytes(ctypes.byref(cfg), int(chunk))


def lf_prefill_batched(model, kv, tokens, chunk: int, workspace, n=None, stream=None) -> None:
    n = tokens.numel() if n is None else n
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().lf_prefill_batched(model, kv, _ptr(tokens), int(n), int(chunk), _ptr(workspace), nbytes,
                                     _stream(stream)))


def lf_prefill_batched_static(model, kv, tokens, chunk: int = 0, n=None, stream=None) -> None:
    n = tokens.numel() if n is None else n
    _check(load().lf_prefill_batched_static(model, kv, _ptr(tokens), int(n), int(chunk), _stream(stream)))


def lf_decode_step(model, kv, token=None, stream=None) -> None:
    _check(load().lf_decode_step(model, kv, _ptr(token), _stream(stream)))


def lf_decode_steps(model, kv, n: int, stream=None) -> None:
    _check(load().lf_decode_steps(model, kv, int(n), _stream(stream)))


def lf_decode_step_batch(model, kvs, tokens=None, stream=None) -> None:
    """One step of each sequence handle in kvs (a list); tokens: device int32 [len(kvs)] or None."""
    arr = (c_void_p * len(kvs))(*kvs)
    _check(load().lf_decode_step_batch(model, arr, len(kvs), _ptr(tokens), _stream(stream)))


def lf_decode_step_hidden(model, kv, x_in, x_out, stream=None) -> None:
    _check(load().lf_decode_step_hidden(model, kv, _ptr(x_in), _ptr(x_out), _stream(stream)))


def lf_logits(model, kv, logits, argmax=None, stream=None) -> None:
    _check(load().lf_logits(model, kv, _ptr(logits), _ptr(argmax), _stream(stream)))


def lf_sample(logits, temperature, u, tokens, stream=None) -> None:
    """Temperature draw per row: logits device fp32 [rows, n] (or [n]), u device
    fp32 [rows], tokens device int32 [rows] (written)."""
    rows = int(u.numel())
    n = int(logits.shape[-1])
    if logits.numel() != rows * n or tokens.numel() != rows:
        raise ValueError("logits must be [rows, n], u and tokens [rows]")
    _check(load().lf_sample(_ptr(logits), rows, n, float(temperature), _ptr(u), _ptr(tokens), _stream(stream)))


def lf_kv_status(kv, stream=None):
    out = (c_int32 * 3)()
    _check(load().lf_kv_status(kv, out, _stream(stream)))
    return int(out[0]), int(out[1]), int(out[2])


def lf_step_kernel_times(model, kv, token=None, x_in=None, x_out=None, cap=512, stream=None):
    """[(kind name, milliseconds)] of one step's kernels in launch order."""
    ms = (c_float * cap)()
    kinds = (c_int32 * cap)()
    n = c_int32()
    _check(load().lf_step_kernel_times(model, kv, _ptr(token), _ptr(x_in), _ptr(x_out), ms, kinds, cap,
                                       ctypes.byref(n), _stream(stream)))
    return [(KERNEL_KINDS[kinds[i]], float(ms[i])) for i in range(n.value)]


def lf_kernel_time(model, kv, kind, layer, reps=16, iters=8, x_in=None, x_out=None, stream=None):
    """Milliseconds per launch of one per-phase kernel (kind name or LF_KERNEL_*) of
    layer `layer`, launched back to back in a graph."""
    k = KERNEL_KINDS.index(kind) if isinstance(kind, str) else int(kind)
    ms = c_float()
    _check(load().lf_kernel_time(model, kv, k, layer, reps, iters, _ptr(x_in), _ptr(x_out), ctypes.byref(ms),
                                 _stream(stream)))
    return float(ms.value)


def lf_read_bandwidth(buf, iters=10, stream=None) -> float:
    """GB/s of a plain streaming read of the device tensor `buf` (see the header)."""
    import torch
    sink = torch.empty(1, dtype=torch.int32, device=buf.device)
    gbs = c_float()
    _check(load().lf_read_bandwidth(_ptr(buf), buf.numel() * buf.element_size(), iters, _ptr(sink),
                                    ctypes.byref(gbs), _stream(stream)))
    return float(gbs.value)
