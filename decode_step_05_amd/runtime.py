"""Torch-owned buffers around the C handles: a Decoder (weights + workspace)
and its Sequences (one KV/state buffer each). All compute is in the library."""
from __future__ import annotations

import numpy as np

from . import lfdecode as C


def _torch():
    import torch
    return torch


class Decoder:
    """Uploads fp16 weights (NumPy arrays or device tensors), allocates the
    workspace with torch and calls lf_model_init. The library copies what it
    needs, so the uploaded weights are released afterwards."""

    def __init__(self, cfg, weights: dict, device="cuda", stream=None, graph=True, mode=None):
        torch = _torch()
        self.cfg = cfg
        self.c = C.make_config(cfg)
        self.device = torch.device(device)
        nbytes = C.lf_workspace_bytes(self.c)
        if nbytes == 0:
            # the library reports why through lf_last_error
            raise C.LfError(C.LF_EINVAL, C.lf_last_error())
        dev_w = {}
        for k, v in weights.items():
            t = torch.from_numpy(np.ascontiguousarray(v)) if isinstance(v, np.ndarray) else v
            dev_w[k] = t.to(device=self.device, dtype=torch.float16).contiguous()
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.handle = C.lf_model_init(self.c, dev_w, self.ws, stream)
        del dev_w
        if not graph:
            C.lf_model_set_graph(self.handle, False)
        if mode is not None:
            C.lf_model_set_mode(self.handle, mode)

    @property
    def mode(self) -> int:
        return C.lf_model_mode(self.handle)

    def set_mode(self, mode: int):
        C.lf_model_set_mode(self.handle, mode)

    def set_graph(self, enabled: bool):
        C.lf_model_set_graph(self.handle, enabled)

    @property
    def fused(self) -> bool:
        """Whether each layer's QKV projection and attention run as one kernel."""
        return C.lf_model_fused(self.handle)

    def set_fused(self, enabled: bool):
        C.lf_model_set_fused(self.handle, enabled)

    def sequence(self) -> "Sequence":
        return Sequence(self)

    def step_batch(self, seqs, tokens=None, stream=None):
        """One decode step of each sequence in seqs (lf_decode_step_batch);
        tokens: None (each its own greedy token), a list of ints, or a device
        int32 tensor [len(seqs)]."""
        torch = _torch()
        if tokens is not None and not torch.is_tensor(tokens):
            tokens = torch.tensor([int(t) for t in tokens], dtype=torch.int32, device=self.device)
        C.lf_decode_step_batch(self.handle, [q.handle for q in seqs], tokens, stream)

    def close(self):
        if getattr(self, "handle", None):
            C.lf_model_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Sequence:
    """One sequence: its device buffer holds the state, token history, last
    logits and the K/V caches (lane-major [layer][lane][pos][kv_in_lane][hd])."""

    def __init__(self, dec: Decoder):
        torch = _torch()
        self.dec = dec
        c = dec.c
        self.buf = torch.empty(C.lf_kv_bytes(c), dtype=torch.uint8, device=dec.device)
        self.handle = C.lf_kv_alloc(dec.handle, self.buf)
        kp, vp = C.lf_kv_cache_ptrs(self.handle)
        kpl = c.n_kv_heads // c.n_lanes
        shape = (c.n_layers, c.n_lanes, c.max_ctx, kpl, c.head_dim)
        n = int(np.prod(shape)) * 2
        base = self.buf.data_ptr()
        self.K = self.buf[kp - base: kp - base + n].view(torch.float16).view(shape)
        self.V = self.buf[vp - base: vp - base + n].view(torch.float16).view(shape)

    # -- cache content supplied by the caller (synthetic caches)
    def load_cache(self, K, V, stream=None):
        """K, V: fp16 [layer, n, kv_head, hd] (keys already rotated); sets len = n."""
        torch = _torch()
        c = self.dec.c
        kpl = c.n_kv_heads // c.n_lanes
        for dst, src in ((self.K, K), (self.V, V)):
            t = torch.as_tensor(np.ascontiguousarray(src)) if isinstance(src, np.ndarray) else src
            L, n = t.shape[0], t.shape[1]
            t = t.to(self.dec.device, torch.float16).view(L, n, c.n_lanes, kpl, c.head_dim).permute(0, 2, 1, 3, 4)
            dst[:, :, :n].copy_(t)
        C.lf_kv_set_len(self.handle, K.shape[1], stream)

    def set_len(self, n, stream=None):
        C.lf_kv_set_len(self.handle, n, stream)

    @property
    def len(self) -> int:
        return C.lf_kv_len(self.handle)

    def prefill(self, tokens, stream=None):
        torch = _torch()
        t = torch.as_tensor(np.asarray(tokens, dtype=np.int32)).to(self.dec.device) if not torch.is_tensor(tokens) else tokens
        C.lf_prefill(self.dec.handle, self.handle, t.to(torch.int32).contiguous(), None, stream)

    def prefill_batched(self, tokens, chunk=1024, stream=None):
        """The prompt pass on the matrix cores, `chunk` positions at a time
        (lf_prefill_batched); its scratch is allocated here with torch and
        kept for later calls of the same or a smaller chunk."""
        torch = _torch()
        t = torch.as_tensor(np.asarray(tokens, dtype=np.int32)).to(self.dec.device) if not torch.is_tensor(tokens) else tokens
        t = t.to(self.dec.device, torch.int32).contiguous()
        chunk = max(1, min(int(chunk), t.numel()))
        need = C.lf_prefill_workspace_bytes(self.dec.c, chunk)
        if need == 0:
            raise ValueError(f"chunk {chunk} is not a valid prompt-pass chunk")
        ws = getattr(self, "_pf_ws", None)
        if ws is None or ws.numel() < need:
            ws = self._pf_ws = torch.empty(need, dtype=torch.uint8, device=self.dec.device)
        C.lf_prefill_batched(self.dec.handle, self.handle, t, chunk, ws, None, stream)

    def step(self, token=None, stream=None):
        """token: None (feed the previous greedy token), an int, or a device int32 tensor."""
        torch = _torch()
        if isinstance(token, (int, np.integer)):
            token = torch.tensor([int(token)], dtype=torch.int32, device=self.dec.device)
        C.lf_decode_step(self.dec.handle, self.handle, token, stream)

    def steps(self, n, stream=None):
        C.lf_decode_steps(self.dec.handle, self.handle, n, stream)

    def step_hidden(self, x_in, x_out, stream=None):
        C.lf_decode_step_hidden(self.dec.handle, self.handle, x_in, x_out, stream)

    def tokens(self, start, n, stream=None):
        """Token ids [start, start + n) of the history, as an int32 device tensor."""
        torch = _torch()
        out = torch.empty(n, dtype=torch.int32, device=self.dec.device)
        C.lf_kv_tokens(self.handle, out, start, n, stream)
        return out

    def logits(self, stream=None):
        torch = _torch()
        z = torch.empty(self.dec.c.vocab, dtype=torch.float32, device=self.dec.device)
        a = torch.empty(1, dtype=torch.int32, device=self.dec.device)
        C.lf_logits(self.dec.handle, self.handle, z, a, stream)
        return z, a

    def status(self, stream=None):
        return C.lf_kv_status(self.handle, stream)

    def close(self):
        if getattr(self, "handle", None):
            C.lf_kv_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
