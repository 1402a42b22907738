"""Batch-1 decode step of a Laneformer-2B-shaped decoder on MI355X (gfx950).

The compute lives in liblfdecode.so (HIP kernels behind the C ABI of
include/lfdecode.h); `lfdecode` is its ctypes binding and `runtime` wraps the
handles with torch-owned device buffers.
"""
from . import lfdecode
from .runtime import Decoder, Sequence

__all__ = ["lfdecode", "Decoder", "Sequence"]
