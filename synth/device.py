"""Device draws of the seeded generator (same definition as ``synth.normals_f32``), via libsynth.so."""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (map torch's HIP runtime before libsynth.so, so the process has only one)

from . import SIGMA_WEIGHTS, stream_seed

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise ImportError(f"{_PATH} is not built; run `python -m bit_quantized_expert_int8_amd.build`")
        _lib = ctypes.CDLL(_PATH)
        _lib.synth_normals_f32.restype = ctypes.c_int
        _lib.synth_normals_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float,
                                           ctypes.c_void_p, ctypes.c_void_p]
    return _lib


def normals_into(out, seed: int, start: int = 0, sigma: float = 1.0, stream=None) -> None:
    """Fill a contiguous float32 CUDA tensor with normals start .. start+numel-1 of the stream."""
    assert out.is_cuda and out.is_contiguous() and str(out.dtype) == "torch.float32"
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    rc = _load().synth_normals_f32(seed, start, out.numel(), sigma, out.data_ptr(), s)
    if rc != 0:
        raise RuntimeError(f"synth_normals_f32 failed: hip error {rc}")


def weight_into(out, cfg: int, layer: int, tag: int, index: int, sigma: float = SIGMA_WEIGHTS, stream=None) -> None:
    """Device twin of ``synth.weight_f32``: the same fp32 values, drawn in place."""
    normals_into(out, stream_seed(cfg, layer, tag, index), 0, sigma, stream)
