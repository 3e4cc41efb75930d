"""Seeded synthetic inputs for the MoE decode path (host side).

This module only draws random inputs; it holds none of the method's arithmetic (no quantizer, no
routing, no GEMV).  Both the CPU oracle and the GPU path take their inputs from here, and the large
expert tensors are drawn on the device by ``synth_gen.hip`` from the *same* definition, so the two
sides see bit-identical fp32 weights without copying a single byte between them.

Generator definition (counter-based, so any element can be drawn on its own):

* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014):
  ``mix(z) = z3`` with ``z1 = (z ^ z>>30) * 0xBF58476D1CE4E5B9``, ``z2 = (z1 ^ z1>>27) * 0x94D049BB133111EB``,
  ``z3 = z2 ^ z2>>31`` (all mod 2^64).  Output ``i`` (i >= 0) of the stream with seed ``s`` is
  ``mix(s + (i+1) * 0x9E3779B97F4A7C15)``.
* Stream seed: ``mix(pack(cfg, layer, tag, index) + 0x9E3779B97F4A7C15)`` with
  ``pack = cfg<<32 | layer<<24 | tag<<16 | index`` (index < 65536).
* Normal number ``i`` of a stream: the Irwin-Hall sum of twelve 16-bit uniforms, i.e. the sixteen-bit
  fields of outputs 3i, 3i+1, 3i+2, ``S = sum(fields)``; ``z = S - 393210`` is an integer with mean 0
  and standard deviation ~65536, and the fp32 sample is ``float32(z) * float32(sigma * 2**-16)``.  Every
  step is exact integer arithmetic or a single IEEE fp32 product, so host and device agree bit for bit.
  The Irwin-Hall(12) law is the classical CLT stand-in for N(0, 1) (tails cut at 6 sigma).

The pages describe one workload (Gemma 4 26B-A4B decode on user prompts, MacBook Air M2 and M5 Pro
measurements); no public dataset or trained checkpoint is available here, so these seeded tensors of
the configured shapes stand in for it.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
IH_MEAN = 393210          # 12 * 32767.5
SIGMA_WEIGHTS = 0.02      # N(0, 0.02) expert, shared and router weights

# stream tags
TAG_ROUTER = 0
TAG_ROUTER_SCALE = 1
TAG_GATE_UP = 2
TAG_DOWN = 3
TAG_SHARED_GATE_UP = 4
TAG_SHARED_DOWN = 5
TAG_X = 6
TAG_GAMMA = 7


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def mix64(z: int) -> int:
    """SplitMix64 output function on one python int (mod 2^64)."""
    with np.errstate(over="ignore"):
        return int(_mix(np.array([z & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))[0])


def stream_seed(cfg: int, layer: int, tag: int, index: int = 0) -> int:
    assert 0 <= cfg < 256 and 0 <= layer < 256 and 0 <= tag < 256 and 0 <= index < 65536
    packed = (cfg << 32) | (layer << 24) | (tag << 16) | index
    return mix64(packed + int(GOLDEN_GAMMA))


def draws(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the SplitMix64 stream with the given seed (uint64)."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        return _mix(np.uint64(seed) + i * GOLDEN_GAMMA)


_HOST_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth_host.so")
_host = None


def _host_lib():
    """The C twin of this generator (synth_host.c, built by the package's build step), or None."""
    global _host
    if _host is None and os.path.exists(_HOST_LIB):
        lib = ctypes.CDLL(_HOST_LIB)
        lib.synth_host_normals_f32.restype = None
        lib.synth_host_normals_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float,
                                               ctypes.c_void_p, ctypes.c_int]
        _host = lib
    return _host


def normals_f32(seed: int, start: int, count: int, sigma: float = 1.0, chunk: int = 1 << 21,
                threads: int = 0) -> np.ndarray:
    """Irwin-Hall(12) normals number start .. start+count-1 of a stream, as fp32 (bit-exact spec).

    Drawn by the C twin (``synth_host.c``, same definition, ``threads`` OpenMP threads, 0 = all) when it
    is built, else by ``normals_f32_numpy``; the two agree bit for bit."""
    lib = _host_lib()
    if lib is None or count == 0:
        return normals_f32_numpy(seed, start, count, sigma, chunk)
    out = np.empty(count, dtype=np.float32)
    lib.synth_host_normals_f32(seed, start, count, sigma, out.ctypes.data, threads)
    return out


def normals_f32_numpy(seed: int, start: int, count: int, sigma: float = 1.0, chunk: int = 1 << 21) -> np.ndarray:
    """The generator's definition in numpy (see normals_f32)."""
    out = np.empty(count, dtype=np.float32)
    scale = np.float32(np.float32(sigma) * np.float32(2.0 ** -16))
    mask = np.uint64(0xFFFF)
    for c0 in range(0, count, chunk):
        n = min(chunk, count - c0)
        r = draws(seed, 3 * (start + c0), 3 * n)
        s = np.zeros(3 * n, dtype=np.int64)
        for f in range(4):
            s += ((r >> np.uint64(16 * f)) & mask).astype(np.int64)
        z = s.reshape(n, 3).sum(axis=1) - IH_MEAN
        out[c0:c0 + n] = z.astype(np.float32) * scale
    return out


def integer_normals(seed: int, start: int, count: int) -> np.ndarray:
    """The integer z = S - 393210 behind normals_f32 (int64)."""
    r = draws(seed, 3 * start, 3 * count)
    s = np.zeros(3 * count, dtype=np.int64)
    for f in range(4):
        s += ((r >> np.uint64(16 * f)) & np.uint64(0xFFFF)).astype(np.int64)
    return s.reshape(count, 3).sum(axis=1) - IH_MEAN


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even), returned as uint16 bit patterns (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return b.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------------------------

def weight_f32(cfg: int, layer: int, tag: int, index: int, rows: int, cols: int,
               sigma: float = SIGMA_WEIGHTS, threads: int = 0) -> np.ndarray:
    """fp32 [rows][cols] N(0, sigma) weights of one expert matrix (row-major draw order)."""
    return normals_f32(stream_seed(cfg, layer, tag, index), 0, rows * cols, sigma, threads=threads).reshape(rows, cols)


def router_int8(cfg: int, layer: int, n_experts: int, d: int):
    """8-bit router: int8 [E][d] and fp32 per-row scale [E].

    The int8 entry is the integer normal z shifted right by 11 (std ~32) and clamped to [-127, 127];
    the row scale is 0.02/32 * (0.75 + 0.5*u), u uniform in [0, 1) from the top 24 bits of one draw,
    so s_e * W[e] has the N(0, 0.02) spread of the other weights and rows differ in scale.
    """
    z = integer_normals(stream_seed(cfg, layer, TAG_ROUTER), 0, n_experts * d)
    w = np.clip(z >> 11, -127, 127).astype(np.int8).reshape(n_experts, d)
    u = (draws(stream_seed(cfg, layer, TAG_ROUTER_SCALE), 0, n_experts) >> np.uint64(40)).astype(np.float32)
    u = u * np.float32(2.0 ** -24)
    s = (np.float32(0.75) + np.float32(0.5) * u) * np.float32(np.float32(0.02) / np.float32(32.0))
    return w, s.astype(np.float32)


def activation(cfg: int, token: int, d: int, bf16: bool = True) -> np.ndarray:
    """x ~ N(0, 1) for one token: bf16 bit patterns (uint16 [d]) or fp32 [d]."""
    assert token < 65536
    x = normals_f32(stream_seed(cfg, 0, TAG_X, token), 0, d, 1.0)
    return f32_to_bf16_bits(x) if bf16 else x


def rms_gamma(cfg: int, layer: int, d: int, ones: bool = True) -> np.ndarray:
    """RMSNorm gain: ones (no trained weights), or 1 + N(0, 0.02) for tests of the gain input."""
    if ones:
        return np.ones(d, dtype=np.float32)
    g = normals_f32(stream_seed(cfg, layer, TAG_GAMMA), 0, d, 0.02)
    return (np.float32(1.0) + g).astype(np.float32)


def zipf_trace(seed: int, n_tokens: int, n_layers: int, k: int, n_experts: int, s: float = 1.1) -> np.ndarray:
    """Forced routing trace int32 [T][L][k]: per (token, layer) draw Zipf(s) ranks over 1..E until k
    distinct ranks are seen; draw order is rank order; expert id = rank - 1."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 6]))
    r = np.arange(1, n_experts + 1, dtype=np.float64)
    pmf = r ** (-s)
    cdf = np.cumsum(pmf / pmf.sum())
    cdf[-1] = 1.0
    out = np.empty((n_tokens, n_layers, k), dtype=np.int32)
    for t in range(n_tokens):
        for l in range(n_layers):
            picked: list[int] = []
            while len(picked) < k:
                for e in np.searchsorted(cdf, rng.random(4 * k), side="right"):
                    e = int(min(e, n_experts - 1))
                    if e not in picked:
                        picked.append(e)
                        if len(picked) == k:
                            break
            out[t, l] = picked
    return out


def zipf_pmf(n_experts: int, s: float = 1.1) -> np.ndarray:
    r = np.arange(1, n_experts + 1, dtype=np.float64)
    p = r ** (-s)
    return p / p.sum()


# ----------------------------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    weight_cfg: int      # seed id of the weights (shared by configs that reuse a layer or stack)
    act_cfg: int         # seed id of the activations
    d: int               # hidden size
    n_experts: int
    k: int
    F: int               # routed expert FFN width
    S: int               # shared expert FFN width
    sb_bf16: bool        # scale/bias dtype: bf16 (True) or fp32
    x_bf16: bool         # activation dtype
    n_layers: int = 1
    n_tokens: int = 1
    n_slots: int = 0     # expert cache slots per layer (0 = all resident)
    rms_norm: bool = False
    group: int = 64


TINY = MoEConfig("tiny layer, d=256 E=8 k=2 F=128 S=128, fp32 scale/bias, fp32 x",
                 weight_cfg=0, act_cfg=0, d=256, n_experts=8, k=2, F=128, S=128, sb_bf16=False, x_bf16=False)
LAYER = MoEConfig("one MoE layer decode, d=2816 E=128 k=8 F=704 S=2816, bf16",
                  weight_cfg=1, act_cfg=1, d=2816, n_experts=128, k=8, F=704, S=2816, sb_bf16=True, x_bf16=True)
STACK = dataclasses.replace(LAYER, name="30-layer MoE stack decode, 256 steps, RMSNorm + residual",
                            weight_cfg=2, act_cfg=2, n_layers=30, n_tokens=256, rms_norm=True)
BATCHED = dataclasses.replace(LAYER, name="batched decode, 32 tokens through one d=2816 layer",
                              act_cfg=3, n_tokens=32)
STREAMED = dataclasses.replace(STACK, name="expert-cache streaming, 30 layers, 16 LFU slots, Zipf(1.1) x 512",
                               act_cfg=4, n_tokens=512, n_slots=16)
CONFIGS = {"tiny": TINY, "layer": LAYER, "stack": STACK, "batched": BATCHED, "streamed": STREAMED}
