"""The oracle for many tokens at full size: the expert FFN in plain C (``ffn_ref.c``), the rest from ``moe``.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
and parity legs may import or run this module; it shares no code with the HIP path.

``moe.py`` is the readable definition and is pinned against the pages and the mathematics.  At the full
stack size (30 layers, 128 experts of 2816 x 704, a shared expert of width 2816) it takes minutes per token,
so this module evaluates the same definition with its one heavy step, the expert FFN on 4-bit affine weights,
in C (quantizer decisions in fp32, everything else in float64, dot products in column order), and the
experts of a layer on a pool of threads.  The C routine is pinned against ``moe.quantize_affine_q4`` (bit for
bit) and ``moe.expert_ffn`` (to 1e-12) in ``tests/test_oracle.py``.

``layer_tokens`` is teacher-forced: each token enters the layer with the input it is given (for a stack, the
GPU's own bf16 input to that layer), and the routing it is given (the GPU's) selects the experts, while the
gate weights are the softmax of the oracle's own logits at those ids; routing decisions are checked
separately against the oracle's logits.
"""
from __future__ import annotations

import concurrent.futures
import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np

import synth
from . import inputs as oin
from . import moe

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liboracle_ffn.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise ImportError(f"{_PATH} is not built; run `python -m bit_quantized_expert_int8_amd.build`")
        lib = ctypes.CDLL(_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        lib.orc_quantize_q4.restype = None
        lib.orc_quantize_q4.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        lib.orc_expert_ffn.restype = i32
        lib.orc_expert_ffn.argtypes = [vp, vp, i32, i32, i32, i32, vp, i32, vp, vp]
        _lib = lib
    return _lib


def default_threads() -> int:
    """Worker threads: the host's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def quantize_q4(w: np.ndarray, sb_bf16: bool):
    """The C encoder: codes uint8 [N][K], scale and bias float32 [N][K/64] (same contract as
    moe.quantize_affine_q4)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, kdim = w.shape
    codes = np.empty((n, kdim), dtype=np.uint8)
    s = np.empty((n, kdim // moe.GROUP), dtype=np.float32)
    b = np.empty_like(s)
    _load().orc_quantize_q4(w.ctypes.data, n, kdim, int(sb_bf16), codes.ctypes.data, s.ctypes.data, b.ctypes.data)
    return codes, s, b


def expert_ffn_rows(w_gate_up: np.ndarray, w_down: np.ndarray, sb_bf16: bool, U: np.ndarray, act: int,
                    want_h: bool = False):
    """y[t] = expert_ffn(encode(w_gate_up, w_down), U[t]) for every row of U [n][d] (float64 [n][d]); with
    want_h also the hidden vectors h [n][F]."""
    w_gate_up = np.ascontiguousarray(w_gate_up, dtype=np.float32)
    w_down = np.ascontiguousarray(w_down, dtype=np.float32)
    U = np.ascontiguousarray(U, dtype=np.float64)
    twoF, d = w_gate_up.shape
    F = twoF // 2
    assert w_down.shape == (d, F) and U.ndim == 2 and U.shape[1] == d
    n = U.shape[0]
    y = np.empty((n, d), dtype=np.float64)
    h = np.empty((n, F), dtype=np.float64) if want_h else None
    rc = _load().orc_expert_ffn(w_gate_up.ctypes.data, w_down.ctypes.data, d, F, int(sb_bf16), int(act), U.ctypes.data,
                                n, y.ctypes.data, h.ctypes.data if want_h else None)
    if rc != 0:
        raise MemoryError("orc_expert_ffn: out of memory")
    return (y, h) if want_h else y


@dataclasses.dataclass
class TokenResult:
    u: np.ndarray            # expert and router input (bf16 values after the norm in a stack), float64
    logits: np.ndarray       # the oracle's logits on u
    ids: np.ndarray          # the routing used (given)
    weights: np.ndarray      # softmax of the oracle's logits at ids
    y_routed: np.ndarray     # [k][d]
    y_shared: Optional[np.ndarray]
    out: np.ndarray          # float64 before the output rounding: sum_i w_i y_i + y_shared (+ x)
    x_next: np.ndarray       # out rounded to the activation dtype (bf16 configurations) or as is


def layer_tokens(cfg: synth.MoEConfig, layer: int, X: np.ndarray, ids: np.ndarray, act: int = moe.ACT_GELU_TANH,
                 eps: float = 1e-6, gamma: Optional[np.ndarray] = None, shared: bool = True,
                 threads: Optional[int] = None) -> list:
    """One MoE layer for n tokens X [n][d] (float64 values of the activation dtype) with the given routing
    ids [n][k]: per token the definition of moe.stack_layer_step (configurations with RMSNorm: u =
    bf16(RMSNorm(x)), residual added, output rounded to bf16) or of moe.moe_layer (without: u = x, no
    residual, output as computed)."""
    X = np.asarray(X, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    n, k = ids.shape
    threads = threads or default_threads()
    rw, rs = synth.router_int8(cfg.weight_cfg, layer, cfg.n_experts, cfg.d)
    if cfg.rms_norm:
        g = np.ones(cfg.d) if gamma is None else np.asarray(gamma, dtype=np.float64)
        U = np.stack([moe.f64_round_to_bf16(moe.rms_norm(X[t], g, eps)) for t in range(n)])
    else:
        U = X.copy()
    logits = np.stack([moe.router_logits(rw, rs, U[t]) for t in range(n)])
    y = np.zeros((n, k, cfg.d))
    ys = np.zeros((n, cfg.d)) if shared else None

    def routed(e):
        rows = [(t, i) for t in range(n) for i in range(k) if ids[t, i] == e]
        wgu, wd = oin.expert_weights(cfg, layer, e, threads=1)
        out = expert_ffn_rows(wgu, wd, cfg.sb_bf16, U[[t for t, _ in rows]], act)
        for (t, i), row in zip(rows, out):
            y[t, i] = row

    def shared_part(t0, t1):
        wgu, wd = oin.shared_weights(cfg, layer, threads=1)
        ys[t0:t1] = expert_ffn_rows(wgu, wd, cfg.sb_bf16, U[t0:t1], act)

    valid = [int(e) for e in np.unique(ids) if 0 <= e < cfg.n_experts]
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        jobs = [ex.submit(routed, e) for e in valid]
        if shared:
            step = max(1, -(-n // threads))
            jobs += [ex.submit(shared_part, t0, min(n, t0 + step)) for t0 in range(0, n, step)]
        for j in jobs:
            j.result()
    res = []
    for t in range(n):
        w = moe.gate_weights(logits[t], ids[t])
        out = moe.combine(y[t], w, ys[t] if shared else None, X[t] if cfg.rms_norm else None)
        x_next = moe.f64_round_to_bf16(out) if cfg.x_bf16 else out
        res.append(TokenResult(U[t], logits[t], ids[t].copy(), w, y[t], ys[t] if shared else None, out, x_next))
    return res
