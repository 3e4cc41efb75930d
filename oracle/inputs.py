"""Oracle-side assembly of a layer's weights from the seeded generator (TEST INFRASTRUCTURE ONLY).

The fp32 draws come from ``synth``; the 4-bit records are made by the oracle's own quantizer.  Records
are built lazily per expert, so a full-size layer (128 experts, 3.3 MB each) can be checked on the few
experts one token selects.
"""
from __future__ import annotations

import functools

import numpy as np

import synth
from . import moe


def expert_weights(cfg: synth.MoEConfig, layer: int, e: int, threads: int = 0):
    """fp32 gate_up [2F][d] and down [d][F] of routed expert e (before quantization)."""
    wgu = synth.weight_f32(cfg.weight_cfg, layer, synth.TAG_GATE_UP, e, 2 * cfg.F, cfg.d, threads=threads)
    wd = synth.weight_f32(cfg.weight_cfg, layer, synth.TAG_DOWN, e, cfg.d, cfg.F, threads=threads)
    return wgu, wd


def shared_weights(cfg: synth.MoEConfig, layer: int, threads: int = 0):
    """fp32 gate_up [2S][d] and down [d][S] of the shared expert (before quantization)."""
    wgu = synth.weight_f32(cfg.weight_cfg, layer, synth.TAG_SHARED_GATE_UP, 0, 2 * cfg.S, cfg.d, threads=threads)
    wd = synth.weight_f32(cfg.weight_cfg, layer, synth.TAG_SHARED_DOWN, 0, cfg.d, cfg.S, threads=threads)
    return wgu, wd


def expert_record(cfg: synth.MoEConfig, layer: int, e: int) -> np.ndarray:
    return moe.encode_record(*expert_weights(cfg, layer, e), cfg.sb_bf16)


def shared_record(cfg: synth.MoEConfig, layer: int) -> np.ndarray:
    return moe.encode_record(*shared_weights(cfg, layer), cfg.sb_bf16)


def oracle_layer(cfg: synth.MoEConfig, layer: int, cache_experts: int = 16, gamma_ones: bool = True) -> moe.OracleLayer:
    rw, rs = synth.router_int8(cfg.weight_cfg, layer, cfg.n_experts, cfg.d)

    @functools.lru_cache(maxsize=cache_experts)
    def rec(e: int) -> np.ndarray:
        return expert_record(cfg, layer, e)

    gamma = synth.rms_gamma(cfg.weight_cfg, layer, cfg.d, ones=gamma_ones) if cfg.rms_norm else None
    return moe.OracleLayer(cfg.d, cfg.F, cfg.S, cfg.sb_bf16, rw, rs, rec, shared_record(cfg, layer), gamma)


def token_input(cfg: synth.MoEConfig, token: int) -> np.ndarray:
    """Activation of one token as float64 values (bf16-exact for bf16 configurations)."""
    x = synth.activation(cfg.act_cfg, token, cfg.d, bf16=cfg.x_bf16)
    return moe.bf16_bits_to_f64(x) if cfg.x_bf16 else x.astype(np.float64)
