"""Decode benchmark of the MoE hot path on one MI355X.

Workload: the 30-layer MoE stack decoded one token at a time (batch 1): per layer RMSNorm -> int8 router
top-8 of 128 -> 4-bit expert GEMVs (gate/up + GELU, down; 8 routed experts + the always-on shared expert,
both in the same launches) -> routing-weighted combine + residual.  d=2816, F=704, shared width 2816,
4-bit affine weights in groups of 64 with bf16 scale/bias, bf16 activations, fp32 accumulation.  All
13.3 GB of expert records are resident in HBM; weights are seeded synthetic draws (no checkpoint).
One step = one token through all 30 layers, replayed from a HIP graph; inputs are 256 seeded tokens
already in HBM, rotated step by step.

Prints one JSON line: decode tokens/s, plus the roofline of the dominant kernel (the expert gate/up
GEMV launch, timed live with HIP events on its stream) and the CPU oracle's speed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE decode tokens/s; 4-bit expert GEMV achieved HBM GB/s vs peak (1 MI355X)"
HBM_PEAK_GBS = 8000.0


def build_stack(cfg, n_layers):
    import numpy as np
    import torch
    import synth
    import synth.device as sdev
    from bit_quantized_expert_int8_amd import decoder, moeq4 as q

    shape = decoder.Shape(d=cfg.d, n_experts=cfg.n_experts, k=cfg.k, F=cfg.F, S=cfg.S, sb_dtype=q.MOE_BF16,
                          x_dtype=q.MOE_BF16, act=q.MOE_ACT_GELU_TANH, rms_norm=True)
    layers = []
    for l in range(n_layers):
        def fill_expert(e, wgu, wd, l=l):
            sdev.weight_into(wgu, cfg.weight_cfg, l, synth.TAG_GATE_UP, e)
            sdev.weight_into(wd, cfg.weight_cfg, l, synth.TAG_DOWN, e)

        def fill_shared(wgu, wd, l=l):
            sdev.weight_into(wgu, cfg.weight_cfg, l, synth.TAG_SHARED_GATE_UP, 0)
            sdev.weight_into(wd, cfg.weight_cfg, l, synth.TAG_SHARED_DOWN, 0)

        rw, rs = synth.router_int8(cfg.weight_cfg, l, cfg.n_experts, cfg.d)
        gamma = torch.from_numpy(synth.rms_gamma(cfg.weight_cfg, l, cfg.d, ones=True))
        layers.append(decoder.pack_layer(shape, fill_expert, fill_shared, torch.from_numpy(rw), torch.from_numpy(rs),
                                         gamma))
    return shape, layers


def gate_up_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one gate/up launch: k routed experts' and the shared expert's gate+up
    codes (d/2 bytes per row) and bf16 scale/bias (d/64 * 4 bytes per row)."""
    row = cfg.d // 2 + (cfg.d // 64) * 4
    return (cfg.k * 2 * cfg.F + 2 * cfg.S) * row


def time_gate_up(dec, cfg, reps):
    """Average duration of the gate/up GEMV launch, from HIP events around a HIP graph of one launch per
    layer (each with that layer's routing of the last decoded token), replayed `reps` times."""
    import torch
    from bit_quantized_expert_int8_amd import moeq4 as q

    s = dec.shape
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for l in range(len(dec.layers)):
                q.q4_expert_gate_up(dec.routed_pools[l], dec.ids_all[l], s.k, dec.shared_pools[l], dec.u, s.x_dtype, 1,
                                    s.act, dec.gemv_ws, dec.gemv_ws_bytes, torch.cuda.current_stream())
        g.replay()
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    e1.synchronize()
    launches = reps * len(dec.layers)
    return e0.elapsed_time(e1) * 1e-3 / launches, launches


def cpu_baseline(cfg, n_layers_sample, token=0):
    """The CPU oracle (float64 numpy) on a bounded sample: one token through the first layers of the
    stack, records of the experts it routes to prepared beforehand (untimed)."""
    import numpy as np
    import synth
    from oracle import inputs as oin
    from oracle import moe

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    layers = [oin.oracle_layer(cfg, l, cache_experts=16) for l in range(n_layers_sample)]
    x0 = moe.f64_round_to_bf16(oin.token_input(cfg, token))
    # untimed pass: draws and encodes the records this token needs
    x = x0
    for L in layers:
        _, _, x = moe.stack_layer_step(L, x, cfg.k)
    t0 = time.perf_counter()
    x = x0
    for L in layers:
        _, _, x = moe.stack_layer_step(L, x, cfg.k)
    dt = time.perf_counter() - t0
    per_layer = dt / n_layers_sample
    return {"value": 1.0 / (per_layer * cfg.n_layers), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"token {token} through {n_layers_sample} of {cfg.n_layers} layers "
                      f"({dt:.2f} s), scaled to one 30-layer token"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--roofline-reps", type=int, default=20)
    ap.add_argument("--cpu-layers", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import numpy as np
    import synth
    from bit_quantized_expert_int8_amd import decoder

    cfg = synth.STACK
    torch.cuda.set_device(0)
    t_build = time.perf_counter()
    shape, layers = build_stack(cfg, args.layers)
    torch.cuda.synchronize()
    t_build = time.perf_counter() - t_build
    dec = decoder.MoEDecoder(shape, layers, T=1)

    n_tok = cfg.n_tokens
    bits = np.stack([synth.activation(cfg.act_cfg, t, cfg.d, bf16=True) for t in range(n_tok)]).astype(np.int16)
    tokens = torch.from_numpy(bits).view(torch.bfloat16).cuda().reshape(n_tok, 1, cfg.d)
    xin = torch.empty((1, cfg.d), dtype=torch.bfloat16, device="cuda")
    xout = torch.empty_like(xin)
    xin.copy_(tokens[0])
    g = dec.capture(xin, xout)

    for i in range(args.warmup):
        xin.copy_(tokens[i % n_tok])
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        xin.copy_(tokens[i % n_tok])
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = e0.elapsed_time(e1) * 1e-3
    tok_s = args.steps / gpu_s

    dur, launches = time_gate_up(dec, cfg, args.roofline_reps)
    nbytes = gate_up_bytes(cfg)
    achieved = nbytes / dur / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "gate_up_kernel (q4_expert_gate_up: 8 routed + shared expert, gate/up + GELU)",
                "bytes_per_launch": nbytes, "avg_launch_us": round(dur * 1e6, 3), "launches_timed": launches}

    out = {"metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(gpu_s / args.steps * 1e3, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{args.layers}-layer MoE stack decode, batch 1, d=2816, 128 experts top-8, "
                                  "F=704, shared 2816, 4-bit g64 bf16 scale/bias, int8 router, RMSNorm + residual",
                      "global_batch": 1, "layers": args.layers, "tokens_in_rotation": n_tok,
                      "expert_bytes_resident_gb": round(sum(L.pool.numel() + L.shared.numel() for L in layers) / 1e9, 3),
                      "parallelism": "single GPU"},
           "roofline": roofline, "wall_s_timed_region": round(wall, 4), "build_s": round(t_build, 1)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_layers)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
