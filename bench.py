"""Decode benchmark of the MoE hot path on one MI355X.

Workload: the 30-layer MoE stack decoded one token at a time (batch 1): per layer RMSNorm -> int8 router
top-8 of 128 -> 4-bit expert GEMVs (gate/up + GELU, down; 8 routed experts + the always-on shared expert,
both in the same launches) -> routing-weighted combine + residual.  d=2816, F=704, shared width 2816,
4-bit affine weights in groups of 64 with bf16 scale/bias, bf16 activations, fp32 accumulation.  All
13.3 GB of expert records are resident in HBM; weights are seeded synthetic draws (no checkpoint).
One step = one token through all 30 layers (one moe_decode_layer launch each), replayed from a HIP
graph; inputs are 256 seeded tokens already in HBM, rotated step by step.

Prints one JSON line: decode tokens/s, plus the roofline of the dominant kernel (the single-launch
layer, timed live with HIP events on its stream) and the CPU oracle's speed on a bounded sample.
Alongside (not the headline value): per-launch times of the layer split in three kernels, a 32-token batched step
and a 128-token prefill chunk through the same stack (grouped products on the matrix cores), the same 4-bit
row routine as one LM-head-sized GEMV (262,144 x 2816), and the same stack served from pinned host memory through 16-slot LFU expert caches (hit rates, host-to-device rate
against a plain pinned copy).
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


# HBM traffic of one layer launch from rocprofv3 FETCH_SIZE and WRITE_SIZE counter runs of this script (2 steps,
# --calibration-copy-mib 256), each scaled by what the counter reads for the plain 256 MiB device copy in the
# same run (FETCH_SIZE x 1.9997, WRITE_SIZE x 1.0).  It is reported only while the kernel's sources are the
# ones the counters were taken on.
LAYER_TRAFFIC_BYTES = 42566437
LAYER_TRAFFIC_SOURCES = ("bit_quantized_expert_int8_amd/csrc/layer.hip", "bit_quantized_expert_int8_amd/csrc/q4_device.h",
                         "bit_quantized_expert_int8_amd/csrc/common.h")
LAYER_TRAFFIC_SHA = "e2f0e1972e8c6818"


def layer_traffic():
    import hashlib
    h = hashlib.sha256()
    for p in LAYER_TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return LAYER_TRAFFIC_BYTES if h.hexdigest()[:16] == LAYER_TRAFFIC_SHA else None


def record_data_bytes(d: int, F: int) -> int:
    """Bytes of one expert's 4-bit codes and bf16 scale/bias (gate/up [2F][d] and down [d][F], groups of 64)."""
    return 2 * F * (d // 2 + (d // 64) * 4) + d * (F // 2 + (F // 64) * 4)


def layer_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one decoded layer: the int8 router and its row scales, the k selected experts'
    records and the shared expert's record (activations, a few KB, not counted)."""
    return cfg.n_experts * cfg.d + cfg.n_experts * 4 + cfg.k * record_data_bytes(cfg.d, cfg.F) + \
        record_data_bytes(cfg.d, cfg.S)


def time_graph(build, reps, stream):
    """Average duration of one replay of the HIP graph that build() records, from HIP events on `stream`."""
    import torch

    with torch.cuda.stream(stream):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            build()
        g.replay()
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def time_layer_kernel(dec, xin, reps):
    """Average duration of the single-launch layer (moe_decode_layer) from HIP events around a graph of one
    launch per layer of the stack, on the stream the launches are captured on."""
    import torch

    out = torch.empty_like(xin)
    bufs = [xin, out]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())

    def layers():
        for l in range(len(dec.layers)):
            dec.layer(l, bufs[l % 2], bufs[(l + 1) % 2], stream=stream)

    return time_graph(layers, reps, stream) / len(dec.layers), reps * len(dec.layers)


def time_split_kernels(dec, xin, reps):
    """Per-launch durations of the layer split in three launches (moe_norm_router_topk; q4_expert_gate_up;
    down + combine = q4_expert_gemv_combine minus gate/up), each from a graph of one launch per layer with
    that layer's routing of the last decoded token."""
    import torch
    from bit_quantized_expert_int8_amd import moeq4 as q

    s, L = dec.shape, len(dec.layers)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    ids_keep = dec.ids_all.clone()
    out = torch.empty_like(xin)
    lg = torch.empty((1, s.n_experts), dtype=torch.float32, device="cuda")
    ids_tmp = torch.empty((1, s.k), dtype=torch.int32, device="cuda")
    w_tmp = torch.empty((1, s.k), dtype=torch.float32, device="cuda")
    u_tmp = torch.empty_like(xin)

    def routers():
        for l, W in enumerate(dec.layers):
            q.moe_norm_router_topk(xin, s.x_dtype, W.gamma, s.eps, 1, s.d, W.router_w, W.router_s, s.n_experts, s.k,
                                   None, ids_tmp, w_tmp, lg, u_tmp, dec.router_ws, dec.router_ws_bytes, stream)

    def gate_ups():
        for l in range(L):
            q.q4_expert_gate_up(dec.routed_pools[l], ids_keep[l], s.k, dec.shared_pools[l], u_tmp, s.x_dtype, 1, s.act,
                                dec.gemv_ws, dec.gemv_ws_bytes, stream)

    def gemv_combines():
        for l in range(L):
            q.q4_expert_gemv_combine(dec.routed_pools[l], ids_keep[l], s.k, dec.shared_pools[l], u_tmp, s.x_dtype, 1,
                                     s.act, dec.weights_all[l], xin, s.x_dtype, out, s.x_dtype, dec.fused_ws,
                                     dec.fused_ws_bytes, stream)

    t_router = time_graph(routers, reps, stream) / L
    t_gate_up = time_graph(gate_ups, reps, stream) / L
    t_gemv_combine = time_graph(gemv_combines, reps, stream) / L
    return {"norm_router_topk_us": round(t_router * 1e6, 3), "gate_up_us": round(t_gate_up * 1e6, 3),
            "down_combine_us": round((t_gemv_combine - t_gate_up) * 1e6, 3)}


def distinct_expert_bytes(dec, cfg):
    """HBM bytes of weights one step reads, from the routing of the last step: per layer the distinct routed
    experts' records, the shared expert's record and the int8 router."""
    from bit_quantized_expert_int8_amd import moeq4 as q

    rb = q.moe_record_bytes(cfg.d, cfg.F, q.MOE_BF16)
    srb = q.moe_record_bytes(cfg.d, cfg.S, q.MOE_BF16)
    total, distinct = 0, []
    for l in range(len(dec.layers)):
        n = int(dec.ids_all[l].unique().numel())
        distinct.append(n)
        total += n * rb + srb + cfg.n_experts * cfg.d
    return total, sum(distinct) / len(distinct)


def measure_batched(shape, layers, cfg, tokens, steps, warmup, T=32):
    """T tokens decoded together through the stack (one grouped call per layer, the expert products on the
    matrix cores), graph-replayed with the token batch rotated each step: 32 (the batched decode
    configuration) or 128 (a prefill chunk)."""
    import torch
    from bit_quantized_expert_int8_amd import decoder

    dec = decoder.MoEDecoder(shape, layers, T=T)
    n_batches = tokens.shape[0] // T
    batches = tokens[: n_batches * T].reshape(n_batches, T, cfg.d)
    xin = torch.empty((T, cfg.d), dtype=torch.bfloat16, device="cuda")
    xout = torch.empty_like(xin)
    xin.copy_(batches[0])
    g = dec.capture(xin, xout)
    for i in range(warmup):
        xin.copy_(batches[i % n_batches])
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        xin.copy_(batches[i % n_batches])
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    step_s = e0.elapsed_time(e1) * 1e-3 / steps
    nbytes, mean_distinct = distinct_expert_bytes(dec, cfg)
    return {"tokens_per_step": T, "tok_s": round(T / step_s, 1), "ms_per_step": round(step_s * 1e3, 4),
            "per_layer_us": round(step_s / len(layers) * 1e6, 2), "distinct_experts_per_layer": round(mean_distinct, 1),
            "weight_bytes_per_step": nbytes, "achieved_GBps": round(nbytes / step_s / 1e9, 1)}


def measure_lm_head(steps=10, reps=10):
    """q4_gemv (the experts' 4-bit row routine as a plain matrix GEMV) at LM-head scale: 262,144 rows (a
    vocabulary) x 2816, bf16 scale/bias, one bf16 token, seeded random codes; graph-timed on its stream."""
    import torch
    from bit_quantized_expert_int8_amd import moeq4 as q

    N, K = 262144, 2816
    g = torch.Generator(device="cuda").manual_seed(5)
    codes = torch.randint(0, 2**31 - 1, (N, K // 8), dtype=torch.int32, device="cuda", generator=g)
    sb = (torch.rand((N, K // 64, 2), device="cuda", generator=g) * 0.01).to(torch.bfloat16)
    x = torch.randn((1, K), device="cuda", generator=g).to(torch.bfloat16)
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())

    def calls():
        for _ in range(steps):
            q.q4_gemv(x, q.MOE_BF16, 1, codes, sb, q.MOE_BF16, N, K, y, stream)

    t = time_graph(calls, reps, stream) / steps
    nbytes = N * (K // 2) + N * (K // 64) * 4
    return {"rows": N, "cols": K, "us_per_call": round(t * 1e6, 2), "weight_bytes": nbytes,
            "achieved_GBps": round(nbytes / t / 1e9, 1), "frac_of_8TBps": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}


def measure_streamed(shape, layers, cfg, dec, n_tokens):
    """Experts served from pinned host memory through a 16-slot LFU cache per layer (routing forced by a
    Zipf(1.1) trace): tokens/s over all tokens and over the second half (warm cache), hit rates, and the
    host-to-device rate against a plain pinned 1 GiB copy measured in the same process."""
    import numpy as np
    import torch
    import synth
    from bit_quantized_expert_int8_amd import moeq4 as q

    L, E, k, n_slots = len(layers), cfg.n_experts, cfg.k, 16
    rb = layers[0].pool.shape[1]
    # pinned-copy reference rate
    ref_h = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    ref_d = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    ref_d.copy_(ref_h, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        ref_d.copy_(ref_h, non_blocking=True)
    e1.record()
    e1.synchronize()
    pinned_gbps = 3 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del ref_h, ref_d

    host = [torch.empty((E, rb), dtype=torch.uint8, pin_memory=True) for _ in range(L)]
    for h, lay in zip(host, layers):
        h.copy_(lay.pool)
    slots = [torch.empty((n_slots, rb), dtype=torch.uint8, device="cuda") for _ in range(L)]
    cache = q.moe_expert_cache_create(L, E, n_slots, rb, [h.data_ptr() for h in host], [s_.data_ptr() for s_ in slots])
    try:
        trace = synth.zipf_trace(4, n_tokens, L, k, E, 1.1)
        forced = torch.from_numpy(trace.astype(np.int32)).cuda()
        slot_pools = [q.pool(s_, rb, n_slots, cfg.d, cfg.F, shape.sb_dtype) for s_ in slots]
        slot_ids = torch.empty((L, 1, k), dtype=torch.int32, device="cuda")
        copy_stream = torch.cuda.Stream()
        compute = torch.cuda.current_stream()
        ready = [torch.cuda.Event() for _ in range(L)]
        freed = [torch.cuda.Event() for _ in range(L)]
        for ev in ready + freed:
            ev.record(copy_stream)
        copy_stream.synchronize()
        bits = np.stack([synth.activation(cfg.act_cfg, t % 64, cfg.d, bf16=True) for t in range(64)]).astype(np.int16)
        toks = torch.from_numpy(bits).view(torch.bfloat16).cuda().reshape(64, 1, cfg.d)
        bufs = [torch.empty((1, cfg.d), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        half = n_tokens // 2
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(n_tokens):
            if t == half:
                torch.cuda.synchronize()
                t_half = time.perf_counter()
                hits_half = sum(q.moe_expert_cache_stats(cache, l)[0] for l in range(L))
                bytes_half = q.moe_expert_cache_stats(cache, -1)[2]
            x = toks[t % 64]
            for l in range(L):
                q.expert_cache_stage(cache, l, trace[t, l].tolist(), slot_ids[l], copy_stream, freed[l], ready[l])
                compute.wait_event(ready[l])
                out = bufs[l % 2]
                dec.layer(l, x, out, forced_ids=forced[t, l].reshape(1, k), routed_pool=slot_pools[l], ids=slot_ids[l])
                freed[l].record(compute)
                x = out
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        hits, misses, nbytes = q.moe_expert_cache_stats(cache, -1)
    finally:
        q.moe_expert_cache_destroy(cache)
    req = n_tokens * L * k
    warm_req = (n_tokens - half) * L * k
    return {"tokens": n_tokens, "layers": L, "slots_per_layer": n_slots, "trace": "Zipf(1.1) forced routing",
            "tok_s_all": round(n_tokens / (t1 - t0), 2), "tok_s_warm": round((n_tokens - half) / (t1 - t_half), 2),
            "hit_rate_all": round(hits / req, 4), "hit_rate_warm": round((hits - hits_half) / warm_req, 4),
            "bytes_copied": int(nbytes), "h2d_GBps_effective_warm": round((nbytes - bytes_half) / (t1 - t_half) / 1e9, 2),
            "pinned_copy_GBps": round(pinned_gbps, 2)}


def cpu_baseline(cfg, n_layers_sample, repeats, token=0):
    """The CPU oracle (float64 numpy) on a bounded sample: one token through the first layers of the
    stack, repeated; the records of the experts it routes to are prepared beforehand (untimed)."""
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
    for _ in range(repeats):
        x = x0
        for L in layers:
            _, _, x = moe.stack_layer_step(L, x, cfg.k)
    dt = time.perf_counter() - t0
    per_layer = dt / (n_layers_sample * repeats)
    return {"value": 1.0 / (per_layer * cfg.n_layers), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"token {token} through layers 0-{n_layers_sample - 1} of {cfg.n_layers}, {repeats} times "
                      f"({dt:.1f} s), scaled to one 30-layer token"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--roofline-reps", type=int, default=20)
    ap.add_argument("--cpu-layers", type=int, default=2)
    ap.add_argument("--cpu-repeats", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the batched and streamed measurements")
    ap.add_argument("--stream-tokens", type=int, default=512)
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one plain device-to-device copy of this many MiB (a reference for the HBM "
                         "traffic counters of a profiled run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
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

    if args.calibration_copy_mib:
        src = torch.empty(args.calibration_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    dur, launches = time_layer_kernel(dec, xin, args.roofline_reps)
    nbytes = layer_bytes(cfg)
    achieved = nbytes / dur / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": layer_traffic(),
                "kernel": "decode_layer_kernel (moe_decode_layer: RMSNorm, int8 router + top-8, 8 routed + shared "
                          "4-bit expert FFNs, combine + residual, one launch per layer)",
                "bytes_per_launch": nbytes, "avg_launch_us": round(dur * 1e6, 3), "launches_timed": launches}
    split = time_split_kernels(dec, xin, args.roofline_reps)
    step_bytes, _ = distinct_expert_bytes(dec, cfg)

    out = {"metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(gpu_s / args.steps * 1e3, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{args.layers}-layer MoE stack decode, batch 1, d=2816, 128 experts top-8, "
                                  "F=704, shared 2816, 4-bit g64 bf16 scale/bias, int8 router, RMSNorm + residual",
                      "global_batch": 1, "layers": args.layers, "tokens_in_rotation": n_tok,
                      "expert_bytes_resident_gb": round(sum(L.pool.numel() + L.shared.numel() for L in layers) / 1e9, 3),
                      "parallelism": "single GPU"},
           "roofline": roofline, "wall_s_timed_region": round(wall, 4), "build_s": round(t_build, 1),
           "step_weight_bytes": step_bytes, "step_achieved_GBps": round(step_bytes / (gpu_s / args.steps) / 1e9, 1),
           "per_layer_us": round(gpu_s / args.steps / args.layers * 1e6, 2),
           "decode_mode": dec.mode, "split_kernels_us": split}
    if not args.no_extras:
        out["batched"] = measure_batched(shape, layers, cfg, tokens.reshape(n_tok, cfg.d), 20, 3)
        out["prefill_chunk_128"] = measure_batched(shape, layers, cfg, tokens.reshape(n_tok, cfg.d), 8, 2, T=128)
        out["lm_head_q4_gemv"] = measure_lm_head()
        out["streamed"] = measure_streamed(shape, layers, cfg, dec, args.stream_tokens)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_layers, args.cpu_repeats)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
