"""Decode benchmark of the MoE hot path on one MI355X.

Workload: the 30-layer MoE stack decoded one token at a time (batch 1): per layer RMSNorm -> int8 router
top-8 of 128 -> 4-bit expert GEMVs (gate/up + GELU, down; 8 routed experts + the always-on shared expert,
both in the same launches) -> routing-weighted combine + residual.  d=2816, F=704, shared width 2816,
4-bit affine weights in groups of 64 with bf16 scale/bias, bf16 activations, fp32 accumulation.  All
13.3 GB of expert records are resident in HBM; weights are seeded synthetic draws (no checkpoint).
One step = one token through all 30 layers in one moe_decode_stack launch (or, with --mode layer, one
moe_decode_layer launch per layer), replayed from a HIP graph; inputs are 256 seeded tokens already in HBM,
rotated step by step.

Prints one JSON line: decode tokens/s, plus the roofline of the dominant kernel (the launch that decodes the
token, timed live with HIP events on its stream), a plain streaming read of 2 GiB as the box's achievable
read rate, and the CPU oracle on a bounded sample of the timed tokens (timed with all host cores and with
one, and checked against the GPU's per-layer results: routing matches, near ties, largest errors).
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


# HBM traffic of one launch of the dominant kernel from rocprofv3 FETCH_SIZE and WRITE_SIZE counter runs of
# this script (2 steps, --calibration-copy-mib 256), each scaled by what the counter reads for the plain
# 256 MiB device copy in the same run.  Keyed by decode mode; reported only while the kernel's sources are
# the ones the counters were taken on (first 16 hex digits of their sha256).
TRAFFIC = {
    # mode: (bytes per launch, sources sha)
    "stack": (1_259_211_654, "03603fed06c398d5"),   # 609,760.8 KiB fetched x 1.99966, 10,384.6 KiB written x 1.0
    "layer": (42_268_500, "7784cc6cbe2214d1"),      # 20,473.0 KiB fetched x 1.99966, 338.8 KiB written x 1.0
}
TRAFFIC_SOURCES = ("bit_quantized_expert_int8_amd/csrc/layer.hip", "bit_quantized_expert_int8_amd/csrc/q4_device.h",
                   "bit_quantized_expert_int8_amd/csrc/common.h")


def log(msg):
    """A progress line on stderr (the JSON result is the only line on stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def sources_sha():
    import hashlib
    h = hashlib.sha256()
    for p in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_traffic(mode):
    t = TRAFFIC.get(mode)
    return t[0] if t and t[1] == sources_sha() else None


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


def time_stack_kernel(dec, xin, reps):
    """Average duration of one moe_decode_stack launch (every layer of the token in one launch), from HIP
    events around a graph of replays of that launch on the stream it is captured on."""
    import torch

    out = torch.empty_like(xin)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    return time_graph(lambda: dec.step(xin, out, stream=stream), reps, stream), reps


def measure_hbm_read(gib=2, reps=10):
    """The box's achievable streaming read rate: moe_hbm_read_probe over a 2 GiB buffer (16-byte nontemporal
    loads on every compute unit), HIP events around `reps` calls on one stream."""
    import torch
    from bit_quantized_expert_int8_amd import moeq4 as q

    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        q.moe_hbm_read_probe(buf, n, sink, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            q.moe_hbm_read_probe(buf, n, sink, stream)
        e1.record(stream)
    e1.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del buf
    return {"bytes": n, "us_per_read": round(t * 1e6, 1), "GBps": round(n / t / 1e9, 1),
            "frac_of_8TBps": round(n / t / 1e9 / HBM_PEAK_GBS, 4)}


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


def measure_lm_head(steps=10, reps=10, warm=200):
    """q4_gemv (the experts' 4-bit row routine as a plain matrix GEMV) at LM-head scale: 262,144 rows (a
    vocabulary) x 2816, bf16 scale/bias, one bf16 token, seeded random codes; graph-timed on its stream after
    `warm` untimed launches (its duration settles only after about 150 back-to-back launches: --study lmhead)."""
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

    with torch.cuda.stream(stream):
        for _ in range(warm):
            q.q4_gemv(x, q.MOE_BF16, 1, codes, sb, q.MOE_BF16, N, K, y, stream)
    t = time_graph(calls, reps, stream) / steps
    nbytes = N * (K // 2) + N * (K // 64) * 4
    return {"rows": N, "cols": K, "warm_launches": warm, "us_per_call": round(t * 1e6, 2), "weight_bytes": nbytes,
            "achieved_GBps": round(nbytes / t / 1e9, 1), "frac_of_8TBps": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}


def lm_head_drift(launches=400, window=20):
    """q4_gemv at the LM-head shape and a plain read of the same number of bytes (moe_hbm_read_probe), each
    launched `launches` times back to back with a HIP event between launches: one JSON line with the mean
    duration of every `window` consecutive launches (whether the duration holds under sustained load)."""
    import torch
    from bit_quantized_expert_int8_amd import moeq4 as q

    N, K = 262144, 2816
    g = torch.Generator(device="cuda").manual_seed(5)
    codes = torch.randint(0, 2**31 - 1, (N, K // 8), dtype=torch.int32, device="cuda", generator=g)
    sb = (torch.rand((N, K // 64, 2), device="cuda", generator=g) * 0.01).to(torch.bfloat16)
    x = torch.randn((1, K), device="cuda", generator=g).to(torch.bfloat16)
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    nbytes = N * (K // 2) + N * (K // 64) * 4
    buf = torch.empty(nbytes // 256 * 256, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()

    def per_launch(fn):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(launches + 1)]
        ev[0].record(s)
        for i in range(launches):
            fn()
            ev[i + 1].record(s)
        torch.cuda.synchronize()
        d = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(launches)]
        return [round(sum(d[i:i + window]) / window, 1) for i in range(0, launches, window)]

    out = {"weight_bytes": nbytes, "window": window}
    for name, fn in (("q4_gemv_us", lambda: q.q4_gemv(x, q.MOE_BF16, 1, codes, sb, q.MOE_BF16, N, K, y, s)),
                     ("read_probe_us", lambda: q.moe_hbm_read_probe(buf, buf.numel(), sink, s)),
                     ("q4_gemv_again_us", lambda: q.q4_gemv(x, q.MOE_BF16, 1, codes, sb, q.MOE_BF16, N, K, y, s))):
        out[name] = per_launch(fn)
        log(f"{name}: {out[name]}")
    print(json.dumps(out), flush=True)


def pinned_pools(layers):
    """Every layer's expert records copied to pinned host memory (the slow tier of the expert cache)."""
    import torch

    host = [torch.empty(lay.pool.shape, dtype=torch.uint8, pin_memory=True) for lay in layers]
    for h, lay in zip(host, layers):
        h.copy_(lay.pool)
    return host


def measure_streamed(shape, layers, cfg, dec, n_tokens, overlap=True, copy_streams=1, pinned_gbps=None, host=None,
                     run_ahead=False):
    """Experts served from pinned host memory through a 16-slot LFU cache per layer (routing forced by a
    Zipf(1.1) trace): tokens/s over all tokens and over the second half (warm cache), hit rates, and the
    host-to-device rate against a plain pinned 1 GiB copy measured in the same process.

    With `overlap`, each layer runs as two launches: the router and the shared expert (moe_decode_layer_part
    part 1) go ahead while the layer's missing experts are copied, and the routed experts and the combine
    (part 2) wait for the copies; without, the whole layer waits for them.  Layers' copies go to
    `copy_streams` streams in turn.  Unless `run_ahead`, the host stages layer l of a token once layer l of the
    previous token has run (a host-side wait, so the copies are enqueued without a device-side wait; the
    copy streams still hold up to a token of work)."""
    import numpy as np
    import torch
    import synth
    from bit_quantized_expert_int8_amd import moeq4 as q

    L, E, k, n_slots = len(layers), cfg.n_experts, cfg.k, 16
    rb = layers[0].pool.shape[1]
    if pinned_gbps is None:
        pinned_gbps = pinned_copy_gbps()

    if host is None:
        host = pinned_pools(layers)
    slots = [torch.empty((n_slots, rb), dtype=torch.uint8, device="cuda") for _ in range(L)]
    cache = q.moe_expert_cache_create(L, E, n_slots, rb, [h.data_ptr() for h in host], [s_.data_ptr() for s_ in slots])
    try:
        trace = synth.zipf_trace(4, n_tokens, L, k, E, 1.1)
        forced = torch.from_numpy(trace.astype(np.int32)).cuda()
        slot_pools = [q.pool(s_, rb, n_slots, cfg.d, cfg.F, shape.sb_dtype) for s_ in slots]
        slot_ids = torch.empty((L, 1, k), dtype=torch.int32, device="cuda")
        cstreams = [torch.cuda.Stream() for _ in range(copy_streams)]
        compute = torch.cuda.current_stream()
        ready = [torch.cuda.Event() for _ in range(L)]
        freed = [torch.cuda.Event() for _ in range(L)]
        for ev in ready + freed:
            ev.record(cstreams[0])
        cstreams[0].synchronize()
        bits = np.stack([synth.activation(cfg.act_cfg, t % 64, cfg.d, bf16=True) for t in range(64)]).astype(np.int16)
        toks = torch.from_numpy(bits).view(torch.bfloat16).cuda().reshape(64, 1, cfg.d)
        bufs = [torch.empty((1, cfg.d), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        half = n_tokens // 2
        host_s = 0.0   # time the host spends issuing the layers' work (policy, copies, launches, events)
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
                th = time.perf_counter()
                if not run_ahead:
                    freed[l].synchronize()
                q.expert_cache_stage(cache, l, trace[t, l].tolist(), slot_ids[l], cstreams[l % copy_streams], freed[l],
                                     ready[l])
                out = bufs[l % 2]
                fi = forced[t, l].reshape(1, k)
                if overlap == "split":
                    # the two launches of the overlap, both after the copies (isolates the launch split)
                    compute.wait_event(ready[l])
                    dec.layer_part(1, l, x, out, forced_ids=fi, routed_pool=slot_pools[l], ids=slot_ids[l])
                    dec.layer_part(2, l, x, out, forced_ids=fi, routed_pool=slot_pools[l], ids=slot_ids[l])
                elif overlap:
                    dec.layer_part(1, l, x, out, forced_ids=fi, routed_pool=slot_pools[l], ids=slot_ids[l])
                    compute.wait_event(ready[l])
                    dec.layer_part(2, l, x, out, forced_ids=fi, routed_pool=slot_pools[l], ids=slot_ids[l])
                else:
                    compute.wait_event(ready[l])
                    dec.layer(l, x, out, forced_ids=fi, routed_pool=slot_pools[l], ids=slot_ids[l])
                freed[l].record(compute)
                host_s += time.perf_counter() - th
                x = out
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        dec.check_status()
        hits, misses, nbytes = q.moe_expert_cache_stats(cache, -1)
        hits_per_layer = [int(q.moe_expert_cache_stats(cache, l)[0]) for l in range(L)]
    finally:
        q.moe_expert_cache_destroy(cache)
    req = n_tokens * L * k
    warm_req = (n_tokens - half) * L * k
    return {"tokens": n_tokens, "layers": L, "slots_per_layer": n_slots, "trace": "Zipf(1.1) forced routing",
            "overlap": ("two launches per layer after the copies" if overlap == "split" else
                        "shared expert during the copies (two launches per layer)" if overlap else "none"),
            "copy_streams": copy_streams,
            "tok_s_all": round(n_tokens / (t1 - t0), 2), "tok_s_warm": round((n_tokens - half) / (t1 - t_half), 2),
            "hit_rate_all": round(hits / req, 4), "hit_rate_warm": round((hits - hits_half) / warm_req, 4),
            "bytes_copied": int(nbytes), "h2d_GBps_effective_warm": round((nbytes - bytes_half) / (t1 - t_half) / 1e9, 2),
            "pinned_copy_GBps": round(pinned_gbps, 2), "host_issue_us_per_layer": round(host_s / (n_tokens * L) * 1e6, 1),
            "wall_us_per_layer": round((t1 - t0) / (n_tokens * L) * 1e6, 1), "hits_per_layer": hits_per_layer,
            "trace_args": {"seed": 4, "tokens": n_tokens, "layers": L, "k": k, "experts": E, "zipf_s": 1.1,
                           "slots": n_slots}}


def lfu_misses(trace, n_slots):
    """The experts each (token, layer) had to copy under the library's LFU policy (moe_expert_cache in its
    host-only mode: the policy and the bookkeeping without a GPU), as a list of sets per token per layer."""
    import numpy as np
    from bit_quantized_expert_int8_amd import moeq4 as q

    T, L, k = trace.shape
    E = int(trace.max()) + 1
    rb = 256
    host = [np.zeros(E * rb, dtype=np.uint8) for _ in range(L)]
    slots = [np.zeros(n_slots * rb, dtype=np.uint8) for _ in range(L)]
    ids_out = np.zeros(k, dtype=np.int32)
    cache = q.moe_expert_cache_create(L, E, n_slots, rb, [h.ctypes.data for h in host], [s_.ctypes.data for s_ in slots],
                                      q.MOE_CACHE_HOST_ONLY)
    missed = [[None] * L for _ in range(T)]
    try:
        for t in range(T):
            for l in range(L):
                before = q.moe_expert_cache_slots(cache, l, n_slots)
                q.expert_cache_stage(cache, l, trace[t, l].tolist(), ids_out.ctypes.data)
                after = q.moe_expert_cache_slots(cache, l, n_slots)
                missed[t][l] = {e for b, e in zip(before, after) if e != b and e >= 0}
    finally:
        q.moe_expert_cache_destroy(cache)
    return missed


def predictor_stats(trace, missed):
    """Cross-layer and temporal prefetch predictors on a routing trace: for each (token, layer) a predictor
    names k experts before the layer's routing is known; precision = share of the named experts the layer
    then uses, coverage = share of the layer's cache misses the named set contains (what a prefetch of it
    would have hidden), waste = named experts that were neither used nor missing (bandwidth spent for
    nothing if prefetched)."""
    import numpy as np

    T, L, k = trace.shape
    preds = {
        "cross_layer": lambda t, l: set(trace[t, l - 1].tolist()) if l > 0 else None,
        "previous_token": lambda t, l: set(trace[t - 1, l].tolist()) if t > 0 else None,
    }
    counts = {}
    for l in range(L):
        counts[l] = np.zeros(int(trace.max()) + 1, dtype=np.int64)
    out = {name: {"precision": 0.0, "coverage_hits": 0, "misses": 0, "named_not_used": 0, "cases": 0}
           for name in list(preds) + ["popularity"]}
    for t in range(T):
        for l in range(L):
            actual = set(trace[t, l].tolist())
            miss = missed[t][l]
            named = {name: f(t, l) for name, f in preds.items()}
            if t > 0:
                named["popularity"] = set(np.argsort(-counts[l], kind="stable")[:k].tolist())
            for name, p in named.items():
                if p is None:
                    continue
                o = out[name]
                o["cases"] += 1
                o["precision"] += len(p & actual) / k
                o["coverage_hits"] += len(p & miss)
                o["misses"] += len(miss)
                o["named_not_used"] += len(p - actual)
            counts[l][trace[t, l]] += 1
    res = {}
    for name, o in out.items():
        n = max(1, o["cases"])
        res[name] = {"precision": round(o["precision"] / n, 4),
                     "miss_coverage": round(o["coverage_hits"] / max(1, o["misses"]), 4),
                     "named_not_used_per_layer": round(o["named_not_used"] / n, 3)}
    return res


def prefetch_study(args):
    """Cross-layer prefetch and overlap granularity on the expert-cache trace: one JSON line.

    Overlap: the streamed decode of the same tokens without overlap (each layer waits for its copies, then
    one launch) and with the per-layer (coarse) overlap (router + shared expert launched before the wait,
    routed experts + combine after it), measured; and a bound for per-expert (fine) overlap, where each
    routed expert would start as soon as its own record has landed: the compute it could hide is at most the
    routed part's duration minus one expert's share, per layer with a miss (the durations measured here).
    Predictors: lfu_misses + predictor_stats on the trace as the bench uses it (every layer ranks experts by
    the same Zipf law) and on a copy whose layers each permute the expert ids (a popularity of their own)."""
    import numpy as np
    import torch
    import synth
    from bit_quantized_expert_int8_amd import decoder

    cfg = synth.STACK
    shape, layers = build_stack(cfg, args.layers)
    dec = decoder.MoEDecoder(shape, layers, T=1, mode=args.mode)
    L, E, k, n_tok = len(layers), cfg.n_experts, cfg.k, args.stream_tokens
    log("stack built")
    pinned = pinned_copy_gbps()
    host = pinned_pools(layers)
    runs = {}
    for name, overlap in (("none", False), ("coarse", True), ("split_no_overlap", "split")):
        runs[name] = measure_streamed(shape, layers, cfg, dec, n_tok, overlap=overlap, copy_streams=args.copy_streams,
                                      pinned_gbps=pinned, host=host)
        log(f"{name}: {runs[name]['tok_s_all']} tokens/s")
    del host
    # part durations of one layer (graph of 30 launches each, HIP events on the launch stream)
    x = torch.zeros((1, cfg.d), dtype=torch.bfloat16, device="cuda")
    bufs = [x, torch.empty_like(x)]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    # part 2 consumes the routing of part 1 of the same call: it is timed as the pair minus part 1, and part 1
    # alone runs on a decoder of its own (a workspace whose part 1 is not followed by part 2 is spent)
    d1 = decoder.MoEDecoder(shape, layers, T=1, mode="layer")
    part_us = {1: time_graph(lambda: [d1.layer_part(1, l, bufs[l % 2], bufs[(l + 1) % 2], stream=stream)
                                      for l in range(L)], 10, stream) / L * 1e6}
    del d1

    def pairs():
        for l in range(L):
            dec.layer_part(1, l, bufs[l % 2], bufs[(l + 1) % 2], stream=stream)
            dec.layer_part(2, l, bufs[l % 2], bufs[(l + 1) % 2], stream=stream)

    part_us[2] = time_graph(pairs, 10, stream) / L * 1e6 - part_us[1]
    dec.check_status()
    # the host's cost of issuing one layer (Python binding and launch), eagerly, as the streamed loop does:
    # one moe_decode_layer call against a part 1 + part 2 pair
    issue_us = {}
    for name, fn in (("layer", lambda l: dec.layer(l, bufs[l % 2], bufs[(l + 1) % 2], stream=stream)),
                     ("parts", lambda l: (dec.layer_part(1, l, bufs[l % 2], bufs[(l + 1) % 2], stream=stream),
                                          dec.layer_part(2, l, bufs[l % 2], bufs[(l + 1) % 2], stream=stream)))):
        torch.cuda.synchronize()
        th = time.perf_counter()
        for _ in range(10):
            for l in range(L):
                fn(l)
        issue_us[name] = round((time.perf_counter() - th) / (10 * L) * 1e6, 1)
        torch.cuda.synchronize()
    dec.check_status()
    trace = synth.zipf_trace(4, n_tok, L, k, E, 1.1)
    missed = lfu_misses(trace, 16)
    layers_with_miss = sum(1 for t in range(n_tok) for l in range(L) if missed[t][l])
    copy_us = layers[0].pool.shape[1] / (pinned * 1e9) * 1e6
    fine_bound_us = layers_with_miss * part_us[2] * (1 - 1 / k)
    coarse_s = n_tok / runs["coarse"]["tok_s_all"]
    rng = np.random.default_rng(np.random.SeedSequence([4, 7]))
    perm = np.stack([rng.permutation(E) for _ in range(L)])
    trace_pl = np.stack([perm[l][trace[:, l]] for l in range(L)], axis=1).astype(np.int32)
    missed_pl = lfu_misses(trace_pl, 16)
    out = {"study": "expert cache: cross-layer prefetch and overlap granularity",
           "trace": f"Zipf(1.1) forced routing, {n_tok} tokens x {L} layers, top-{k} of {E}, 16 slots per layer",
           "overlap": {kk: {m: runs[kk][m] for m in ("tok_s_all", "tok_s_warm", "hit_rate_all", "h2d_GBps_effective_warm",
                                                     "host_issue_us_per_layer", "wall_us_per_layer")}
                       for kk in runs},
           "pinned_copy_GBps": round(pinned, 2), "record_copy_us": round(copy_us, 1),
           "part_us": {"router_shared": round(part_us[1], 2), "routed_combine": round(part_us[2], 2)},
           "host_issue_us_per_layer_no_copies": issue_us,
           "fine_bound": {"layers_with_a_miss": layers_with_miss,
                          "hideable_us_total": round(fine_bound_us, 1),
                          "tok_s_if_all_hidden": round(n_tok / max(1e-9, coarse_s - fine_bound_us * 1e-6), 2)},
           "predictors_same_ranks": predictor_stats(trace, missed),
           "predictors_per_layer_ranks": predictor_stats(trace_pl, missed_pl)}
    print(json.dumps(out), flush=True)


def pinned_copy_gbps(reps=3):
    """A plain pinned host -> device copy of 1 GiB: the host link's practical rate, the reference for the
    expert cache's copies."""
    import torch

    ref_h = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    ref_d = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    ref_d.copy_(ref_h, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        ref_d.copy_(ref_h, non_blocking=True)
    e1.record()
    e1.synchronize()
    gbps = reps * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del ref_h, ref_d
    return gbps


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cache_hits_vs_oracle(streamed):
    """The streamed run's per-layer cache hits against the oracle's LFU simulation of the same trace (every
    token, every layer): they must be equal."""
    import numpy as np
    import synth
    from oracle import moe

    a = streamed["trace_args"]
    trace = synth.zipf_trace(a["seed"], a["tokens"], a["layers"], a["k"], a["experts"], a["zipf_s"])
    _, hits = moe.lfu_simulate(np.asarray(trace), a["slots"])
    sim = [int(v) for v in hits.sum(axis=0)]
    equal = sim == streamed["hits_per_layer"]
    if not equal:
        log(f"expert cache hits differ from the oracle's LFU simulation: gpu {streamed['hits_per_layer']} "
            f"oracle {sim}")
    return {"tokens": a["tokens"], "layers": a["layers"], "hits_gpu": sum(streamed["hits_per_layer"]),
            "hits_oracle": sum(sim), "per_layer_equal": equal}


def oracle_leg(shape, layers, cfg, tokens, n_sample, st_layers, xout_graph=None):
    """The CPU oracle on a bounded sample of the timed tokens, and the parity of the GPU's results on them.

    The GPU runs the sampled tokens layer by layer (the single-layer launch, which equals the stack launch bit
    for bit) and keeps every layer's input, normalized activation, routing and logits.  The oracle (float64;
    its expert FFN in C, the experts of a layer on a thread pool) then evaluates every layer of every sampled
    token on the GPU's input to that layer (teacher forcing), once with all host cores (timed: the value) and
    for the first token over `st_layers` layers with one thread (timed, scaled to 30 layers)."""
    import numpy as np
    import torch
    import synth
    from bit_quantized_expert_int8_amd import decoder
    from oracle import fast
    from oracle import moe

    L = len(layers)
    toks = list(range(0, len(tokens), max(1, len(tokens) // n_sample)))[:n_sample]
    dec = decoder.MoEDecoder(shape, layers, T=1, mode="layer", record_u=True)
    X = np.zeros((L + 1, len(toks), cfg.d))
    U = np.zeros((L, len(toks), cfg.d))
    IDS = np.zeros((L, len(toks), cfg.k), dtype=np.int64)
    LG = np.zeros((L, len(toks), cfg.n_experts))
    f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)   # noqa: E731
    for j, tok in enumerate(toks):
        x = tokens[tok].clone()
        X[0, j] = f64(x)[0]
        for l in range(L):
            out = torch.empty_like(x)
            dec.layer(l, x, out)
            torch.cuda.synchronize()
            U[l, j], IDS[l, j], LG[l, j], X[l + 1, j] = f64(dec.u_all[l])[0], dec.ids_all[l].cpu().numpy()[0], \
                dec.logits_all[l].cpu().numpy()[0], f64(out)[0]
            x = out
    dec.check_status()
    threads = fast.default_threads()
    t0 = time.perf_counter()
    res = [fast.layer_tokens(cfg, l, X[l], IDS[l], threads=threads) for l in range(L)]
    t_all = time.perf_counter() - t0
    t0 = time.perf_counter()
    for l in range(st_layers):
        fast.layer_tokens(cfg, l, X[l, :1], IDS[l, :1], threads=1)
    t_one = time.perf_counter() - t0
    # parity of the sampled tokens
    exact = ties = 0
    worst = net = lg_err = 0.0
    for l in range(L):
        rw, rs = synth.router_int8(cfg.weight_cfg, l, cfg.n_experts, cfg.d)
        for j in range(len(toks)):
            r = res[l][j]
            lg = moe.router_logits(rw, rs, U[l, j])
            lg_err = max(lg_err, float(np.abs(LG[l, j] - lg).max() / max(1.0, np.abs(lg).max())))
            order = np.lexsort((np.arange(cfg.n_experts), -lg))
            if lg[order[cfg.k - 1]] - lg[order[cfg.k]] > 1e-3:
                exact += int(list(IDS[l, j]) == list(order[:cfg.k]))
            else:
                ties += 1
            got = X[l + 1, j]
            worst = max(worst, float(np.abs(got - r.x_next).max() / np.abs(r.x_next).max()))
            _, E = np.frexp(np.abs(r.x_next))
            ulp = np.where(r.x_next != 0, np.ldexp(1.0, E - 8), 0.0)
            excess = max(float((np.abs(got - r.x_next) - ulp).max()), 0.0)
            net = max(net, excess / np.abs(r.out - X[l, j]).max())
    n = L * len(toks)
    same = None
    if xout_graph is not None:   # the timed launch's output for the last sampled token equals the layer chain's
        same = bool(np.array_equal(xout_graph, X[L, -1]))
    cpu = {"value": len(toks) / t_all, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{len(toks)} of the {len(tokens)} timed tokens through all {L} layers, teacher-forced on the "
                     f"GPU's per-layer inputs ({t_all:.1f} s with {threads} threads; float64, expert FFN in C, weights "
                     f"drawn from the seeded generator and encoded inside the timed region)",
           "single_thread_value": 1.0 / (t_one / st_layers * L),
           "single_thread_sample": f"token {toks[0]} through layers 0-{st_layers - 1} with 1 thread ({t_one:.1f} s), "
                                   f"scaled to {L} layers",
           "nproc": os.cpu_count(), "cpu_model": cpu_model()}
    parity = {"tokens": len(toks), "layers": L, "topk_exact": exact, "topk_compared": n - ties, "near_ties": ties,
              "max_rel_err": round(worst, 5), "moe_branch_err_beyond_rounding": round(net, 6),
              "max_logit_err": float(f"{lg_err:.2e}"), "bar": "top-k exact when the 8th/9th gap > 1e-3; "
              "max relative error <= 1e-2", "timed_launch_equals_layer_chain": same}
    return cpu, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--mode", choices=("stack", "layer"), default="stack",
                    help="stack: one moe_decode_stack launch per token; layer: one moe_decode_layer launch per layer")
    ap.add_argument("--roofline-reps", type=int, default=20)
    ap.add_argument("--cpu-tokens", type=int, default=16, help="timed tokens the oracle leg checks (all layers)")
    ap.add_argument("--cpu-single-layers", type=int, default=10, help="layers of the one-thread oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the batched and streamed measurements")
    ap.add_argument("--stream-tokens", type=int, default=512)
    ap.add_argument("--copy-streams", type=int, default=4,
                    help="streams the expert cache's copies alternate over (4: the overlap schedule's best of 1-8)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one plain device-to-device copy of this many MiB (a reference for the HBM "
                         "traffic counters of a profiled run)")
    ap.add_argument("--study", choices=("prefetch", "lmhead"), default=None,
                    help="instead of the bench line: the expert-cache study (prefetch: cross-layer prefetch, overlap "
                         "granularity) or the LM-head GEMV's duration over sustained launches (lmhead)")
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
    if args.study == "prefetch":
        prefetch_study(args)
        return
    if args.study == "lmhead":
        lm_head_drift()
        return
    t_build = time.perf_counter()
    shape, layers = build_stack(cfg, args.layers)
    torch.cuda.synchronize()
    t_build = time.perf_counter() - t_build
    log(f"built {args.layers} layers in {t_build:.1f} s")
    dec = decoder.MoEDecoder(shape, layers, T=1, mode=args.mode)

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
    dec.check_status()      # every bounded wait inside the timed launches completed
    log(f"timed {args.steps} steps: {tok_s:.1f} tokens/s")

    if args.calibration_copy_mib:
        src = torch.empty(args.calibration_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    nbytes = layer_bytes(cfg)
    lay_dur, lay_launches = time_layer_kernel(dec, xin, args.roofline_reps)
    if args.mode == "stack":
        dur, launches = time_stack_kernel(dec, xin, args.roofline_reps)
        per_launch = nbytes * args.layers
        kname = (f"decode_stack_kernel (moe_decode_stack: the {args.layers} layers of one token in one launch; per "
                 "layer RMSNorm, int8 router + top-8, 8 routed + shared 4-bit expert FFNs, combine + residual)")
    else:
        dur, launches, per_launch = lay_dur, lay_launches, nbytes
        kname = ("decode_stack_kernel (moe_decode_layer: RMSNorm, int8 router + top-8, 8 routed + shared 4-bit "
                 "expert FFNs, combine + residual, one launch per layer)")
    dec.check_status()
    achieved = per_launch / dur / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": kernel_traffic(args.mode), "kernel": kname,
                "bytes_per_launch": per_launch, "avg_launch_us": round(dur * 1e6, 3), "launches_timed": launches,
                "per_layer_us": round(dur / (args.layers if args.mode == "stack" else 1) * 1e6, 3)}
    log(f"roofline launch: {dur * 1e6:.1f} us")
    split = time_split_kernels(dec, xin, args.roofline_reps)
    split["layer_launch_us"] = round(lay_dur * 1e6, 3)
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
           "decode_mode": dec.mode, "split_kernels_us": split, "hbm_read_2GiB": measure_hbm_read()}
    if not args.no_extras:
        out["batched"] = measure_batched(shape, layers, cfg, tokens.reshape(n_tok, cfg.d), 20, 3)
        log(f"batched: {out['batched']['tok_s']} tokens/s")
        out["prefill_chunk_128"] = measure_batched(shape, layers, cfg, tokens.reshape(n_tok, cfg.d), 8, 2, T=128)
        log(f"prefill chunk: {out['prefill_chunk_128']['tok_s']} tokens/s")
        out["lm_head_q4_gemv"] = measure_lm_head()
        log(f"lm head: {out['lm_head_q4_gemv']['achieved_GBps']} GB/s")
        pinned = pinned_copy_gbps()
        host = pinned_pools(layers)
        out["streamed"] = measure_streamed(shape, layers, cfg, dec, args.stream_tokens, overlap=True,
                                           copy_streams=args.copy_streams, pinned_gbps=pinned, host=host)
        log(f"streamed: {out['streamed']['tok_s_all']} tokens/s")
        base = measure_streamed(shape, layers, cfg, dec, args.stream_tokens // 2, overlap=False,
                                copy_streams=args.copy_streams, pinned_gbps=pinned, host=host)
        del host
        out["streamed"]["without_overlap"] = {kk: base[kk] for kk in ("tokens", "tok_s_all", "tok_s_warm",
                                                                     "h2d_GBps_effective_warm")}
    if not args.no_cpu_baseline:
        # the timed launch's output for the last token the oracle leg samples
        toks = list(range(0, n_tok, max(1, n_tok // args.cpu_tokens)))[:args.cpu_tokens]
        xin.copy_(tokens[toks[-1]])
        g.replay()
        torch.cuda.synchronize()
        xo = xout.float().cpu().numpy().astype(np.float64)[0]
        log("oracle leg")
        out["cpu_baseline"], out["parity"] = oracle_leg(shape, layers, cfg, tokens, args.cpu_tokens,
                                                        args.cpu_single_layers, xout_graph=xo)
        if "streamed" in out:
            out["parity"]["expert_cache"] = cache_hits_vs_oracle(out["streamed"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
