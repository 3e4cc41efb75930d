"""GPU checks of the stacked decode, graph replays, batched tokens and the expert cache (MI355X).

The stack is checked by per-layer teacher forcing: the oracle runs layer l on the GPU's bf16 input to
layer l (a near-tie that flips one expert would otherwise change every later layer)."""
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from oracle import moe  # noqa: E402
from oracle import inputs as oin  # noqa: E402
from bit_quantized_expert_int8_amd import decoder, moeq4 as q  # noqa: E402
import gpu_helpers as H  # noqa: E402

TOL = 1e-2


def _bf16_to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def stack():
    cfg = synth.STACK
    layers = [H.device_layer(cfg, l) for l in range(cfg.n_layers)]
    dec = decoder.MoEDecoder(H.shape_of(cfg), layers, T=1, record_u=True)
    return cfg, layers, dec


def _run_layers_eager(dec, x0, n):
    xs = [x0.clone()]
    for l in range(n):
        out = torch.empty_like(x0)
        dec.layer(l, xs[-1], out)
        xs.append(out)
    torch.cuda.synchronize()
    return xs


def _stack_per_layer(dec, cfg, toks):
    """Run each token through every layer eagerly, keeping every layer's input, normalized activation,
    routing and logits (the GPU's residual stream, for teacher forcing)."""
    L, n = cfg.n_layers, len(toks)
    X = np.zeros((L + 1, n, cfg.d))
    U = np.zeros((L, n, cfg.d))
    IDS = np.zeros((L, n, cfg.k), dtype=np.int64)
    LG = np.zeros((L, n, cfg.n_experts))
    for j, tok in enumerate(toks):
        x = H.token_batch(cfg, [tok])
        X[0, j] = _bf16_to_f64(x)[0]
        for l in range(L):
            out = torch.empty_like(x)
            dec.layer(l, x, out)
            torch.cuda.synchronize()
            U[l, j] = _bf16_to_f64(dec.u_all[l])[0]
            IDS[l, j] = dec.ids_all[l].cpu().numpy()[0]
            LG[l, j] = dec.logits_all[l].cpu().numpy()[0]
            X[l + 1, j] = _bf16_to_f64(out)[0]
            x = out
    dec.check_status()
    return X, U, IDS, LG


def test_stack_teacher_forced_every_layer(stack):
    """The 30-layer stack (d=2816, 128 experts top-8, shared 2816, RMSNorm + residual, bf16) on all 256 of
    its tokens, every layer against the oracle on the GPU's own input to that layer (teacher forcing: a
    near-tie that flips one expert would otherwise change every later layer).  Per layer and token: the
    kernel's normalized activation within one bf16 step of the oracle's; the oracle's router on the kernel's
    u gives the kernel's logits within 1e-4 and its ranking (exact ids when the 8th/9th gap exceeds 1e-3);
    the layer output within the parity bar of the oracle on that routing."""
    from oracle import fast
    cfg, layers, dec = stack
    toks = list(range(cfg.n_tokens))
    X, U, IDS, LG = _stack_per_layer(dec, cfg, toks)
    exact = ties = 0
    worst_err = worst_allow = worst_lg = worst_net = 0.0
    t0 = time.perf_counter()
    for l in range(cfg.n_layers):
        rw, rs = synth.router_int8(cfg.weight_cfg, l, cfg.n_experts, cfg.d)
        res = fast.layer_tokens(cfg, l, X[l], IDS[l])
        for j, tok in enumerate(toks):
            r = res[j]
            assert H.bf16_steps(U[l, j], r.u) <= 1, f"layer {l} token {tok}: u"
            lg = moe.router_logits(rw, rs, U[l, j])
            worst_lg = max(worst_lg, float(np.abs(LG[l, j] - lg).max() / max(1.0, np.abs(lg).max())))
            order = np.lexsort((np.arange(cfg.n_experts), -lg))
            if lg[order[cfg.k - 1]] - lg[order[cfg.k]] > 1e-3:
                exact += int(list(IDS[l, j]) == list(order[:cfg.k]))
            else:
                ties += 1
            assert H.topk_consistent(IDS[l, j].tolist(), lg, cfg.k), f"layer {l} token {tok}: {IDS[l, j]}"
            got = X[l + 1, j]
            moe_max = np.abs(r.out - X[l, j]).max()
            worst_err = max(worst_err, H.max_rel_err(got, r.x_next))
            # per element: the MoE branch within TOL of its own magnitude, plus one bf16 step of the output
            allowed = TOL * moe_max + H.bf16_ulp(r.x_next)
            worst_allow = max(worst_allow, float((np.abs(got - r.x_next) / allowed).max()))
            worst_net = max(worst_net, H.net_err(got, r.x_next, moe_max))
    n = cfg.n_layers * len(toks)
    print(f"stack, {len(toks)} tokens x {cfg.n_layers} layers: top-k exact {exact}/{n - ties} (near ties {ties}), "
          f"max rel err {worst_err:.2e}, error / allowance {worst_allow:.2f}, MoE-branch error beyond one output "
          f"rounding {worst_net:.2e}, logit err {worst_lg:.1e}, oracle {time.perf_counter() - t0:.1f} s")
    assert worst_lg <= 1e-4
    assert worst_err <= TOL and worst_allow <= 1.0
    assert worst_net <= H.REGRESSION["stack_layer"]


def test_graph_replays_match_eager(stack):
    """The whole 30-layer step captured in one HIP graph: every replay, with eager work in between,
    reproduces the eager result bit for bit (the kernels are deterministic)."""
    cfg, layers, dec = stack
    x0 = H.token_batch(cfg, [3])
    eager = _run_layers_eager(dec, x0, cfg.n_layers)[-1].clone()
    xin, xout = x0.clone(), torch.empty_like(x0)
    g = dec.capture(xin, xout)
    for r in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xout, eager), f"replay {r}"
        _run_layers_eager(dec, H.token_batch(cfg, [100 + r]), 2)       # unrelated eager work in between
    xin.copy_(H.token_batch(cfg, [5]))
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(xout, _run_layers_eager(dec, H.token_batch(cfg, [5]), cfg.n_layers)[-1])


def test_batched_tokens_match_single_token(stack):
    """32 tokens in one call (the batched configuration, grouped by expert on the matrix cores) match each
    token run alone through the same library calls (norm + router, then expert GEMVs with the combine), on
    layer 0, within the parity bar (max relative error 1e-2)."""
    cfg, layers, _ = stack
    T = 32
    decT = decoder.MoEDecoder(H.shape_of(cfg), layers[:1], T=T)
    dec1 = decoder.MoEDecoder(H.shape_of(cfg), layers[:1], T=1, mode="fused")
    assert decT.mode == "fused"
    x = H.token_batch(cfg, range(T))
    out = torch.empty_like(x)
    decT.layer(0, x, out)
    torch.cuda.synchronize()
    for t in (0, 9, 31):
        o1 = torch.empty_like(x[t:t + 1])
        dec1.layer(0, x[t:t + 1].contiguous(), o1)
        torch.cuda.synchronize()
        err = H.max_rel_err(H.to_f64(out[t]), H.to_f64(o1[0]))
        assert err <= 1e-2, f"token {t}: {err:.3e}"


def test_batched_layer_vs_oracle():
    """The batched configuration: 32 tokens through one d=2816 layer in one call (grouped by expert, products
    on the matrix cores); every token's logits, routing and output against the oracle."""
    from oracle import fast
    cfg = synth.BATCHED
    dev = H.device_layer(cfg, 0)
    T = cfg.n_tokens
    dec = decoder.MoEDecoder(H.shape_of(cfg), [dev], T=T)
    x = H.token_batch(cfg, range(T))
    out = torch.empty_like(x)
    dec.layer(0, x, out)
    torch.cuda.synchronize()
    got, ids, lgs = _bf16_to_f64(out), dec.ids_all[0].cpu().numpy(), dec.logits_all[0].cpu().numpy()
    rw, rs = synth.router_int8(cfg.weight_cfg, 0, cfg.n_experts, cfg.d)
    X = np.stack([oin.token_input(cfg, t) for t in range(T)])
    res = fast.layer_tokens(cfg, 0, X, ids)
    worst = net = 0.0
    for t in range(T):
        lg = moe.router_logits(rw, rs, X[t])
        assert np.abs(lgs[t] - lg).max() <= 1e-4 * max(1.0, np.abs(lg).max()), f"token {t}"
        assert H.topk_consistent(ids[t].tolist(), lg, cfg.k), f"token {t}"
        worst = max(worst, H.max_rel_err(got[t], res[t].out))
        net = max(net, H.net_err(got[t], res[t].x_next, np.abs(res[t].out).max()))
    print(f"batched layer, {T} tokens: max rel err {worst:.2e}, error beyond one output rounding {net:.2e}")
    assert worst <= TOL and net <= H.REGRESSION["batched"]


def test_expert_cache_streaming_matches_resident_and_oracle_policy():
    """Two d=2816 layers with their 128 experts in pinned host memory and 16 HBM slots each, routing forced
    by a Zipf(1.1) trace: slot contents equal the host records, layer outputs equal the all-resident run
    with the same forced ids bit for bit, and hit counts equal the oracle's LFU simulation."""
    cfg = synth.STREAMED
    L, T, k, E, n_slots = 2, 40, cfg.k, cfg.n_experts, cfg.n_slots
    layers = [H.device_layer(cfg, l) for l in range(L)]
    shape = H.shape_of(cfg)
    rb = layers[0].pool.shape[1]
    host = [lay.pool.cpu().pin_memory() for lay in layers]
    slots = [torch.empty((n_slots, rb), dtype=torch.uint8, device="cuda") for _ in range(L)]
    cache = q.moe_expert_cache_create(L, E, n_slots, rb, [h.data_ptr() for h in host], [s.data_ptr() for s in slots])
    trace = synth.zipf_trace(4, T, L, k, E, 1.1)
    sim_slots, sim_hits = moe.lfu_simulate(trace, n_slots)
    dec = decoder.MoEDecoder(shape, layers, T=1)
    slot_pools = [q.pool(s, rb, n_slots, cfg.d, cfg.F, shape.sb_dtype) for s in slots]
    copy_stream = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    ready = [torch.cuda.Event() for _ in range(L)]
    freed = [torch.cuda.Event() for _ in range(L)]
    for ev in ready + freed:            # torch creates the HIP event on first record: make the handles exist
        ev.record(copy_stream)
    copy_stream.synchronize()
    assert all(ev.cuda_event for ev in ready + freed)
    slot_ids = torch.empty((L, k), dtype=torch.int32, device="cuda")
    forced = torch.from_numpy(trace.astype(np.int32)).cuda()
    try:
        for t in range(T):
            x = H.token_batch(cfg, [t])
            for l in range(L):
                q.expert_cache_stage(cache, l, trace[t, l].tolist(), slot_ids[l], copy_stream,
                                     freed[l] if t > 0 else None, ready[l])
                compute.wait_event(ready[l])
                out_c, out_r = torch.empty_like(x), torch.empty_like(x)
                dec.layer(l, x, out_c, forced_ids=forced[t, l].reshape(1, k), routed_pool=slot_pools[l],
                          ids=slot_ids[l].reshape(1, k))
                freed[l].record(compute)
                dec.layer(l, x, out_r, forced_ids=forced[t, l].reshape(1, k))
                torch.cuda.synchronize()
                assert slot_ids[l].cpu().numpy().tolist() == sim_slots[t, l].tolist()
                assert torch.equal(out_c, out_r), f"token {t} layer {l}"
                x = out_r
        for l in range(L):
            h, m, b = q.moe_expert_cache_stats(cache, l)
            assert h == int(sim_hits[:, l].sum()) and h + m == T * k and b == m * rb
            held = q.moe_expert_cache_slots(cache, l, n_slots)
            for s, e in enumerate(held):
                if e >= 0:
                    assert torch.equal(slots[l][s], layers[l].pool[e]), f"layer {l} slot {s}"
    finally:
        q.moe_expert_cache_destroy(cache)


def test_expert_cache_run_ahead_matches_resident():
    """The host stages and launches every layer of every token without waiting for the device, so copies,
    slot ids and layer launches queue far ahead; the trace repeats a token's experts (every id of the next
    token hits, so that layer copies nothing but still rewrites its slot ids) and mixes in Zipf tokens.
    Every layer output equals the all-resident run with the same forced ids bit for bit."""
    cfg = synth.STREAMED
    L, T, k, E, n_slots = 2, 24, cfg.k, cfg.n_experts, cfg.n_slots
    layers = [H.device_layer(cfg, l) for l in range(L)]
    shape = H.shape_of(cfg)
    rb = layers[0].pool.shape[1]
    host = [lay.pool.cpu().pin_memory() for lay in layers]
    slots = [torch.empty((n_slots, rb), dtype=torch.uint8, device="cuda") for _ in range(L)]
    cache = q.moe_expert_cache_create(L, E, n_slots, rb, [h.data_ptr() for h in host], [s.data_ptr() for s in slots])
    trace = synth.zipf_trace(8, T, L, k, E, 1.1)
    for t in range(1, T, 3):
        trace[t] = trace[t - 1][:, ::-1]          # all hits, slot ids in another order
    dec = decoder.MoEDecoder(shape, layers, T=1)
    slot_pools = [q.pool(s, rb, n_slots, cfg.d, cfg.F, shape.sb_dtype) for s in slots]
    copy_stream = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    ready = [torch.cuda.Event() for _ in range(L)]
    freed = [torch.cuda.Event() for _ in range(L)]
    for ev in ready + freed:
        ev.record(copy_stream)
    copy_stream.synchronize()
    slot_ids = torch.empty((L, k), dtype=torch.int32, device="cuda")
    forced = torch.from_numpy(np.ascontiguousarray(trace).astype(np.int32)).cuda()
    xs = H.token_batch(cfg, range(T))
    outs = torch.empty((T, L, 1, cfg.d), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    try:
        for t in range(T):
            x = xs[t:t + 1]
            for l in range(L):
                q.expert_cache_stage(cache, l, trace[t, l].tolist(), slot_ids[l], copy_stream,
                                     freed[l] if t > 0 else None, ready[l])
                compute.wait_event(ready[l])
                dec.layer(l, x, outs[t, l], forced_ids=forced[t, l].reshape(1, k), routed_pool=slot_pools[l],
                          ids=slot_ids[l].reshape(1, k))
                freed[l].record(compute)
                x = outs[t, l]
        torch.cuda.synchronize()
        dec.check_status()
        for t in range(T):
            x = xs[t:t + 1]
            for l in range(L):
                ref = torch.empty_like(x)
                dec.layer(l, x, ref, forced_ids=forced[t, l].reshape(1, k))
                torch.cuda.synchronize()
                assert torch.equal(outs[t, l], ref), f"token {t} layer {l}"
                x = ref
        sim_slots, sim_hits = moe.lfu_simulate(trace, n_slots)
        for l in range(L):
            assert q.moe_expert_cache_stats(cache, l)[0] == int(sim_hits[:, l].sum())
    finally:
        q.moe_expert_cache_destroy(cache)
