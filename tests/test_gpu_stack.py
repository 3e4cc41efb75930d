"""GPU checks of the stacked decode, graph replays, batched tokens and the expert cache (MI355X).

The stack is checked by per-layer teacher forcing: the oracle runs layer l on the GPU's bf16 input to
layer l (a near-tie that flips one expert would otherwise change every later layer)."""
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
    dec = decoder.MoEDecoder(H.shape_of(cfg), layers, T=1)
    return cfg, layers, dec


def _run_layers_eager(dec, x0, n):
    xs = [x0.clone()]
    for l in range(n):
        out = torch.empty_like(x0)
        dec.layer(l, xs[-1], out)
        xs.append(out)
    torch.cuda.synchronize()
    return xs


def test_stack_teacher_forced_sampled_layers(stack):
    """30 layers, d=2816, 128 experts, top-8: layers 0, 13 and 29 of one token against the oracle on the
    GPU's own layer inputs (norm output, top-k under the gap rule, layer output)."""
    cfg, layers, dec = stack
    x0 = H.token_batch(cfg, [7])
    xs = _run_layers_eager(dec, x0, cfg.n_layers)
    for l in (0, 13, 29):
        orc = oin.oracle_layer(cfg, l, cache_experts=16)
        x_in = _bf16_to_f64(xs[l])[0]
        # the GPU's routing of layer l: rerun that layer alone to read its ids
        tmp = torch.empty_like(x0)
        dec.layer(l, xs[l], tmp)
        torch.cuda.synchronize()
        ids = dec.ids_all[l].cpu().numpy()[0]
        u_ref = moe.f64_round_to_bf16(moe.rms_norm(x_in, np.ones(cfg.d), 1e-6))
        if dec.mode not in ("layer", "stack"):   # the single-launch kernels keep u internal
            u_gpu = _bf16_to_f64(dec.u)[0]
            assert H.max_rel_err(u_gpu, u_ref) <= 2 ** -7
        lg = moe.router_logits(orc.router_w, orc.router_s, u_ref)
        assert H.topk_consistent(ids.tolist(), lg, cfg.k), f"layer {l}"
        _, res, x_next = moe.stack_layer_step(orc, x_in, cfg.k, forced_ids=ids)
        got = _bf16_to_f64(xs[l + 1])[0]
        err = H.max_rel_err(got, x_next)
        # per element: the MoE branch within TOL of its own magnitude, plus one bf16 ulp of the rounded output
        moe_ref = res.out - x_in
        allowed = TOL * np.abs(moe_ref).max() + 2.0 ** -8 * np.abs(x_next)
        worst = float((np.abs(got - x_next) / allowed).max())
        print(f"stack layer {l}: output rel err {err:.2e}, per-element error / allowance {worst:.2f}")
        assert err <= TOL and worst <= 1.0


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
    """The batched configuration: 32 tokens through one d=2816 layer; four sampled tokens vs the oracle."""
    cfg = synth.BATCHED
    dev = H.device_layer(cfg, 0)
    orc = oin.oracle_layer(cfg, 0, cache_experts=40)
    T = cfg.n_tokens
    dec = decoder.MoEDecoder(H.shape_of(cfg), [dev], T=T)
    x = H.token_batch(cfg, range(T))
    out = torch.empty_like(x)
    dec.layer(0, x, out)
    torch.cuda.synchronize()
    got, ids = _bf16_to_f64(out), dec.ids_all[0].cpu().numpy()
    for t in (0, 11, 22, 31):
        u = oin.token_input(cfg, t)
        lg = moe.router_logits(orc.router_w, orc.router_s, u)
        assert H.topk_consistent(ids[t].tolist(), lg, cfg.k)
        ref = moe.moe_layer(orc, u, cfg.k, forced_ids=ids[t])
        assert H.max_rel_err(got[t], ref.out) <= TOL, f"token {t}"


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
