"""GPU checks of moe_decode_layer, the single-launch MoE layer (MI355X): against the oracle, against itself
across calls on one workspace (its counters must come back to zero, its error flag must stay clear), with
forced routing and cache-slot indirection, and on the small fp32 configuration without norm."""
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


@pytest.fixture(scope="module")
def stack_layer():
    cfg = synth.STACK
    return cfg, H.device_layer(cfg, 0), H.shape_of(cfg)


def _pools(cfg, dev, shape, shared=True):
    rp = q.pool(dev.pool, dev.pool.shape[1], shape.n_experts, shape.d, shape.F, shape.sb_dtype)
    sp = q.pool(dev.shared, dev.shared.shape[1], 1, shape.d, shape.S, shape.sb_dtype) if shared else None
    return rp, sp


def _ws(cfg, shared=True):
    b = q.moe_decode_layer_workspace_bytes(cfg.d, cfg.n_experts, cfg.k, cfg.F, cfg.S if shared else 0)
    return torch.zeros(b, dtype=torch.uint8, device="cuda"), b


def _run(cfg, dev, shape, x, ws, ws_b, gamma, residual, forced=None, routed=None, gemv_ids=None, shared=True, u=None,
         k=None, router_w=None, router_s=None):
    rp, sp = _pools(cfg, dev, shape, shared)
    k = k or cfg.k
    ids = torch.full((k,), -5, dtype=torch.int32, device="cuda")
    w = torch.empty((k,), dtype=torch.float32, device="cuda")
    lg = torch.empty((cfg.n_experts,), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    xdt = q.MOE_BF16 if cfg.x_bf16 else q.MOE_F32
    q.moe_decode_layer(x, xdt, gamma, 1e-6, residual, dev.router_w if router_w is None else router_w,
                       dev.router_s if router_s is None else router_s, cfg.n_experts, k, forced,
                       routed or rp, gemv_ids, sp, shape.act, ids, w, lg, out, ws, ws_b, u=u)
    return ids, w, lg, out


def _check_clean(ws, cfg, calls):
    """Word 0 (sticky error flag) clear; in the synchronisation region (moe_decode_layer_sync_bytes) every
    counter back to zero and every flag zero or holding the number of calls made on the workspace."""
    torch.cuda.synchronize()
    n = q.moe_decode_layer_sync_bytes(cfg.d, cfg.k)
    assert 0 < n < ws.numel()
    words = ws[:n].view(torch.int32).cpu().numpy()
    assert words[0] == 0, "a wait inside the layer kernel ran out"
    bad = np.nonzero((words != 0) & (words != calls))[0]
    assert bad.size == 0, f"synchronisation words left at {words[bad[:8]]} (call {calls}) at {bad[:8]}"
    assert (words == calls).any(), "no flag carries this call's number"


@pytest.mark.parametrize("gamma_ones", [True, False])
def test_decode_layer_vs_oracle(stack_layer, gamma_ones):
    """One d=2816 layer (RMSNorm, router, 8 of 128 experts + shared, residual) on eight tokens, one call
    each on one workspace.  The kernel's own normalized activation u (its optional output) is within one
    bf16 step of the oracle's and equals moe_rmsnorm's bit for bit (the same summation order); the oracle's
    router run on that u gives the kernel's logits within 1e-4 and
    ranks them like the kernel (exact ids when the 8th/9th gap exceeds 1e-3); the gate weights are the
    softmax of the logits; the output is within the parity bar of the oracle on the kernel's routing."""
    cfg, dev, shape = stack_layer
    gamma_np = synth.rms_gamma(cfg.weight_cfg, 0, cfg.d, ones=gamma_ones)
    gamma = torch.from_numpy(gamma_np).cuda()
    orc = oin.oracle_layer(cfg, 0, cache_experts=48)
    orc.gamma = gamma_np.astype(np.float64)
    ws, ws_b = _ws(cfg)
    u_dev = torch.empty((cfg.d,), dtype=torch.bfloat16, device="cuda")
    for call, tok in enumerate((0, 5, 77, 200, 31, 32, 129, 255), 1):
        x = H.token_batch(cfg, [tok])[0]
        ids, w, lg, out = _run(cfg, dev, shape, x, ws, ws_b, gamma, 1, u=u_dev)
        _check_clean(ws, cfg, call)
        x64 = H.to_f64(x)
        u_ref = moe.f64_round_to_bf16(moe.rms_norm(x64, orc.gamma, 1e-6))
        u_gpu = H.to_f64(u_dev)
        assert H.bf16_steps(u_gpu, u_ref) <= 1, f"token {tok}: u off by more than one bf16 step"
        u_sep = torch.empty_like(u_dev)
        q.moe_rmsnorm(x, q.MOE_BF16, gamma, 1e-6, 1, cfg.d, u_sep, q.MOE_BF16)
        torch.cuda.synchronize()
        assert torch.equal(u_dev, u_sep), f"token {tok}: the layer's u differs from moe_rmsnorm's"
        ref_lg = moe.router_logits(orc.router_w, orc.router_s, u_gpu)
        got_lg = lg.cpu().numpy().astype(np.float64)
        assert np.abs(got_lg - ref_lg).max() <= 1e-4 * max(1.0, np.abs(ref_lg).max()), f"token {tok}"
        ids_np = ids.cpu().numpy()
        assert H.topk_consistent(ids_np.tolist(), ref_lg, cfg.k), f"token {tok}: {ids_np}"
        assert np.allclose(w.cpu().numpy(), moe.gate_weights(got_lg, ids_np), rtol=0, atol=1e-6)
        _, res, x_next = moe.stack_layer_step(orc, x64, cfg.k, forced_ids=ids_np)
        got = H.to_f64(out)
        moe_max = np.abs(res.out - x64).max()
        allowed = TOL * moe_max + H.bf16_ulp(x_next)
        worst = float((np.abs(got - x_next) / allowed).max())
        err = H.max_rel_err(got, x_next)
        net = H.net_err(got, x_next, moe_max)
        print(f"layer kernel token {tok}: rel err {err:.2e}, error / allowance {worst:.2f}, MoE-branch error "
              f"beyond one output rounding {net:.2e}")
        assert err <= TOL and worst <= 1.0
        assert net <= H.REGRESSION["layer_kernel"], f"token {tok}: {net:.2e} above the measured-error bound"


def test_decode_layer_repeatable_on_one_workspace(stack_layer):
    """Five calls in a row on one workspace equal the same calls on fresh workspaces, bit for bit."""
    cfg, dev, shape = stack_layer
    gamma = torch.ones(cfg.d, dtype=torch.float32, device="cuda")
    ws, ws_b = _ws(cfg)
    for call, tok in enumerate((3, 4, 3, 9, 4), 1):
        x = H.token_batch(cfg, [tok])[0]
        ids, w, lg, out = _run(cfg, dev, shape, x, ws, ws_b, gamma, 1)
        fresh, fb = _ws(cfg)
        ids2, w2, lg2, out2 = _run(cfg, dev, shape, x, fresh, fb, gamma, 1)
        _check_clean(ws, cfg, call)
        _check_clean(fresh, cfg, 1)
        assert torch.equal(ids, ids2) and torch.equal(w, w2) and torch.equal(lg, lg2) and torch.equal(out, out2)


def test_decode_layer_forced_and_slot_indirection(stack_layer):
    """Forced routing (a Zipf trace) with the experts read from a 16-slot pool through slot ids equals forced
    routing on the resident pool, bit for bit; ids come back as forced and weights as the softmax at them."""
    cfg, dev, shape = stack_layer
    gamma = torch.ones(cfg.d, dtype=torch.float32, device="cuda")
    trace = synth.zipf_trace(13, 3, 1, cfg.k, cfg.n_experts, 1.1)[:, 0, :]
    rb = dev.pool.shape[1]
    for t in range(3):
        forced = torch.from_numpy(trace[t].astype(np.int32)).cuda()
        slots = torch.zeros((16, rb), dtype=torch.uint8, device="cuda")
        slot_of = (np.arange(cfg.k) * 5 + 3 + t) % 16
        for i, e in enumerate(trace[t]):
            slots[slot_of[i]].copy_(dev.pool[int(e)])
        slot_pool = q.pool(slots, rb, 16, cfg.d, cfg.F, shape.sb_dtype)
        gemv_ids = torch.from_numpy(slot_of.astype(np.int32)).cuda()
        x = H.token_batch(cfg, [30 + t])[0]
        ws, ws_b = _ws(cfg)
        ids_a, w_a, _, out_a = _run(cfg, dev, shape, x, ws, ws_b, gamma, 1, forced=forced)
        ids_b, w_b, _, out_b = _run(cfg, dev, shape, x, ws, ws_b, gamma, 1, forced=forced, routed=slot_pool,
                                    gemv_ids=gemv_ids)
        _check_clean(ws, cfg, 2)
        assert ids_a.cpu().numpy().tolist() == trace[t].tolist()
        assert torch.equal(ids_a, ids_b) and torch.equal(w_a, w_b) and torch.equal(out_a, out_b), f"token {t}"


@pytest.mark.parametrize("shared", [True, False])
def test_decode_layer_tiny_no_norm_vs_oracle(shared):
    """The small configuration (d=256, 8 experts, top-2, fp32 activations and scale/bias), no norm and no
    residual, with and without the shared expert: 16 tokens against the oracle."""
    cfg = synth.TINY
    dev = H.device_layer(cfg, 0)
    shape = H.shape_of(cfg)
    orc = oin.oracle_layer(cfg, 0)
    if not shared:
        orc.shared = None
    ws, ws_b = _ws(cfg, shared)
    worst = 0.0
    for tok in range(16):
        x = H.token_batch(cfg, [tok])[0]
        ids, w, lg, out = _run(cfg, dev, shape, x, ws, ws_b, None, 0, shared=shared)
        _check_clean(ws, cfg, tok + 1)
        u = oin.token_input(cfg, tok)
        ref_lg = moe.router_logits(orc.router_w, orc.router_s, u)
        assert np.abs(lg.cpu().numpy() - ref_lg).max() <= 1e-5 * max(1.0, np.abs(ref_lg).max())
        assert H.topk_consistent(ids.cpu().numpy().tolist(), ref_lg, cfg.k)
        ref = moe.moe_layer(orc, u, cfg.k, forced_ids=ids.cpu().numpy())
        worst = max(worst, H.max_rel_err(H.to_f64(out), ref.out))
    print(f"tiny layer kernel (shared={shared}): max rel err {worst:.3e}")
    assert worst <= TOL and worst <= H.REGRESSION["tiny_layer"]


def test_decode_stack_equals_chained_layers():
    """Four d=2816 layers in one moe_decode_stack launch equal four chained moe_decode_layer calls bit for bit
    (output, and every layer's ids, weights and logits), twice in a row on one workspace; in every layer's
    synchronisation region the counters are back to zero and the flags zero or at the call number, and the
    error flag is clear."""
    cfg = synth.STACK
    L = 4
    devs = [H.device_layer(cfg, l) for l in range(L)]
    shape = H.shape_of(cfg)
    rp, sp = _pools(cfg, devs[0], shape)
    E, k, d = cfg.n_experts, cfg.k, cfg.d
    ids = torch.full((L, k), -1, dtype=torch.int32, device="cuda")
    wts = torch.zeros((L, k), dtype=torch.float32, device="cuda")
    lgs = torch.zeros((L, E), dtype=torch.float32, device="cuda")
    descs = q.stack_layers([{"router_w_dev": W.router_w, "router_scale_dev": W.router_s, "gamma_dev": W.gamma,
                             "routed_base_dev": W.pool, "shared_base_dev": W.shared, "ids_dev": ids[l],
                             "weights_dev": wts[l], "logits_dev": lgs[l]} for l, W in enumerate(devs)])
    sb = q.moe_decode_stack_workspace_bytes(L, d, E, k, cfg.F, cfg.S)
    region = q.moe_decode_layer_workspace_bytes(d, E, k, cfg.F, cfg.S)
    assert sb == L * region
    ws = torch.zeros(sb, dtype=torch.uint8, device="cuda")
    lws, lwb = _ws(cfg)
    for call, tok in enumerate((11, 12), 1):
        x = H.token_batch(cfg, [tok])[0]
        out = torch.empty_like(x)
        q.moe_decode_stack(descs, L, x, q.MOE_BF16, 1e-6, 1, E, k, rp, sp, shape.act, out, ws, sb)
        xs = x
        for l, W in enumerate(devs):
            i1, w1, g1, o1 = _run(cfg, W, shape, xs, lws, lwb, W.gamma, 1)
            torch.cuda.synchronize()
            assert torch.equal(i1, ids[l]) and torch.equal(w1, wts[l]) and torch.equal(g1, lgs[l]), f"layer {l}"
            xs = o1
        assert torch.equal(xs, out), f"token {tok}"
        words = ws.view(torch.int32)
        assert int(words[0].item()) == 0, "a wait inside the stack kernel ran out"
        n = q.moe_decode_layer_sync_bytes(d, k) // 4
        for l in range(L):
            seg = words[l * region // 4: l * region // 4 + n].cpu().numpy()
            bad = np.nonzero((seg != 0) & (seg != call))[0]
            assert bad.size == 0, f"layer {l}: synchronisation words left at {seg[bad[:8]]} (call {call})"


@pytest.mark.parametrize("shared,k", [(True, 2), (False, 2), (True, 8)])
def test_decode_stack_small_fp32_equals_chained_layers(shared, k):
    """Six layers of the small configuration (d=256, 8 experts top-2, fp32 activations and scale/bias, RMSNorm
    with a seeded gain, residual) in one moe_decode_stack launch, with and without the shared expert, top-2 and
    top-8 (every expert): the
    multi-layer instantiations for fp32 activations and without the shared expert's roles equal six chained
    moe_decode_layer calls bit for bit (output, ids, weights, logits), twice in a row on one workspace, and
    leave the error flag clear."""
    cfg = synth.TINY
    L = 6
    devs = [H.device_layer(cfg, l) for l in range(L)]
    shape = H.shape_of(cfg)
    rp, sp = _pools(cfg, devs[0], shape, shared)
    E, d = cfg.n_experts, cfg.d
    S = cfg.S if shared else 0
    gammas = [torch.from_numpy(synth.rms_gamma(cfg.weight_cfg, l, d, ones=False)).cuda() for l in range(L)]
    ids = torch.full((L, k), -1, dtype=torch.int32, device="cuda")
    wts = torch.zeros((L, k), dtype=torch.float32, device="cuda")
    lgs = torch.zeros((L, E), dtype=torch.float32, device="cuda")
    descs = q.stack_layers([{"router_w_dev": W.router_w, "router_scale_dev": W.router_s, "gamma_dev": gammas[l],
                             "routed_base_dev": W.pool, "shared_base_dev": W.shared if shared else None,
                             "ids_dev": ids[l], "weights_dev": wts[l], "logits_dev": lgs[l]}
                            for l, W in enumerate(devs)])
    sb = q.moe_decode_stack_workspace_bytes(L, d, E, k, cfg.F, S)
    ws = torch.zeros(sb, dtype=torch.uint8, device="cuda")
    lwb = q.moe_decode_layer_workspace_bytes(d, E, k, cfg.F, S)
    lws = torch.zeros(lwb, dtype=torch.uint8, device="cuda")
    for call, tok in enumerate((3, 4), 1):
        x = H.token_batch(cfg, [tok])[0]
        out = torch.empty_like(x)
        q.moe_decode_stack(descs, L, x, q.MOE_F32, 1e-6, 1, E, k, rp, sp, shape.act, out, ws, sb)
        xs = x
        for l, W in enumerate(devs):
            i1, w1, g1, o1 = _run(cfg, W, shape, xs, lws, lwb, gammas[l], 1, shared=shared, k=k)
            torch.cuda.synchronize()
            assert torch.equal(i1, ids[l]) and torch.equal(w1, wts[l]) and torch.equal(g1, lgs[l]), f"layer {l}"
            xs = o1
        assert torch.equal(xs, out), f"token {tok}"
        assert int(ws.view(torch.int32)[0].item()) == 0, "a wait inside the stack kernel ran out"


# ---------------------------------------------------------------------------------------------------
# the method's degenerate cases on the single-launch layer (small configuration: d=256, 8 experts)
# ---------------------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny_layer():
    cfg = synth.TINY
    return cfg, H.device_layer(cfg, 0), H.shape_of(cfg), oin.oracle_layer(cfg, 0)


def test_decode_layer_zero_input(tiny_layer, stack_layer):
    """x = 0: every logit is 0, so the first k ids in order are chosen with weights 1/k, and every expert
    output is exactly zero; with the norm (eps > 0) u = 0 too and the output is the residual, 0."""
    for cfg, dev, shape, gamma, residual in ((tiny_layer[0], tiny_layer[1], tiny_layer[2], None, 0),
                                             (stack_layer[0], stack_layer[1], stack_layer[2],
                                              torch.ones(stack_layer[0].d, device="cuda"), 1)):
        ws, ws_b = _ws(cfg)
        x = torch.zeros((cfg.d,), dtype=torch.bfloat16 if cfg.x_bf16 else torch.float32, device="cuda")
        ids, w, lg, out = _run(cfg, dev, shape, x, ws, ws_b, gamma, residual)
        _check_clean(ws, cfg, 1)
        assert ids.cpu().tolist() == list(range(cfg.k))
        assert np.all(lg.cpu().numpy() == 0.0)
        assert np.allclose(w.cpu().numpy(), 1.0 / cfg.k, rtol=0, atol=1e-7)
        assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("k", [1, 8])
def test_decode_layer_k_one_and_k_all(tiny_layer, k):
    """k = 1: the arg-max expert with weight exactly 1.  k = E = 8: every expert, ranked by logit (a full
    sort), weights the softmax over all logits (the textbook dense softmax MoE).  Both against the oracle."""
    cfg, dev, shape, orc = tiny_layer
    b = q.moe_decode_layer_workspace_bytes(cfg.d, cfg.n_experts, k, cfg.F, cfg.S)
    ws = torch.zeros(b, dtype=torch.uint8, device="cuda")
    worst = 0.0
    for tok in range(6):
        x = H.token_batch(cfg, [tok])[0]
        ids, w, lg, out = _run(cfg, dev, shape, x, ws, b, None, 0, k=k)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == 0
        u = oin.token_input(cfg, tok)
        ref_lg = moe.router_logits(orc.router_w, orc.router_s, u)
        ids_np, w_np = ids.cpu().numpy(), w.cpu().numpy()
        assert H.topk_consistent(ids_np.tolist(), ref_lg, k)
        if k == 1:
            assert w_np[0] == 1.0
        else:
            assert sorted(ids_np.tolist()) == list(range(cfg.n_experts))
            p = np.exp(ref_lg - ref_lg.max())
            p /= p.sum()
            assert np.allclose(w_np, p[ids_np], rtol=0, atol=1e-6)
        ref = moe.moe_layer(orc, u, k, forced_ids=ids_np)
        worst = max(worst, H.max_rel_err(H.to_f64(out), ref.out))
    print(f"tiny layer kernel k={k}: max rel err {worst:.2e}")
    assert worst <= TOL and worst <= H.REGRESSION["tiny_layer"]


def test_decode_layer_exact_logit_tie(tiny_layer):
    """Two experts with identical router rows and scales have bit-identical logits: the lower id ranks
    first (the selection rule), in the kernel and in the oracle, with equal gate weights."""
    cfg, dev, shape, orc = tiny_layer
    rw = dev.router_w.clone()
    rs = dev.router_s.clone()
    rw[6] = rw[2]
    rs[6] = rs[2]
    rw_np, rs_np = rw.cpu().numpy(), rs.cpu().numpy()
    seen_tie = 0
    for tok in range(12):
        x = H.token_batch(cfg, [tok])[0]
        for k in (cfg.k, cfg.n_experts):
            b = q.moe_decode_layer_workspace_bytes(cfg.d, cfg.n_experts, k, cfg.F, cfg.S)
            ws = torch.zeros(b, dtype=torch.uint8, device="cuda")
            ids, w, lg, out = _run(cfg, dev, shape, x, ws, b, None, 0, k=k, router_w=rw, router_s=rs)
            torch.cuda.synchronize()
            lg_np = lg.cpu().numpy()
            assert lg_np[2] == lg_np[6]
            ids_l = ids.cpu().tolist()
            ref = moe.select_topk(moe.router_logits(rw_np, rs_np, oin.token_input(cfg, tok)), k).tolist()
            assert H.topk_consistent(ids_l, moe.router_logits(rw_np, rs_np, oin.token_input(cfg, tok)), k)
            if 2 in ids_l and 6 in ids_l:
                seen_tie += 1
                assert ids_l.index(2) + 1 == ids_l.index(6), ids_l      # adjacent, lower id first
                wl = w.cpu().numpy()
                assert wl[ids_l.index(2)] == wl[ids_l.index(6)]
                assert ref.index(2) + 1 == ref.index(6)
            elif 6 in ids_l:
                pytest.fail(f"expert 6 selected without its tie partner 2: {ids_l}")
    assert seen_tie >= 12   # with k = E both are always selected


# ---------------------------------------------------------------------------------------------------
# the layer in two launches (router + shared expert, then routed experts + combine)
# ---------------------------------------------------------------------------------------------------

def _run_parts(cfg, dev, shape, x, ws, ws_b, gamma, residual, forced=None, routed=None, gemv_ids=None, u=None):
    rp, sp = _pools(cfg, dev, shape)
    ids = torch.full((cfg.k,), -5, dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.k,), dtype=torch.float32, device="cuda")
    lg = torch.empty((cfg.n_experts,), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    xdt = q.MOE_BF16 if cfg.x_bf16 else q.MOE_F32
    for part in (1, 2):
        q.moe_decode_layer_part(part, x, xdt, gamma, 1e-6, residual, dev.router_w, dev.router_s, cfg.n_experts, cfg.k,
                                forced, routed or rp, gemv_ids, sp, shape.act, ids, w, lg, u, out, ws, ws_b)
    return ids, w, lg, out


def test_decode_layer_parts_equal_whole_calls(stack_layer):
    """Part 1 then part 2 on one workspace equal one moe_decode_layer call bit for bit (routing, weights,
    logits, normalized activation, output), with self-routing and with forced routing through cache slots,
    alternating with whole calls on the same workspace; the synchronisation words stay consistent."""
    cfg, dev, shape = stack_layer
    gamma = torch.from_numpy(synth.rms_gamma(cfg.weight_cfg, 0, cfg.d, ones=False)).cuda()
    trace = synth.zipf_trace(21, 2, 1, cfg.k, cfg.n_experts, 1.1)[:, 0, :]
    rb = dev.pool.shape[1]
    ws, ws_b = _ws(cfg)
    ws2, _ = _ws(cfg)
    calls = 0
    for t, tok in enumerate((4, 90, 91, 250)):
        x = H.token_batch(cfg, [tok])[0]
        forced = routed = gemv_ids = None
        if t >= 2:   # forced routing, experts read through slots
            forced = torch.from_numpy(trace[t - 2].astype(np.int32)).cuda()
            slots = torch.zeros((16, rb), dtype=torch.uint8, device="cuda")
            slot_of = (np.arange(cfg.k) * 3 + 1 + t) % 16
            for i, e in enumerate(trace[t - 2]):
                slots[slot_of[i]].copy_(dev.pool[int(e)])
            routed = q.pool(slots, rb, 16, cfg.d, cfg.F, shape.sb_dtype)
            gemv_ids = torch.from_numpy(slot_of.astype(np.int32)).cuda()
        ua = torch.empty((cfg.d,), dtype=torch.bfloat16, device="cuda")
        ub = torch.empty_like(ua)
        a = _run(cfg, dev, shape, x, ws2, ws_b, gamma, 1, forced=forced,
                 routed=None if forced is None else q.pool(dev.pool, rb, cfg.n_experts, cfg.d, cfg.F, shape.sb_dtype),
                 u=ua)
        b = _run_parts(cfg, dev, shape, x, ws, ws_b, gamma, 1, forced, routed, gemv_ids, ub)
        calls += 1
        _check_clean(ws, cfg, calls)
        for name, ta, tb in zip(("ids", "weights", "logits", "out"), a, b):
            assert torch.equal(ta, tb), f"token {tok}: {name}"
        assert torch.equal(ua, ub), f"token {tok}: u"
        # a whole call on the same workspace in between
        _run(cfg, dev, shape, x, ws, ws_b, gamma, 1)
        calls += 1
        _check_clean(ws, cfg, calls)


def test_expert_cache_copies_wait_for_a_pending_reader():
    """expert_cache_stage with a wait_event still pending (recorded after a 1 ms read on the compute stream)
    enqueues its copies behind that reader: the ready event completes after it.  With a wait_event already
    complete it copies at once.  Either way the slots then hold the host records of their experts."""
    cfg = synth.STREAMED
    dev = H.device_layer(cfg, 0)
    k, E, n_slots = cfg.k, cfg.n_experts, cfg.n_slots
    rb = dev.pool.shape[1]
    host = dev.pool.cpu().pin_memory()
    slots = torch.zeros((n_slots, rb), dtype=torch.uint8, device="cuda")
    cache = q.moe_expert_cache_create(1, E, n_slots, rb, [host.data_ptr()], [slots.data_ptr()])
    copy_stream = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    n = 1 << 31
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    slot_ids = torch.empty((k,), dtype=torch.int32, device="cuda")
    try:
        for call, ids in enumerate((list(range(k)), list(range(k, 2 * k)))):
            freed = torch.cuda.Event(enable_timing=True)
            ready = torch.cuda.Event(enable_timing=True)
            ready.record(copy_stream)           # torch creates the HIP event on first record
            torch.cuda.synchronize()
            for _ in range(4):
                q.moe_hbm_read_probe(buf, n, sink, compute)
            freed.record(compute)
            if call == 1:
                freed.synchronize()
            pending = not freed.query()
            assert pending == (call == 0)
            q.expert_cache_stage(cache, 0, ids, slot_ids, copy_stream, freed, ready)
            torch.cuda.synchronize()
            if call == 0:
                assert freed.elapsed_time(ready) > 0.0   # the copies ran after the reader
            held = q.moe_expert_cache_slots(cache, 0, n_slots)
            assert sorted(e for e in held if e >= 0) == list(range(k * (call + 1)))
            for s_, e in enumerate(held):
                if e >= 0:
                    assert torch.equal(slots[s_], dev.pool[e]), f"call {call} slot {s_}"
    finally:
        q.moe_expert_cache_destroy(cache)


def test_shared_expert_runs_inside_the_expert_copy_window():
    """Expert-cache streaming with the layer in two launches: part 1 (router and shared expert) runs on the
    compute stream while the layer's missing experts are copied from pinned host memory on the copy stream,
    and part 2 waits for the copies.  Event timestamps: part 1 starts after the copies start and ends before
    they end; the layer's output equals the resident run bit for bit."""
    cfg = synth.STREAMED
    dev = H.device_layer(cfg, 0)
    shape = H.shape_of(cfg)
    k, E, n_slots = cfg.k, cfg.n_experts, cfg.n_slots
    rb = dev.pool.shape[1]
    host = [dev.pool.cpu().pin_memory()]
    slots = torch.empty((n_slots, rb), dtype=torch.uint8, device="cuda")
    cache = q.moe_expert_cache_create(1, E, n_slots, rb, [host[0].data_ptr()], [slots.data_ptr()])
    dec = decoder.MoEDecoder(shape, [dev], T=1)
    slot_pool = q.pool(slots, rb, n_slots, cfg.d, cfg.F, shape.sb_dtype)
    copy_stream = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    ready = torch.cuda.Event()
    ready.record(copy_stream)
    copy_stream.synchronize()
    slot_ids = torch.empty((k,), dtype=torch.int32, device="cuda")
    trace = synth.zipf_trace(31, 1, 1, k, E, 1.1)[0, 0]
    forced = torch.from_numpy(trace.astype(np.int32)).cuda()
    x = H.token_batch(cfg, [7])
    out, ref = torch.empty_like(x), torch.empty_like(x)
    ev = {n: torch.cuda.Event(enable_timing=True) for n in ("c0", "c1", "p0", "p1", "e")}
    try:
        # one untimed pair of launches first (the first launch of a kernel in a process pays its loading)
        dec.layer_part(1, 0, x, ref, forced_ids=forced.reshape(1, k))
        dec.layer_part(2, 0, x, ref, forced_ids=forced.reshape(1, k))
        torch.cuda.synchronize()
        ev["c0"].record(copy_stream)
        q.expert_cache_stage(cache, 0, trace.tolist(), slot_ids, copy_stream, None, ready)   # cold: 8 misses
        ev["c1"].record(copy_stream)
        compute.wait_event(ev["c0"])
        ev["p0"].record(compute)
        dec.layer_part(1, 0, x, out, forced_ids=forced.reshape(1, k), routed_pool=slot_pool, ids=slot_ids.reshape(1, k))
        ev["p1"].record(compute)
        compute.wait_event(ready)
        dec.layer_part(2, 0, x, out, forced_ids=forced.reshape(1, k), routed_pool=slot_pool, ids=slot_ids.reshape(1, k))
        ev["e"].record(compute)
        torch.cuda.synchronize()
        dec.check_status()
        copy_ms = ev["c0"].elapsed_time(ev["c1"])
        p1_ms = ev["p0"].elapsed_time(ev["p1"])
        print(f"copies {copy_ms * 1e3:.0f} us; part 1 from {ev['c0'].elapsed_time(ev['p0']) * 1e3:.1f} to "
              f"{ev['c0'].elapsed_time(ev['p1']) * 1e3:.1f} us; part 2 ends at {ev['c0'].elapsed_time(ev['e']) * 1e3:.0f} us")
        assert ev["c0"].elapsed_time(ev["p0"]) >= 0.0           # part 1 starts after the copies start
        assert ev["p1"].elapsed_time(ev["c1"]) > 0.0            # and ends before they end
        assert p1_ms < copy_ms
        assert ev["c1"].elapsed_time(ev["e"]) > 0.0             # part 2 ends after the copies
        dec.layer(0, x, ref, forced_ids=forced.reshape(1, k))
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    finally:
        q.moe_expert_cache_destroy(cache)
