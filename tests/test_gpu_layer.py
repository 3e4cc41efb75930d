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
from bit_quantized_expert_int8_amd import moeq4 as q  # noqa: E402
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


def _run(cfg, dev, shape, x, ws, ws_b, gamma, residual, forced=None, routed=None, gemv_ids=None, shared=True):
    rp, sp = _pools(cfg, dev, shape, shared)
    ids = torch.full((cfg.k,), -5, dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.k,), dtype=torch.float32, device="cuda")
    lg = torch.empty((cfg.n_experts,), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    xdt = q.MOE_BF16 if cfg.x_bf16 else q.MOE_F32
    q.moe_decode_layer(x, xdt, gamma, 1e-6, residual, dev.router_w, dev.router_s, cfg.n_experts, cfg.k, forced,
                       routed or rp, gemv_ids, sp, shape.act, ids, w, lg, out, ws, ws_b)
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
    """One d=2816 layer (RMSNorm, router, 8 of 128 experts + shared, residual) on four tokens, one call
    each on one workspace: routing valid for the oracle's logits on the norm output, weights the softmax
    of those logits, output within the parity bar of the oracle run on the GPU's routing."""
    cfg, dev, shape = stack_layer
    gamma_np = synth.rms_gamma(cfg.weight_cfg, 0, cfg.d, ones=gamma_ones)
    gamma = torch.from_numpy(gamma_np).cuda()
    orc = oin.oracle_layer(cfg, 0, cache_experts=24)
    orc.gamma = gamma_np.astype(np.float64)
    ws, ws_b = _ws(cfg)
    for call, tok in enumerate((0, 5, 77, 200), 1):
        x = H.token_batch(cfg, [tok])[0]
        ids, w, lg, out = _run(cfg, dev, shape, x, ws, ws_b, gamma, 1)
        _check_clean(ws, cfg, call)
        x64 = H.to_f64(x)
        u_ref = moe.f64_round_to_bf16(moe.rms_norm(x64, orc.gamma, 1e-6))
        ref_lg = moe.router_logits(orc.router_w, orc.router_s, u_ref)
        got_lg = lg.cpu().numpy().astype(np.float64)
        assert np.abs(got_lg - ref_lg).max() <= 2e-2 * max(1.0, np.abs(ref_lg).max()), f"token {tok}"
        ids_np = ids.cpu().numpy()
        assert H.topk_consistent(ids_np.tolist(), ref_lg, cfg.k, gap=5e-3), f"token {tok}: {ids_np}"
        assert np.allclose(w.cpu().numpy(), moe.gate_weights(got_lg, ids_np), rtol=0, atol=1e-6)
        _, res, x_next = moe.stack_layer_step(orc, x64, cfg.k, forced_ids=ids_np)
        got = H.to_f64(out)
        allowed = TOL * np.abs(res.out - x64).max() + 2.0 ** -8 * np.abs(x_next)
        worst = float((np.abs(got - x_next) / allowed).max())
        print(f"layer kernel token {tok}: rel err {H.max_rel_err(got, x_next):.2e}, error / allowance {worst:.2f}")
        assert H.max_rel_err(got, x_next) <= TOL and worst <= 1.0


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
    assert worst <= TOL


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
