"""GPU checks of the two fused entry points of the stacked decode (MI355X): moe_norm_router_topk against
moe_rmsnorm + moe_router_topk and the oracle, and q4_expert_gemv_combine against q4_expert_gemv +
moe_combine (bit for bit) on one d=2816, 128-expert layer of the stack."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from oracle import moe  # noqa: E402
from oracle import inputs as oin  # noqa: E402
from bit_quantized_expert_int8_amd import moeq4 as q  # noqa: E402
import gpu_helpers as H  # noqa: E402


@pytest.fixture(scope="module")
def layer0():
    cfg = synth.STACK
    return cfg, H.device_layer(cfg, 0), H.shape_of(cfg)


def _pools(dev, shape, shared=True):
    rp = q.pool(dev.pool, dev.pool.shape[1], shape.n_experts, shape.d, shape.F, shape.sb_dtype)
    sp = q.pool(dev.shared, dev.shared.shape[1], 1, shape.d, shape.S, shape.sb_dtype) if shared else None
    return rp, sp


def _route(cfg, dev, x, T):
    ws_b = q.moe_router_workspace_bytes(T, cfg.n_experts)
    ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    q.moe_router_topk(x, q.MOE_BF16, T, cfg.d, dev.router_w, dev.router_s, cfg.n_experts, cfg.k, None, ids, w, None,
                      ws, ws_b)
    return ids, w


def _unfused(rp, sp, ids, k, x, T, d, act, w, res, res_dt, out_dt):
    gb = q.q4_expert_gemv_workspace_bytes(rp, k, sp, T)
    gws = torch.empty(max(gb, 256), dtype=torch.uint8, device="cuda")
    yr = torch.empty((T, max(k, 1), d), dtype=torch.float32, device="cuda")
    ys = torch.empty((T, d), dtype=torch.float32, device="cuda") if sp is not None else None
    q.q4_expert_gemv(rp, ids, k, sp, x, q.MOE_BF16, T, act, yr if k else None, ys, gws, gb)
    out = torch.empty((T, d), dtype=torch.bfloat16 if out_dt == q.MOE_BF16 else torch.float32, device="cuda")
    q.moe_combine(yr, w, ys, res, res_dt, T, k, d, out, out_dt)
    return out


def _fused(rp, sp, ids, k, x, T, d, act, w, res, res_dt, out_dt, ws, ws_b):
    out = torch.empty((T, d), dtype=torch.bfloat16 if out_dt == q.MOE_BF16 else torch.float32, device="cuda")
    q.q4_expert_gemv_combine(rp, ids, k, sp, x, q.MOE_BF16, T, q.MOE_ACT_GELU_TANH if act is None else act, w, res,
                             res_dt, out, out_dt, ws, ws_b)
    return out


@pytest.mark.parametrize("T", [1, 5])
def test_gemv_combine_bit_exact_vs_unfused(layer0, T):
    """Routed + shared experts with a bf16 residual, two calls in a row on one workspace (the second on other
    tokens: the tile counters must have been left at zero), each equal to q4_expert_gemv + moe_combine."""
    cfg, dev, shape = layer0
    rp, sp = _pools(dev, shape)
    ws_b = q.q4_expert_gemv_combine_workspace_bytes(rp, cfg.k, sp, T)
    ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
    for call, toks in enumerate((range(T), range(40, 40 + T))):
        x = H.token_batch(cfg, toks)
        res = H.token_batch(cfg, [t + 100 for t in toks])
        ids, w = _route(cfg, dev, x, T)
        ref = _unfused(rp, sp, ids, cfg.k, x, T, cfg.d, shape.act, w, res, q.MOE_BF16, q.MOE_BF16)
        got = _fused(rp, sp, ids, cfg.k, x, T, cfg.d, shape.act, w, res, q.MOE_BF16, q.MOE_BF16, ws, ws_b)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"call {call}"
        assert torch.isfinite(got.float()).all()
    counters = ws[ws_b - ((T * cfg.d // 16 * 4 + 255) // 256 * 256):].view(torch.int32)
    assert int(counters.abs().sum()) == 0


def test_gemv_combine_variants_bit_exact(layer0):
    """Shared expert only (k = 0), routed only (no shared pool), no residual, fp32 output; plus the fused
    result against the oracle's layer on one token."""
    cfg, dev, shape = layer0
    T = 3
    x = H.token_batch(cfg, range(7, 7 + T))
    ids, w = _route(cfg, dev, x, T)
    for k, shared, res_on in ((0, True, True), (cfg.k, False, False), (cfg.k, True, False)):
        rp, sp = _pools(dev, shape, shared)
        rp = rp if k else None
        ws_b = q.q4_expert_gemv_combine_workspace_bytes(rp, k, sp, T)
        ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
        res = x if res_on else None
        ref = _unfused(rp, sp, ids, k, x, T, cfg.d, shape.act, w, res, q.MOE_BF16, q.MOE_F32)
        got = _fused(rp, sp, ids, k, x, T, cfg.d, shape.act, w if k else None, res, q.MOE_BF16, q.MOE_F32, ws, ws_b)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"k={k} shared={shared} residual={res_on}"
    # the last variant (routed + shared, no residual) against the oracle for token 7
    orc = oin.oracle_layer(cfg, 0, cache_experts=16)
    u = H.to_f64(x)[0]
    r = moe.moe_layer(orc, u, cfg.k, forced_ids=ids.cpu().numpy()[0])
    assert H.max_rel_err(H.to_f64(got)[0], r.out) <= 1e-2


def test_gemv_combine_invalid_id_gives_nan_token(layer0):
    """An expert id outside the pool turns that token's whole output into NaN; the other token is unchanged."""
    cfg, dev, shape = layer0
    T = 2
    rp, sp = _pools(dev, shape)
    x = H.token_batch(cfg, [1, 2])
    ids, w = _route(cfg, dev, x, T)
    good = _fused(rp, sp, ids, cfg.k, x, T, cfg.d, shape.act, w, x, q.MOE_BF16, q.MOE_F32,
                  *_ws(rp, sp, cfg.k, T))
    ids[1, 3] = cfg.n_experts + 5
    ws, ws_b = _ws(rp, sp, cfg.k, T)
    bad = _fused(rp, sp, ids, cfg.k, x, T, cfg.d, shape.act, w, x, q.MOE_BF16, q.MOE_F32, ws, ws_b)
    torch.cuda.synchronize()
    assert torch.equal(bad[0], good[0])
    assert torch.isnan(bad[1]).all()
    # the counters were still reset: a valid call on the same workspace is exact again
    ids[1, 3] = 0
    again = _fused(rp, sp, ids, cfg.k, x, T, cfg.d, shape.act, w, x, q.MOE_BF16, q.MOE_F32, ws, ws_b)
    ref = _unfused(rp, sp, ids, cfg.k, x, T, cfg.d, shape.act, w, x, q.MOE_BF16, q.MOE_F32)
    torch.cuda.synchronize()
    assert torch.equal(again, ref)


def _ws(rp, sp, k, T):
    b = q.q4_expert_gemv_combine_workspace_bytes(rp, k, sp, T)
    return torch.zeros(b, dtype=torch.uint8, device="cuda"), b


@pytest.mark.parametrize("gamma_ones", [True, False])
def test_norm_router_vs_separate_and_oracle(gamma_ones):
    """moe_norm_router_topk: u equal to moe_rmsnorm's bit for bit (one token alone or four together, with
    the same logits, ids and weights) and within one bf16 ulp of the oracle's RMSNorm; ids a valid top-8 of
    the oracle's logits on that u; weights the softmax of those logits; forced ids honoured."""
    cfg = synth.STACK
    d, E, k, T = cfg.d, cfg.n_experts, cfg.k, 4
    rw, rs = synth.router_int8(cfg.weight_cfg, 0, E, d)
    gamma_np = synth.rms_gamma(cfg.weight_cfg, 0, d, ones=gamma_ones)
    w_dev, s_dev = torch.from_numpy(rw).cuda(), torch.from_numpy(rs).cuda()
    gamma = torch.from_numpy(gamma_np).cuda()
    x = H.token_batch(cfg, range(20, 20 + T))
    ws_b = q.moe_router_workspace_bytes(T, E)
    ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
    u = torch.empty_like(x)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    q.moe_norm_router_topk(x, q.MOE_BF16, gamma, 1e-6, T, d, w_dev, s_dev, E, k, None, ids, wts, lg, u, ws, ws_b)
    u_sep = torch.empty_like(x)
    q.moe_rmsnorm(x, q.MOE_BF16, gamma, 1e-6, T, d, u_sep, q.MOE_BF16)
    torch.cuda.synchronize()
    uf, us = H.to_f64(u), H.to_f64(u_sep)
    assert torch.equal(u, u_sep)     # the same summation order: bit for bit
    # the one-token launch (router_kernel) normalizes the same way as the batched one
    u1 = torch.empty_like(x[:1])
    ids1 = torch.empty((1, k), dtype=torch.int32, device="cuda")
    wts1 = torch.empty((1, k), dtype=torch.float32, device="cuda")
    lg1 = torch.empty((1, E), dtype=torch.float32, device="cuda")
    ws1_b = q.moe_router_workspace_bytes(1, E)
    ws1 = torch.zeros(ws1_b, dtype=torch.uint8, device="cuda")
    q.moe_norm_router_topk(x[:1].contiguous(), q.MOE_BF16, gamma, 1e-6, 1, d, w_dev, s_dev, E, k, None, ids1, wts1, lg1,
                           u1, ws1, ws1_b)
    torch.cuda.synchronize()
    assert torch.equal(u1[0], u[0])
    assert torch.equal(ids1[0], ids[0]) and torch.equal(wts1[0], wts[0]) and torch.equal(lg1[0], lg[0])
    xs = H.to_f64(x)
    for t in range(T):
        u_ref = moe.rms_norm(xs[t], gamma_np.astype(np.float64), 1e-6)
        assert H.max_rel_err(uf[t], u_ref) <= 2 ** -7
        ref_lg = moe.router_logits(rw, rs, uf[t])
        assert np.abs(lg.cpu().numpy()[t] - ref_lg).max() <= 1e-5 * max(1.0, np.abs(ref_lg).max())
        assert H.topk_consistent(ids[t].tolist(), ref_lg, k)
        assert np.allclose(wts[t].cpu().numpy(), moe.gate_weights(ref_lg, ids[t].cpu().numpy()), rtol=0, atol=1e-6)
    forced = torch.tensor([[(5 * t + 3 * i) % E for i in range(k)] for t in range(T)], dtype=torch.int32, device="cuda")
    q.moe_norm_router_topk(x, q.MOE_BF16, gamma, 1e-6, T, d, w_dev, s_dev, E, k, forced, ids, wts, lg, u, ws, ws_b)
    torch.cuda.synchronize()
    assert torch.equal(ids, forced)
    for t in range(T):
        ref_lg = moe.router_logits(rw, rs, uf[t])
        assert np.allclose(wts[t].cpu().numpy(), moe.gate_weights(ref_lg, forced[t].cpu().numpy()), rtol=0, atol=1e-6)


@pytest.mark.parametrize("T", [2, 32, 33])
def test_norm_router_paths_agree_bit_for_bit(T):
    """moe_norm_router_topk runs one launch per token block for T = 1, a launch whose last logit block of each
    token selects for 2 <= T <= 32, and logits then selection (two launches) above: every token's u, logits,
    ids and weights equal the one-token call's bit for bit (same norm order, same dot products, same ranking)."""
    cfg = synth.STACK
    d, E, k = cfg.d, cfg.n_experts, cfg.k
    rw, rs = synth.router_int8(cfg.weight_cfg, 1, E, d)
    gamma = torch.from_numpy(synth.rms_gamma(cfg.weight_cfg, 1, d, ones=False)).cuda()
    w_dev, s_dev = torch.from_numpy(rw).cuda(), torch.from_numpy(rs).cuda()
    x = H.token_batch(cfg, range(40, 40 + T))

    def run(xs):
        n = xs.shape[0]
        ws_b = q.moe_router_workspace_bytes(n, E)
        ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
        u = torch.empty_like(xs)
        ids = torch.empty((n, k), dtype=torch.int32, device="cuda")
        wts = torch.empty((n, k), dtype=torch.float32, device="cuda")
        lg = torch.empty((n, E), dtype=torch.float32, device="cuda")
        q.moe_norm_router_topk(xs, q.MOE_BF16, gamma, 1e-6, n, d, w_dev, s_dev, E, k, None, ids, wts, lg, u, ws, ws_b)
        return u, ids, wts, lg

    u, ids, wts, lg = run(x)
    torch.cuda.synchronize()
    for t in range(T):
        u1, ids1, wts1, lg1 = run(x[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(u1[0], u[t]) and torch.equal(lg1[0], lg[t]), f"token {t}"
        assert torch.equal(ids1[0], ids[t]) and torch.equal(wts1[0], wts[t]), f"token {t}"


@pytest.mark.gpu
@pytest.mark.parametrize("d,E,k,x_f32", [(512, 16, 2, False), (1536, 72, 8, True), (4096, 128, 8, False),
                                         (5120, 256, 16, True), (8192, 40, 4, False)])
def test_router_launch_paths_agree_across_row_lengths(d, E, k, x_f32):
    """Every row-length instantiation of the several-token router (d <= 1024 NCH, the norm's register passes
    sized from it) gives, for 3 tokens (one launch, ticket selection) and 37 tokens (logits, then selection),
    each token's u, logits, ids and weights equal to the one-token launch's, bit for bit."""
    g = torch.Generator().manual_seed(d + E)
    w_dev = torch.randint(-127, 128, (E, d), dtype=torch.int8, generator=g).cuda()
    s_dev = (torch.rand(E, generator=g) * 4e-3 + 1e-3).cuda()
    gamma = (torch.rand(d, generator=g) + 0.5).cuda()
    dt, xd = (torch.float32, q.MOE_F32) if x_f32 else (torch.bfloat16, q.MOE_BF16)
    x = torch.randn(37, d, generator=g).to(dt).cuda()

    def run(xs):
        n = xs.shape[0]
        ws_b = q.moe_router_workspace_bytes(n, E)
        ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
        u = torch.empty_like(xs)
        ids = torch.empty((n, k), dtype=torch.int32, device="cuda")
        wts = torch.empty((n, k), dtype=torch.float32, device="cuda")
        lg = torch.empty((n, E), dtype=torch.float32, device="cuda")
        q.moe_norm_router_topk(xs, xd, gamma, 1e-6, n, d, w_dev, s_dev, E, k, None, ids, wts, lg, u, ws, ws_b)
        torch.cuda.synchronize()
        return u, ids, wts, lg

    one = [run(x[t:t + 1].contiguous()) for t in range(37)]
    for T in (3, 37):
        u, ids, wts, lg = run(x[:T].contiguous())
        for t in range(T):
            u1, ids1, wts1, lg1 = one[t]
            assert torch.equal(u1[0], u[t]) and torch.equal(lg1[0], lg[t]), f"T={T} token {t}"
            assert torch.equal(ids1[0], ids[t]) and torch.equal(wts1[0], wts[t]), f"T={T} token {t}"
    # and the one-token logits are the int8 dot products of the call's own u (fp64, rounding-level bound)
    u1, _, _, lg1 = one[0]
    ref = (w_dev.double().cpu() @ u1[0].double().cpu()) * s_dev.double().cpu()
    bound = 1e-5 * (w_dev.double().abs().cpu() @ u1[0].double().abs().cpu()) * s_dev.double().cpu() + 1e-30
    assert torch.all((lg1[0].double().cpu() - ref).abs() <= bound)
