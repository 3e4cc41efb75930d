"""GPU checks of the batched (T > 1) path on MI355X: the device grouping of (token, slot) pairs against the
oracle's stable sort (bit-exact), and the grouped expert GEMVs, which run on the matrix cores, against the
oracle and against one-token calls (within the parity bar: the two paths scale and sum the activations
differently, so their roundings differ)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from oracle import moe  # noqa: E402
from oracle import inputs as oin  # noqa: E402
from bit_quantized_expert_int8_amd import moeq4 as q  # noqa: E402
import gpu_helpers as H  # noqa: E402

TOL = 1e-2   # max relative error of floating outputs (the parity bar)


def _group_on_gpu(ids_np, n_valid):
    T, k = ids_np.shape
    gmax = q.moe_group_pairs_max_groups(T, k, n_valid)
    ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
    n = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    groups = torch.full((gmax, 4), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    q.moe_group_pairs(ids, T, k, n_valid, n, groups, perm)
    torch.cuda.synchronize()
    ng = int(n.item())
    return [tuple(r[:3]) for r in groups.cpu().numpy()[:ng].tolist()], perm.cpu().numpy()


@pytest.mark.parametrize("T,k,n_valid,kind", [(32, 8, 128, "router"), (32, 8, 128, "zipf"), (1, 8, 128, "router"),
                                              (1000, 8, 128, "zipf"), (300, 3, 4096, "uniform"), (64, 2, 1, "invalid")])
def test_group_pairs_bit_exact_vs_oracle(T, k, n_valid, kind):
    """Routing of the batched configuration (top-8 of 128 per token), Zipf(1.1) routing with repeats across
    tokens, batches large enough for several placement rounds, the largest pool, and out-of-pool ids."""
    rng = np.random.default_rng(T * 31 + k)
    if kind == "router":
        ids = np.stack([rng.permutation(n_valid)[:k] for _ in range(T)])
    elif kind == "zipf":
        ids = synth.zipf_trace(9, T, 1, k, n_valid, 1.1)[:, 0, :]
    elif kind == "uniform":
        ids = rng.integers(0, n_valid, size=(T, k))
    else:
        ids = rng.integers(-3, 4, size=(T, k))
    g_ref, p_ref = moe.group_pairs(ids, n_valid)
    g, p = _group_on_gpu(ids, n_valid)
    assert g == g_ref
    assert np.array_equal(p, p_ref)


def _tiny_pools(cfg, dev, shape):
    rp = q.pool(dev.pool, dev.pool.shape[1], shape.n_experts, shape.d, shape.F, shape.sb_dtype)
    sp = q.pool(dev.shared, dev.shared.shape[1], 1, shape.d, shape.S, shape.sb_dtype)
    return rp, sp


def _gemv(rp, sp, ids, k, x, x_dtype, T, act, d):
    wb = q.q4_expert_gemv_workspace_bytes(rp, k, sp, T)
    ws = torch.empty(max(wb, 256), dtype=torch.uint8, device="cuda")
    yr = torch.full((T, max(k, 1), d), 7.0, dtype=torch.float32, device="cuda")
    ys = torch.full((T, d), 7.0, dtype=torch.float32, device="cuda") if sp is not None else None
    q.q4_expert_gemv(rp if k else None, ids, k, sp, x, x_dtype, T, act, yr if k else None, ys, ws, wb)
    return yr, ys


def _oracle_act(shape):
    return moe.ACT_GELU_TANH if shape.act == q.MOE_ACT_GELU_TANH else moe.ACT_SILU


@pytest.mark.parametrize("cfg_name", ["tiny", "batched"])
def test_grouped_gemv_matches_one_token_calls(cfg_name):
    """Grouped T-token call vs T separate one-token calls, y_routed and y_shared within the parity bar, and
    (batched) sampled expert outputs against the oracle.  The ids carry repeats across tokens, a duplicate
    within a token and (tiny) an id outside the pool, whose rows are NaN on both paths."""
    cfg = synth.TINY if cfg_name == "tiny" else synth.BATCHED
    dev = H.device_layer(cfg, 0)
    shape = H.shape_of(cfg)
    rp, sp = _tiny_pools(cfg, dev, shape)
    T, k, E = (24, cfg.k, cfg.n_experts) if cfg_name == "tiny" else (cfg.n_tokens, cfg.k, cfg.n_experts)
    rng = np.random.default_rng(11)
    ids_np = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids_np[3, 1] = ids_np[3, 0]                      # duplicate expert within one token
    if cfg_name == "tiny":
        ids_np[5, 0] = E + 2                          # outside the pool
    ids = torch.from_numpy(ids_np).cuda()
    x = H.token_batch(cfg, range(T))
    xdt = q.MOE_BF16 if cfg.x_bf16 else q.MOE_F32
    yr, ys = _gemv(rp, sp, ids, k, x, xdt, T, shape.act, cfg.d)
    check = range(T) if cfg_name == "tiny" else (0, 3, 17, 31)
    worst = 0.0
    for t in check:
        yr1, ys1 = _gemv(rp, sp, ids[t:t + 1].contiguous(), k, x[t:t + 1].contiguous(), xdt, 1, shape.act, cfg.d)
        torch.cuda.synchronize()
        worst = max(worst, H.max_rel_err(H.to_f64(ys[t]), H.to_f64(ys1[0])))
        for i in range(k):
            if ids_np[t, i] >= E:
                assert torch.isnan(yr[t, i]).all() and torch.isnan(yr1[0, i]).all()
            else:
                assert torch.isfinite(yr[t, i]).all(), f"token {t} slot {i}"
                worst = max(worst, H.max_rel_err(H.to_f64(yr[t, i]), H.to_f64(yr1[0, i])))
    print(f"{cfg_name}: grouped vs one-token calls, max rel difference {worst:.3e}")
    assert worst <= TOL
    if cfg_name == "batched":
        orc = oin.oracle_layer(cfg, 0)
        act = _oracle_act(shape)
        yr64, ys64 = H.to_f64(yr), H.to_f64(ys)
        err = 0.0
        for t in (0, 3, 31):
            u = H.to_f64(x[t])
            err = max(err, H.max_rel_err(ys64[t], moe.expert_ffn(orc.decoded_shared(), u, act)))
            for i in range(k):
                err = max(err, H.max_rel_err(yr64[t, i], moe.expert_ffn(orc.decoded(int(ids_np[t, i])), u, act)))
        print(f"batched grouped expert gemv vs oracle: max rel err {err:.3e}")
        assert err <= TOL


def test_grouped_gemv_tiny_vs_oracle():
    """Tiny configuration (fp32 x and scale/bias), 24 tokens, every expert output against the oracle."""
    cfg = synth.TINY
    dev = H.device_layer(cfg, 0)
    orc = oin.oracle_layer(cfg, 0)
    shape = H.shape_of(cfg)
    rp, sp = _tiny_pools(cfg, dev, shape)
    T, k = 24, cfg.k
    rng = np.random.default_rng(4)
    ids_np = np.stack([rng.permutation(cfg.n_experts)[:k] for _ in range(T)]).astype(np.int32)
    x = H.token_batch(cfg, range(T))
    yr, ys = _gemv(rp, sp, torch.from_numpy(ids_np).cuda(), k, x, q.MOE_F32, T, shape.act, cfg.d)
    torch.cuda.synchronize()
    yr, ys = H.to_f64(yr), H.to_f64(ys)
    worst = 0.0
    for t in range(T):
        u = oin.token_input(cfg, t)
        for i in range(k):
            ref = moe.expert_ffn(orc.decoded(int(ids_np[t, i])), u, moe.ACT_GELU_TANH)
            worst = max(worst, H.max_rel_err(yr[t, i], ref))
        worst = max(worst, H.max_rel_err(ys[t], moe.expert_ffn(orc.decoded_shared(), u, moe.ACT_GELU_TANH)))
    print(f"tiny grouped expert gemv: max rel err {worst:.3e}")
    assert worst <= TOL


def test_grouped_fused_combine_matches_one_token_calls():
    """q4_expert_gemv_combine with 32 tokens (grouped on the matrix cores, then the combine) matches 32
    one-token fused calls within the parity bar, twice in a row on one workspace."""
    cfg = synth.STACK
    dev = H.device_layer(cfg, 0)
    shape = H.shape_of(cfg)
    rp, sp = _tiny_pools(cfg, dev, shape)
    T, k, E = 32, cfg.k, cfg.n_experts
    ws_b = q.q4_expert_gemv_combine_workspace_bytes(rp, k, sp, T)
    ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
    ws1_b = q.q4_expert_gemv_combine_workspace_bytes(rp, k, sp, 1)
    ws1 = torch.zeros(ws1_b, dtype=torch.uint8, device="cuda")
    for call in range(2):
        rng = np.random.default_rng(100 + call)
        ids_np = synth.zipf_trace(20 + call, T, 1, k, E, 1.1)[:, 0, :].astype(np.int32)
        ids = torch.from_numpy(ids_np).cuda()
        w = torch.from_numpy(rng.dirichlet(np.ones(k), size=T).astype(np.float32)).cuda()
        x = H.token_batch(cfg, range(50 * call, 50 * call + T))
        res = H.token_batch(cfg, range(200, 200 + T))
        out = torch.empty_like(x)
        q.q4_expert_gemv_combine(rp, ids, k, sp, x, q.MOE_BF16, T, shape.act, w, res, q.MOE_BF16, out, q.MOE_BF16, ws,
                                 ws_b)
        for t in range(T):
            o1 = torch.empty_like(x[t:t + 1])
            q.q4_expert_gemv_combine(rp, ids[t:t + 1].contiguous(), k, sp, x[t:t + 1].contiguous(), q.MOE_BF16, 1,
                                     shape.act, w[t:t + 1].contiguous(), res[t:t + 1].contiguous(), q.MOE_BF16, o1,
                                     q.MOE_BF16, ws1, ws1_b)
            torch.cuda.synchronize()
            err = H.max_rel_err(H.to_f64(out[t]), H.to_f64(o1[0]))
            assert err <= TOL, f"call {call} token {t}: {err:.3e}"


def test_prefill_chunk_128_tokens_vs_oracle():
    """A 128-token chunk (the pages' prefill processes a prompt's tokens together) through the full-size
    experts: about 8 tokens per expert, several experts with more than 16 (more than one token chunk of the
    matrix-core kernel), 8 chunks of the shared expert.  Sampled expert outputs against the oracle; every
    output finite."""
    cfg = synth.BATCHED
    dev = H.device_layer(cfg, 0)
    shape = H.shape_of(cfg)
    rp, sp = _tiny_pools(cfg, dev, shape)
    T, k, E = 128, cfg.k, cfg.n_experts
    ids_np = synth.zipf_trace(31, T, 1, k, E, 1.1)[:, 0, :].astype(np.int32)
    counts = np.bincount(ids_np.ravel(), minlength=E)
    assert counts.max() > 16   # the multi-chunk path is exercised
    x = H.token_batch(cfg, range(300, 300 + T))
    yr, ys = _gemv(rp, sp, torch.from_numpy(ids_np).cuda(), k, x, q.MOE_BF16, T, shape.act, cfg.d)
    torch.cuda.synchronize()
    assert torch.isfinite(yr).all() and torch.isfinite(ys).all()
    orc = oin.oracle_layer(cfg, 0)
    act = _oracle_act(shape)
    yr64, ys64 = H.to_f64(yr), H.to_f64(ys)
    busiest = int(np.argmax(counts))
    err = 0.0
    for t in sorted({0, 17, 77, 127, *np.nonzero((ids_np == busiest).any(1))[0][-2:].tolist()}):
        u = H.to_f64(x[t])
        err = max(err, H.max_rel_err(ys64[t], moe.expert_ffn(orc.decoded_shared(), u, act)))
        for i in range(k):
            err = max(err, H.max_rel_err(yr64[t, i], moe.expert_ffn(orc.decoded(int(ids_np[t, i])), u, act)))
    print(f"128-token chunk: max rel err {err:.3e} (busiest expert {busiest}: {counts[busiest]} tokens)")
    assert err <= TOL


def test_grouped_gemv_longest_rows_vs_oracle():
    """Rows of the largest supported length (d = 8192: 32 groups per wavefront in the gate/up products, the
    widest register and LDS configuration of the matrix-core kernel), fp32 scale/bias and activations,
    5 tokens, every expert output and the shared expert's against the oracle."""
    d, F, S, E, k, T = 8192, 128, 192, 3, 2, 5
    rng = np.random.default_rng(8192)
    recs, decoded = [], []
    for _ in range(E + 1):
        wgu = (rng.standard_normal((2 * F, d)) * 0.02).astype(np.float32)
        wd = (rng.standard_normal((d, F)) * 0.02).astype(np.float32)
        recs.append(moe.encode_record(wgu, wd, False))
        decoded.append(moe.decode_record(recs[-1], d, F, False))
    wgu = (rng.standard_normal((2 * S, d)) * 0.02).astype(np.float32)
    wd = (rng.standard_normal((d, S)) * 0.02).astype(np.float32)
    srec = moe.encode_record(wgu, wd, False)
    sdec = moe.decode_record(srec, d, S, False)
    pool = torch.from_numpy(np.stack(recs[:E])).cuda()
    shared = torch.from_numpy(srec[None, :].copy()).cuda()
    rp = q.pool(pool, pool.shape[1], E, d, F, q.MOE_F32)
    sp = q.pool(shared, shared.shape[1], 1, d, S, q.MOE_F32)
    ids_np = np.array([[0, 2], [1, 0], [2, 1], [0, 1], [2, 0]], dtype=np.int32)
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).cuda()
    yr, ys = _gemv(rp, sp, torch.from_numpy(ids_np).cuda(), k, x, q.MOE_F32, T, q.MOE_ACT_GELU_TANH, d)
    torch.cuda.synchronize()
    yr, ys, u = H.to_f64(yr), H.to_f64(ys), H.to_f64(x)
    err = 0.0
    for t in range(T):
        err = max(err, H.max_rel_err(ys[t], moe.expert_ffn(sdec, u[t], moe.ACT_GELU_TANH)))
        for i in range(k):
            err = max(err, H.max_rel_err(yr[t, i], moe.expert_ffn(decoded[ids_np[t, i]], u[t], moe.ACT_GELU_TANH)))
    print(f"d=8192 grouped expert gemv: max rel err {err:.3e}")
    assert err <= TOL


def test_grouped_gemv_silu_ragged_batch_vs_oracle():
    """SiLU activation, 7 tokens (a ragged token chunk), top-2 of the tiny pool with one expert taken by
    every token (a 7-token run) and one by none; every output against the oracle."""
    cfg = synth.TINY
    dev = H.device_layer(cfg, 0)
    orc = oin.oracle_layer(cfg, 0)
    shape = H.shape_of(cfg)
    rp, sp = _tiny_pools(cfg, dev, shape)
    T, k = 7, cfg.k
    ids_np = np.array([[3, 0], [3, 5], [1, 3], [3, 6], [2, 3], [3, 4], [0, 3]], dtype=np.int32)
    x = H.token_batch(cfg, range(40, 40 + T))
    yr, ys = _gemv(rp, sp, torch.from_numpy(ids_np).cuda(), k, x, q.MOE_F32, T, q.MOE_ACT_SILU, cfg.d)
    torch.cuda.synchronize()
    yr, ys = H.to_f64(yr), H.to_f64(ys)
    err = 0.0
    for t in range(T):
        u = H.to_f64(x[t])
        err = max(err, H.max_rel_err(ys[t], moe.expert_ffn(orc.decoded_shared(), u, moe.ACT_SILU)))
        for i in range(k):
            err = max(err, H.max_rel_err(yr[t, i], moe.expert_ffn(orc.decoded(int(ids_np[t, i])), u, moe.ACT_SILU)))
    print(f"tiny grouped expert gemv, SiLU, 7 tokens: max rel err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("cfg_name,T", [("tiny", 24), ("batched", 32), ("batched", 128)])
def test_split_calls_equal_whole_call(cfg_name, T):
    """q4_expert_gate_up followed by q4_expert_down on the same workspace (the hidden vectors left there as
    fp32) equals q4_expert_gemv bit for bit with several tokens.  The batch holds a zero token (every hidden
    value 0), a token scaled by 2^-40 (hidden vectors near 2^-80, staged with exponents near -93) and, on
    the tiny pool, an id outside the pool (NaN rows on both)."""
    cfg = synth.TINY if cfg_name == "tiny" else synth.BATCHED
    dev = H.device_layer(cfg, 0)
    shape = H.shape_of(cfg)
    rp, sp = _tiny_pools(cfg, dev, shape)
    k, E = cfg.k, cfg.n_experts
    ids_np = synth.zipf_trace(T, T, 1, k, E, 1.1)[:, 0, :].astype(np.int32)
    if cfg_name == "tiny":
        ids_np[5, 0] = E + 2
    ids = torch.from_numpy(ids_np).cuda()
    x = H.token_batch(cfg, range(500, 500 + T)).clone()
    x[2] = 0
    x[7] = x[7] * 2.0 ** -40
    xdt = q.MOE_BF16 if cfg.x_bf16 else q.MOE_F32
    yr, ys = _gemv(rp, sp, ids, k, x, xdt, T, shape.act, cfg.d)
    wb = q.q4_expert_gemv_workspace_bytes(rp, k, sp, T)
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda")
    yr2 = torch.full_like(yr, 7.0)
    ys2 = torch.full_like(ys, 7.0)
    q.q4_expert_gate_up(rp, ids, k, sp, x, xdt, T, shape.act, ws, wb)
    q.q4_expert_down(rp, ids, k, sp, T, yr2, ys2, ws, wb)
    torch.cuda.synchronize()
    bad = torch.from_numpy(ids_np >= E).cuda()
    assert torch.isnan(yr[bad]).all() and torch.isnan(yr2[bad]).all()
    assert torch.equal(yr[~bad], yr2[~bad]) and torch.equal(ys, ys2)
    assert torch.isfinite(yr[~bad]).all() and torch.isfinite(ys).all()
    assert torch.all(ys[2] == 0) and torch.all(yr[2][~bad[2]] == 0)


def test_grouped_gemv_many_chunks_split_on_device_vs_oracle():
    """4096 tokens on the tiny pool (top-2 of 8: 256 token chunks of the shared expert, 512 routed chunks):
    more chunks than the launch can give one block each, so the blocks split the work themselves instead of
    reading descriptors from the grouping launch.  Sampled tokens' expert outputs against the
    oracle; every output finite."""
    cfg = synth.TINY
    dev = H.device_layer(cfg, 0)
    orc = oin.oracle_layer(cfg, 0)
    shape = H.shape_of(cfg)
    rp, sp = _tiny_pools(cfg, dev, shape)
    T, k = 4096, cfg.k
    rng = np.random.default_rng(4096)
    ids_np = np.stack([rng.permutation(cfg.n_experts)[:k] for _ in range(T)]).astype(np.int32)
    x = torch.from_numpy(rng.standard_normal((T, cfg.d)).astype(np.float32)).cuda()
    yr, ys = _gemv(rp, sp, torch.from_numpy(ids_np).cuda(), k, x, q.MOE_F32, T, shape.act, cfg.d)
    torch.cuda.synchronize()
    assert torch.isfinite(yr).all() and torch.isfinite(ys).all()
    yr, ys, u = H.to_f64(yr), H.to_f64(ys), H.to_f64(x)
    act = _oracle_act(shape)
    err = 0.0
    for t in sorted({0, 1, 15, 16, 17, 511, 1024, 2047, 4094, 4095, *rng.integers(0, T, 20).tolist()}):
        err = max(err, H.max_rel_err(ys[t], moe.expert_ffn(orc.decoded_shared(), u[t], act)))
        for i in range(k):
            err = max(err, H.max_rel_err(yr[t, i], moe.expert_ffn(orc.decoded(int(ids_np[t, i])), u[t], act)))
    print(f"4096 tokens, tiny pool: max rel err {err:.3e}")
    assert err <= TOL
